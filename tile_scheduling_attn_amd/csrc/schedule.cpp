// Host-side schedule generator and DAG critical-path simulator.
//
// Schedules (DASH paper, figures as captioned on the pith.science review
// page): the FlashAttention-3 baseline (Fig. 3), Descending Q-Tile Iteration
// (Fig. 4), Shift Scheduling (Fig. 6) and Symmetric Shift Scheduling with
// two-phase workload folding (Fig. 7).  Readings where the pages leave a
// step open:
//  - baseline: Q tiles ascending, dQ accumulated in ascending KV order;
//  - descending: Q tiles descending, same dQ order as the baseline;
//  - shift: KV tile i visits Q tiles i, i+1, ... (mod n); dQ_j is accumulated
//    in visiting order, i.e. by KV j, j-1, ... (mod n); masked tiles skipped;
//  - symmetric shift (causal, n even, h = n/2): work item p < h runs
//    phase 1 = (KV p, Q h + (p+t) mod h) for t < h, then phase 2 walks the
//    folded square from the diagonal: (KV p, Q p+u) while u < h-p, then
//    (KV n-1-p, Q n-1+h-p-u) up to u = h.  dQ accumulated in step order.
//
// The simulator replays the pages' DAG model (each task = compute phase c
// then reduction phase r; a reduction waits for the previous contributor of
// its dQ tile; a worker runs one phase at a time; review page, "What carries
// the argument" and Axiom ledger) as a discrete-event simulation.
#include "attn_bwd.h"
#include "internal.h"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <queue>
#include <vector>

namespace attn {

static bool visible(bool causal, int kv, int q) { return !causal || kv <= q; }

int build_schedule(int n, bool causal, int schedule, Schedule& out) {
    if (n < 0) return ATTN_ERR_INVALID_ARG;
    if (schedule < ATTN_SCHED_NAIVE || schedule > ATTN_SCHED_ATOMIC) return ATTN_ERR_INVALID_ARG;
    int kind = schedule;
    if (kind == ATTN_SCHED_SYMMETRIC_SHIFT && !causal) kind = ATTN_SCHED_SHIFT;  // empty fold
    if (kind == ATTN_SCHED_SYMMETRIC_SHIFT && (n % 2) != 0) return ATTN_ERR_UNSUPPORTED;

    out = Schedule{};
    out.n = n;
    out.causal = causal;
    out.schedule = schedule;
    out.rank.assign((size_t)n * n, -1);
    out.count.assign(n, 0);
    out.item_begin.push_back(0);

    auto close_item = [&]() { out.item_begin.push_back((int)out.task_kv.size()); };
    auto add = [&](int kv, int q) {
        out.task_kv.push_back(kv);
        out.task_q.push_back(q);
    };

    if (kind == ATTN_SCHED_NAIVE || kind == ATTN_SCHED_DESCENDING || kind == ATTN_SCHED_ATOMIC) {
        for (int kv = 0; kv < n; ++kv) {
            for (int t = 0; t < n; ++t) {
                int q = (kind == ATTN_SCHED_DESCENDING) ? n - 1 - t : t;
                if (visible(causal, kv, q)) add(kv, q);
            }
            close_item();
        }
        // ascending KV order inside every dQ tile
        for (int q = 0; q < n; ++q) {
            int pos = 0;
            for (int kv = 0; kv < n; ++kv)
                if (visible(causal, kv, q)) out.rank[(size_t)kv * n + q] = pos++;
        }
    } else if (kind == ATTN_SCHED_SHIFT) {
        for (int kv = 0; kv < n; ++kv) {
            for (int t = 0; t < n; ++t) {
                int q = (kv + t) % n;
                if (visible(causal, kv, q)) add(kv, q);
            }
            close_item();
        }
        // KV kv reaches Q q after (q - kv) mod n steps; the dQ order of q is
        // the order in which its contributors visit it.
        for (int q = 0; q < n; ++q) {
            int pos = 0;
            for (int t = 0; t < n; ++t) {
                int kv = ((q - t) % n + n) % n;
                if (visible(causal, kv, q)) out.rank[(size_t)kv * n + q] = pos++;
            }
        }
    } else {  // symmetric shift, causal, n even
        const int h = n / 2;
        std::vector<int> step((size_t)n * n, -1);
        for (int p = 0; p < h; ++p) {
            int t = 0;
            for (int u = 0; u < h; ++u, ++t) {
                int q = h + (p + u) % h;
                add(p, q);
                step[(size_t)p * n + q] = t;
            }
            for (int u = 0; u <= h; ++u, ++t) {
                int kv, q;
                if (u < h - p) { kv = p; q = p + u; }
                else { kv = n - 1 - p; q = n - 1 + h - p - u; }
                add(kv, q);
                step[(size_t)kv * n + q] = t;
            }
            close_item();
        }
        for (int q = 0; q < n; ++q) {
            std::vector<std::pair<int, int>> by_step;
            for (int kv = 0; kv <= q; ++kv) by_step.push_back({step[(size_t)kv * n + q], kv});
            std::sort(by_step.begin(), by_step.end());
            for (size_t pos = 0; pos < by_step.size(); ++pos)
                out.rank[(size_t)by_step[pos].second * n + q] = (int)pos;
        }
    }
    for (int q = 0; q < n; ++q)
        for (int kv = 0; kv < n; ++kv)
            if (visible(causal, kv, q)) out.count[q]++;
    if (schedule == ATTN_SCHED_ATOMIC) std::fill(out.rank.begin(), out.rank.end(), -1);
    return ATTN_OK;
}

int min_workers(const Schedule& sc) {
    if (sc.schedule == ATTN_SCHED_NAIVE || sc.schedule == ATTN_SCHED_DESCENDING ||
        sc.schedule == ATTN_SCHED_ATOMIC)
        return 1;
    return std::max(1, sc.num_items());
}

// Discrete-event simulation of `heads` copies of the schedule on `workers`
// workers.  Events are processed in (time, worker) order.
int simulate(const Schedule& sc, int heads, int workers, int placement, double c, double r,
             double* makespan, double* wait_time, double* busy_time) {
    if (heads < 0 || workers <= 0 || c < 0 || r < 0 || (placement != 0 && placement != 1))
        return ATTN_ERR_INVALID_ARG;
    const int n = sc.n, items_per_head = sc.num_items();
    const long long total_items = (long long)heads * items_per_head;
    const bool ordered = sc.schedule != ATTN_SCHED_ATOMIC;

    // next expected rank and finish time of the last reduction, per (head, q)
    std::vector<int> next_rank((size_t)heads * n, 0);
    std::vector<double> last_finish((size_t)heads * n, 0.0);
    // worker state
    struct W {
        long long item = -1;   // global item index, -1 = none
        int task = 0;          // absolute task index in the pattern
        int end = 0;
        int waiting_key = -1;  // (head*n+q) it waits on, -1 if not waiting
        double wait_since = 0;
    };
    std::vector<W> ws(workers);
    std::vector<std::vector<long long>> static_lists;
    std::vector<size_t> static_pos;
    if (placement == 0) {
        static_lists.resize(workers);
        static_pos.assign(workers, 0);
        for (long long g = 0; g < total_items; ++g) static_lists[g % workers].push_back(g);
    }
    long long next_ticket = 0;
    // waiters per (head, q): at most one worker can wait for a given rank;
    // keep a list and scan it (lists stay short).
    std::vector<std::vector<int>> waiters((size_t)heads * n);

    typedef std::pair<double, int> Ev;  // (time, worker): worker ready to act
    std::priority_queue<Ev, std::vector<Ev>, std::greater<Ev>> pq;
    enum Phase { NEED_ITEM, COMPUTE_DONE };
    std::vector<int> phase(workers, NEED_ITEM);
    for (int w = 0; w < workers; ++w) pq.push({0.0, w});

    double t_end = 0.0, waited = 0.0, busy = 0.0;
    long long tasks_done = 0, tasks_total = 0;
    for (int it = 0; it < items_per_head; ++it)
        tasks_total += sc.item_begin[it + 1] - sc.item_begin[it];
    tasks_total *= heads;

    // start the reduction of worker w's current task at time t
    auto start_reduction = [&](int w, double t, auto& self_pq) {
        W& s = ws[w];
        const int head = (int)(s.item / items_per_head);
        const int q = sc.task_q[s.task];
        const size_t key = (size_t)head * n + q;
        double fin = t + r;
        busy += r;
        next_rank[key]++;
        last_finish[key] = fin;
        if (fin > t_end) t_end = fin;
        tasks_done++;
        // wake the worker waiting for the next rank of this tile
        auto& lst = waiters[key];
        for (size_t x = 0; x < lst.size(); ++x) {
            int w2 = lst[x];
            W& s2 = ws[w2];
            int kv2 = sc.task_kv[s2.task];
            if (sc.rank[(size_t)kv2 * n + q] == next_rank[key]) {
                lst.erase(lst.begin() + x);
                waited += fin - s2.wait_since;
                s2.waiting_key = -1;
                self_pq.push({fin, w2 + workers});  // +workers: "reduction may start"
                break;
            }
        }
        s.task++;
        phase[w] = NEED_ITEM;
        self_pq.push({fin, w});
    };

    while (!pq.empty()) {
        Ev ev = pq.top();
        pq.pop();
        double t = ev.first;
        int w = ev.second;
        if (w >= workers) {  // a blocked worker's predecessor finished
            w -= workers;
            start_reduction(w, t, pq);
            continue;
        }
        W& s = ws[w];
        if (phase[w] == NEED_ITEM) {
            if (s.item >= 0 && s.task >= s.end) s.item = -1;
            if (s.item < 0) {
                long long g = -1;
                if (placement == 0) {
                    if (static_pos[w] < static_lists[w].size()) g = static_lists[w][static_pos[w]++];
                } else if (next_ticket < total_items) {
                    g = next_ticket++;
                }
                if (g < 0) continue;  // worker retires
                int pat = (int)(g % items_per_head);
                s.item = g;
                s.task = sc.item_begin[pat];
                s.end = sc.item_begin[pat + 1];
                if (s.task >= s.end) { pq.push({t, w}); s.item = -1; continue; }
            }
            busy += c;
            phase[w] = COMPUTE_DONE;
            pq.push({t + c, w});
            continue;
        }
        // compute phase of the current task finished at t
        const int head = (int)(s.item / items_per_head);
        const int kv = sc.task_kv[s.task], q = sc.task_q[s.task];
        const size_t key = (size_t)head * n + q;
        if (!ordered || sc.rank[(size_t)kv * n + q] == next_rank[key]) {
            double st = ordered ? std::max(t, last_finish[key]) : t;
            if (st > t) waited += st - t;
            start_reduction(w, st, pq);
        } else {
            s.waiting_key = (int)key;
            s.wait_since = t;
            waiters[key].push_back(w);
        }
    }
    if (tasks_done != tasks_total) return ATTN_ERR_DEADLOCK;
    if (makespan) *makespan = t_end;
    if (wait_time) *wait_time = waited;
    if (busy_time) *busy_time = busy;
    return ATTN_OK;
}

}  // namespace attn

extern "C" int attn_sched_size(int n, int causal, int schedule, int* num_items, int* num_tasks) {
    attn::Schedule sc;
    int rc = attn::build_schedule(n, causal != 0, schedule, sc);
    if (rc != ATTN_OK) return attn::fail(rc, "attn_sched_size: invalid or unsupported schedule");
    if (num_items) *num_items = sc.num_items();
    if (num_tasks) *num_tasks = (int)sc.task_kv.size();
    return ATTN_OK;
}

extern "C" int attn_sched_get(int n, int causal, int schedule, int* item_begin, int* task_kv,
                              int* task_q, int* rank, int* count) {
    attn::Schedule sc;
    int rc = attn::build_schedule(n, causal != 0, schedule, sc);
    if (rc != ATTN_OK) return attn::fail(rc, "attn_sched_get: invalid or unsupported schedule");
    if (item_begin) std::memcpy(item_begin, sc.item_begin.data(), sc.item_begin.size() * sizeof(int));
    if (task_kv) std::memcpy(task_kv, sc.task_kv.data(), sc.task_kv.size() * sizeof(int));
    if (task_q) std::memcpy(task_q, sc.task_q.data(), sc.task_q.size() * sizeof(int));
    if (rank) std::memcpy(rank, sc.rank.data(), sc.rank.size() * sizeof(int));
    if (count) std::memcpy(count, sc.count.data(), sc.count.size() * sizeof(int));
    return ATTN_OK;
}

extern "C" int attn_sched_min_workers(int n, int causal, int schedule) {
    attn::Schedule sc;
    int rc = attn::build_schedule(n, causal != 0, schedule, sc);
    if (rc != ATTN_OK) return attn::fail(rc, "attn_sched_min_workers: invalid or unsupported schedule");
    return attn::min_workers(sc);
}

extern "C" int attn_dagsim(int n, int causal, int schedule, int heads, int workers, int placement,
                           double c, double r, double* makespan, double* wait_time,
                           double* busy_time) {
    attn::Schedule sc;
    int rc = attn::build_schedule(n, causal != 0, schedule, sc);
    if (rc != ATTN_OK) return attn::fail(rc, "attn_dagsim: invalid or unsupported schedule");
    rc = attn::simulate(sc, heads, workers, placement, c, r, makespan, wait_time, busy_time);
    if (rc == ATTN_ERR_DEADLOCK) return attn::fail(rc, "attn_dagsim: the schedule deadlocks with this many workers");
    if (rc != ATTN_OK) return attn::fail(rc, "attn_dagsim: invalid arguments");
    return ATTN_OK;
}

// ---------------------------------------------------------------------------
// Schedule selection and cost calibration on the DAG model
// ---------------------------------------------------------------------------
extern "C" int attn_sched_select(int n, int causal, int heads, int workers, double c, double r,
                                 int* schedule, double* makespan) {
    if (n <= 0 || heads <= 0 || workers <= 0 || !(c >= 0) || !(r >= 0))
        return attn::fail(ATTN_ERR_INVALID_ARG, "attn_sched_select: invalid arguments");
    int best = -1;
    double best_t = 0;
    for (int s : {ATTN_SCHED_NAIVE, ATTN_SCHED_DESCENDING, ATTN_SCHED_SHIFT, ATTN_SCHED_SYMMETRIC_SHIFT}) {
        attn::Schedule sc;
        if (attn::build_schedule(n, causal != 0, s, sc) != ATTN_OK) continue;  // e.g. odd n, fold
        if (attn::min_workers(sc) > workers) continue;                          // cannot be co-scheduled
        double t = 0;
        if (attn::simulate(sc, heads, workers, 1, c, r, &t, nullptr, nullptr) != ATTN_OK) continue;
        if (best < 0 || t < best_t * (1 - 1e-12)) {
            best = s;
            best_t = t;
        }
    }
    if (best < 0) return attn::fail(ATTN_ERR_UNSUPPORTED, "attn_sched_select: no schedule runs on this many workers");
    if (schedule) *schedule = best;
    if (makespan) *makespan = best_t;
    return ATTN_OK;
}

namespace {
// Simulated makespans of every sample with compute cost 1 and reduction
// cost rho; false when a sample cannot be simulated.
bool unit_makespans(int count, const int* n, const int* causal, const int* schedule, const int* heads,
                    const int* workers, double rho, std::vector<double>& m) {
    m.resize(count);
    for (int k = 0; k < count; ++k) {
        attn::Schedule sc;
        if (attn::build_schedule(n[k], causal[k] != 0, schedule[k], sc) != ATTN_OK) return false;
        if (attn::simulate(sc, heads[k], workers[k], 1, 1.0, rho, &m[k], nullptr, nullptr) != ATTN_OK) return false;
    }
    return true;
}

// For fixed rho the makespan is proportional to c: the c minimising the
// relative squared error sum (c m_k / T_k - 1)^2 is sum(x) / sum(x^2) with
// x_k = m_k / T_k.  Returns the RMS relative error at that c.
double best_scale(const std::vector<double>& m, const double* measured, double* c) {
    double sx = 0, sxx = 0;
    for (size_t k = 0; k < m.size(); ++k) {
        const double x = m[k] / measured[k];
        sx += x;
        sxx += x * x;
    }
    *c = sxx > 0 ? sx / sxx : 0;
    double e = 0;
    for (size_t k = 0; k < m.size(); ++k) {
        const double d = *c * m[k] / measured[k] - 1;
        e += d * d;
    }
    return std::sqrt(e / (double)m.size());
}
}  // namespace

extern "C" int attn_sched_fit(int count, const int* n, const int* causal, const int* schedule, const int* heads,
                              const int* workers, const double* measured, double* c, double* r, double* rms) {
    if (count <= 0 || !n || !causal || !schedule || !heads || !workers || !measured)
        return attn::fail(ATTN_ERR_INVALID_ARG, "attn_sched_fit: invalid arguments");
    for (int k = 0; k < count; ++k)
        if (!(measured[k] > 0) || n[k] <= 0 || heads[k] <= 0 || workers[k] <= 0)
            return attn::fail(ATTN_ERR_INVALID_ARG, "attn_sched_fit: invalid sample");
    // coarse search over rho = r / c on a log grid (1e-4 .. 1e2), then a
    // golden-section refinement of log(rho) around the best grid point
    std::vector<double> m;
    auto err_at = [&](double lr, double* cc) {
        if (!unit_makespans(count, n, causal, schedule, heads, workers, std::exp(lr), m)) return -1.0;
        return best_scale(m, measured, cc);
    };
    const double lo = std::log(1e-4), hi = std::log(1e2);
    const int steps = 60;
    double best_lr = lo, best_e = -1, cc = 0;
    for (int i = 0; i <= steps; ++i) {
        const double lr = lo + (hi - lo) * i / steps;
        const double e = err_at(lr, &cc);
        if (e < 0) return attn::fail(ATTN_ERR_UNSUPPORTED, "attn_sched_fit: a sample cannot be simulated");
        if (best_e < 0 || e < best_e) {
            best_e = e;
            best_lr = lr;
        }
    }
    const double h = (hi - lo) / steps, g = 0.6180339887498949;
    double a = best_lr - h, b = best_lr + h;
    double x1 = b - g * (b - a), x2 = a + g * (b - a);
    double f1 = err_at(x1, &cc), f2 = err_at(x2, &cc);
    for (int it = 0; it < 40; ++it) {
        if (f1 < f2) {
            b = x2; x2 = x1; f2 = f1; x1 = b - g * (b - a); f1 = err_at(x1, &cc);
        } else {
            a = x1; x1 = x2; f1 = f2; x2 = a + g * (b - a); f2 = err_at(x2, &cc);
        }
    }
    double lr = 0.5 * (a + b);
    double e = err_at(lr, &cc);
    double cg = 0;
    const double eg = err_at(best_lr, &cg);  // keep the grid point if the refinement did not help
    if (eg <= e) {
        lr = best_lr;
        e = eg;
        cc = cg;
    }
    if (c) *c = cc;
    if (r) *r = cc * std::exp(lr);
    if (rms) *rms = e;
    return ATTN_OK;
}
