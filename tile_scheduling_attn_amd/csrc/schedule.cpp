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
//    with more KV tiles than kShiftRound (more than the work groups that can
//    be resident at once; Axiom ledger: KV tiles != SMs is handled by refining
//    heads) the KV tiles are cut into rounds of at most kShiftRound
//    consecutive tiles, items keep the cyclic order, and dQ_j is accumulated
//    round by round, inside a round in visiting order;
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

// Q tile q sees KV tile kv unless the causal mask removes every pair: with
// `ratio` Q tiles per KV tile, when ratio * kv <= q
static bool visible(bool causal, int kv, int q, int ratio) { return !causal || ratio * kv <= q; }

int build_schedule(int n, bool causal, int schedule, Schedule& out, int ratio) {
    if (n < 0 || ratio < 1) return ATTN_ERR_INVALID_ARG;
    if (n > kMaxTiles || ratio > 8 || (long long)ratio * n > kMaxTiles) return ATTN_ERR_UNSUPPORTED;
    if (schedule < ATTN_SCHED_NAIVE || schedule > ATTN_SCHED_ATOMIC) return ATTN_ERR_INVALID_ARG;
    int kind = schedule;
    if (kind == ATTN_SCHED_SYMMETRIC_SHIFT && !causal) kind = ATTN_SCHED_SHIFT;  // empty fold
    if (kind == ATTN_SCHED_SYMMETRIC_SHIFT && (n % 2) != 0) return ATTN_ERR_UNSUPPORTED;
    // rounds are defined for square tiles only
    if (kind == ATTN_SCHED_SHIFT && ratio > 1 && n > kShiftRound) return ATTN_ERR_UNSUPPORTED;
    const int nq = ratio * n;

    out = Schedule{};
    out.n = n;
    out.nq = nq;
    out.causal = causal;
    out.schedule = schedule;
    out.rank.assign((size_t)n * nq, -1);
    out.count.assign(nq, 0);
    out.item_begin.push_back(0);

    auto close_item = [&]() { out.item_begin.push_back((int)out.task_kv.size()); };
    auto add = [&](int kv, int q) {
        out.task_kv.push_back(kv);
        out.task_q.push_back(q);
    };

    if (kind == ATTN_SCHED_NAIVE || kind == ATTN_SCHED_DESCENDING || kind == ATTN_SCHED_ATOMIC) {
        for (int kv = 0; kv < n; ++kv) {
            for (int t = 0; t < nq; ++t) {
                int q = (kind == ATTN_SCHED_DESCENDING) ? nq - 1 - t : t;
                if (visible(causal, kv, q, ratio)) add(kv, q);
            }
            close_item();
        }
        // ascending KV order inside every dQ tile
        for (int q = 0; q < nq; ++q) {
            int pos = 0;
            for (int kv = 0; kv < n; ++kv)
                if (visible(causal, kv, q, ratio)) out.rank[(size_t)kv * nq + q] = pos++;
        }
    } else if (kind == ATTN_SCHED_SHIFT) {
        for (int kv = 0; kv < n; ++kv) {
            for (int t = 0; t < nq; ++t) {
                int q = (ratio * kv + t) % nq;
                if (visible(causal, kv, q, ratio)) add(kv, q);
            }
            close_item();
        }
        // KV kv reaches Q q after (q - ratio * kv) mod nq steps; the dQ order
        // of q is the order in which its contributors visit it, round by round
        const int rounds = (n + kShiftRound - 1) / kShiftRound;
        const int w = n > 0 ? (n + rounds - 1) / rounds : 0;
        out.round_size = w;
        for (int q = 0; q < nq; ++q) {
            std::vector<std::pair<int, int>> order;  // (round, step) of each contributor
            for (int kv = 0; kv < n; ++kv)
                if (visible(causal, kv, q, ratio)) order.push_back({(kv / w) * nq + ((q - ratio * kv) % nq + nq) % nq, kv});
            std::sort(order.begin(), order.end());
            for (size_t pos = 0; pos < order.size(); ++pos) out.rank[(size_t)order[pos].second * nq + q] = (int)pos;
        }
    } else {  // symmetric shift, causal, n even
        const int h = n / 2, rh = ratio * h;
        std::vector<int> step((size_t)n * nq, -1);
        for (int p = 0; p < h; ++p) {
            int t = 0;
            // phase 1: the dense block of Q tiles rh .. nq-1 against KV 0 .. h-1
            for (int u = 0; u < rh; ++u, ++t) {
                int q = rh + (ratio * p + u) % rh;
                add(p, q);
                step[(size_t)p * nq + q] = t;
            }
            // phase 2: KV p from its diagonal up to Q rh-1, then KV n-1-p from
            // the last Q tile back to its diagonal
            for (int u = 0; u < rh + ratio; ++u, ++t) {
                const int x = ratio * p + u;
                int kv, q;
                if (x < rh) { kv = p; q = x; }
                else { kv = n - 1 - p; q = 3 * rh - 1 - x; }
                add(kv, q);
                step[(size_t)kv * nq + q] = t;
            }
            close_item();
        }
        for (int q = 0; q < nq; ++q) {
            std::vector<std::pair<int, int>> by_step;
            for (int kv = 0; kv < n; ++kv)
                if (visible(causal, kv, q, ratio)) by_step.push_back({step[(size_t)kv * nq + q], kv});
            std::sort(by_step.begin(), by_step.end());
            for (size_t pos = 0; pos < by_step.size(); ++pos)
                out.rank[(size_t)by_step[pos].second * nq + q] = (int)pos;
        }
    }
    for (int q = 0; q < nq; ++q)
        for (int kv = 0; kv < n; ++kv)
            if (visible(causal, kv, q, ratio)) out.count[q]++;
    if (schedule == ATTN_SCHED_ATOMIC) std::fill(out.rank.begin(), out.rank.end(), -1);
    return ATTN_OK;
}

// The chunks of a head are contiguous runs of its items, and a plan is used
// only if every chunk carries at most kChunkImbalance times the mean work.
// Schedules whose items must all be resident at once (min_workers > 1: the
// Shift family) take the fewest chunks (1, 2, 4 or 8) of equal item count
// that each fit the ⌊grid/8⌋ work groups of a queue: the queues of a group
// then move through their heads at one rate.  The others only ever wait on
// items of the head taken earlier from the same or a lower queue of the
// group, so any chunk size keeps them deadlock-free: they take the fewest
// chunks that still give every queue a head (a whole head per XCD when there
// are eight heads or more, so that no reduction chain leaves its XCD), cut
// at about equal work.
constexpr double kChunkImbalance = 1.1;

XcdPlan xcd_plan(const std::vector<int>& item_begin, int min_workers, long long grid, long long heads) {
    XcdPlan none;
    const int items_per_head = (int)item_begin.size() - 1;
    const long long per_queue = grid / kQueues;
    if (per_queue < 1 || items_per_head < 1 || heads < 1) return none;
    const long long total = item_begin[items_per_head] - item_begin[0];
    for (int g = 1; g <= kQueues; g *= 2) {
        if (min_workers <= 1 && g < kQueues && kQueues / g > heads) continue;
        XcdPlan p;
        p.bounds[0] = 0;
        for (int k = 1; k < g; ++k) {
            if (min_workers > 1) {  // equal item counts
                p.bounds[k] = std::min(k * ((items_per_head + g - 1) / g), items_per_head);
                continue;
            }
            // the cut whose work before it is closest to k/g of the head's
            const double target = (double)total * k / g;
            int b = p.bounds[k - 1];
            while (b < items_per_head && std::fabs((double)(item_begin[b + 1] - item_begin[0]) - target) <=
                                             std::fabs((double)(item_begin[b] - item_begin[0]) - target))
                ++b;
            p.bounds[k] = b;
        }
        p.bounds[g] = items_per_head;
        int max_chunk = 0;
        long long max_work = 0;
        for (int k = 0; k < g; ++k) {
            max_chunk = std::max(max_chunk, p.bounds[k + 1] - p.bounds[k]);
            max_work = std::max<long long>(max_work, item_begin[p.bounds[k + 1]] - item_begin[p.bounds[k]]);
        }
        if (min_workers > 1 && max_chunk > per_queue) continue;
        if (max_work > kChunkImbalance * (double)total / g) continue;
        p.chunks = g;
        p.groups = kQueues / g;
        p.max_chunk = max_chunk;
        p.slots = (heads + p.groups - 1) / p.groups;
        return p;
    }
    return none;
}

int min_workers(const Schedule& sc) {
    if (sc.schedule == ATTN_SCHED_NAIVE || sc.schedule == ATTN_SCHED_DESCENDING ||
        sc.schedule == ATTN_SCHED_ATOMIC)
        return 1;
    // the Shift family waits cyclically inside a round (Shift: a round of at
    // most kShiftRound KV tiles; Symmetric Shift: all of a head's items)
    if (sc.round_size > 0) return std::max(1, sc.round_size);
    return std::max(1, sc.num_items());
}

// Discrete-event simulation of `heads` copies of the schedule on `workers`
// workers.  Events are processed in (time, worker) order.  Placement 0:
// item g on worker g % workers; 1: one ticket queue in item order; 2: the
// kernel's XCD placement (worker w serves queue w % kQueues with the chunks
// of xcd_plan, else as 1), where the edge cost e applies only to a hand-off
// between workers of different queues (XCDs); under 0 and 1 to every one.
int simulate(const Schedule& sc, int heads, int workers, int placement, double c, double r, double e,
             double* makespan, double* wait_time, double* busy_time) {
    if (heads < 0 || workers <= 0 || c < 0 || r < 0 || e < 0 || placement < 0 || placement > 2)
        return ATTN_ERR_INVALID_ARG;
    if (workers > kMaxWorkers || (long long)heads * (long long)sc.task_kv.size() > kMaxSimTasks)
        return ATTN_ERR_UNSUPPORTED;
    // per-(head, Q tile) state: n is the Q tile count here
    const int n = sc.nq, items_per_head = sc.num_items();
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
    // XCD placement: per-queue ticket counters and the queue of each (head,
    // q)'s last contributor
    XcdPlan plan;
    if (placement == 2) plan = xcd_plan(sc.item_begin, min_workers(sc), workers, heads);
    const bool xcd = placement == 2 && plan.chunks > 0;
    std::vector<long long> queue_ticket(kQueues, 0);
    std::vector<int> last_queue((size_t)heads * n, -1);
    // edge cost of a hand-off from queue qa to worker w
    auto edge = [&](int qa, int w) { return !xcd || qa != w % kQueues ? e : 0.0; };
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
        last_queue[key] = w % kQueues;
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
                const double ed = edge(w % kQueues, w2);
                waited += fin + ed - s2.wait_since;
                s2.waiting_key = -1;
                self_pq.push({fin + ed, w2 + workers});  // +workers: "reduction may start"
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
                } else if (xcd) {
                    const int qq = w % kQueues, grp = qq / plan.chunks, chunk = qq % plan.chunks;
                    const int lo = plan.bounds[chunk], size = plan.bounds[chunk + 1] - lo;
                    if (size > 0) {
                        const long long k = queue_ticket[qq]++;
                        const long long head = grp + (long long)plan.groups * (k / size);
                        if (head < heads) g = head * items_per_head + lo + k % size;
                    }
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
            // a contributor after the first starts once the previous one's
            // release has reached it (edge cost e)
            double st = t;
            if (ordered && next_rank[key] > 0) st = std::max(t, last_finish[key] + edge(last_queue[key], w));
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

static const char* kSchedErr =
    "invalid or unsupported schedule (n < 0, more than 2048 Q tiles, ratio outside 1..8, an odd n for the causal "
    "fold, or ratio > 1 with more than 256 KV tiles under Shift)";

extern "C" int attn_sched_size_rect(int n, int ratio, int causal, int schedule, int* num_items, int* num_tasks) {
    return attn::guarded([&]() -> int {
        attn::Schedule sc;
        int rc = attn::build_schedule(n, causal != 0, schedule, sc, ratio);
        if (rc != ATTN_OK) return attn::fail(rc, kSchedErr);
        if (num_items) *num_items = sc.num_items();
        if (num_tasks) *num_tasks = (int)sc.task_kv.size();
        return ATTN_OK;
    });
}

extern "C" int attn_sched_size(int n, int causal, int schedule, int* num_items, int* num_tasks) {
    return attn_sched_size_rect(n, 1, causal, schedule, num_items, num_tasks);
}

extern "C" int attn_sched_get_rect(int n, int ratio, int causal, int schedule, int* item_begin, int* task_kv,
                                   int* task_q, int* rank, int* count) {
    return attn::guarded([&]() -> int {
        attn::Schedule sc;
        int rc = attn::build_schedule(n, causal != 0, schedule, sc, ratio);
        if (rc != ATTN_OK) return attn::fail(rc, kSchedErr);
        if (item_begin) std::memcpy(item_begin, sc.item_begin.data(), sc.item_begin.size() * sizeof(int));
        if (task_kv) std::memcpy(task_kv, sc.task_kv.data(), sc.task_kv.size() * sizeof(int));
        if (task_q) std::memcpy(task_q, sc.task_q.data(), sc.task_q.size() * sizeof(int));
        if (rank) std::memcpy(rank, sc.rank.data(), sc.rank.size() * sizeof(int));
        if (count) std::memcpy(count, sc.count.data(), sc.count.size() * sizeof(int));
        return ATTN_OK;
    });
}

extern "C" int attn_sched_get(int n, int causal, int schedule, int* item_begin, int* task_kv,
                              int* task_q, int* rank, int* count) {
    return attn_sched_get_rect(n, 1, causal, schedule, item_begin, task_kv, task_q, rank, count);
}

extern "C" int attn_sched_min_workers_rect(int n, int ratio, int causal, int schedule) {
    return attn::guarded([&]() -> int {
        attn::Schedule sc;
        int rc = attn::build_schedule(n, causal != 0, schedule, sc, ratio);
        if (rc != ATTN_OK) return attn::fail(rc, kSchedErr);
        return attn::min_workers(sc);
    });
}

extern "C" int attn_sched_min_workers(int n, int causal, int schedule) {
    return attn_sched_min_workers_rect(n, 1, causal, schedule);
}

extern "C" int attn_dagsim(int n, int causal, int schedule, int heads, int workers, int placement,
                           double c, double r, double* makespan, double* wait_time,
                           double* busy_time) {
    return attn::guarded([&]() -> int {
        return attn_dagsim_edge(n, causal, schedule, heads, workers, placement, c, r, 0.0, makespan, wait_time,
                                busy_time);
    });
}

extern "C" int attn_dagsim_rect(int n, int ratio, int causal, int schedule, int heads, int workers, int placement,
                                double c, double r, double e, double* makespan, double* wait_time,
                                double* busy_time) {
    return attn::guarded([&]() -> int {
        attn::Schedule sc;
        int rc = attn::build_schedule(n, causal != 0, schedule, sc, ratio);
        if (rc != ATTN_OK) return attn::fail(rc, kSchedErr);
        rc = attn::simulate(sc, heads, workers, placement, c, r, e, makespan, wait_time, busy_time);
        if (rc == ATTN_ERR_DEADLOCK) return attn::fail(rc, "attn_dagsim: the schedule deadlocks with this many workers");
        if (rc != ATTN_OK) return attn::fail(rc, "attn_dagsim: invalid arguments, or more heads * tasks or workers than the simulator accepts");
        return ATTN_OK;
    });
}

extern "C" int attn_dagsim_edge(int n, int causal, int schedule, int heads, int workers, int placement,
                                double c, double r, double e, double* makespan, double* wait_time,
                                double* busy_time) {
    return attn_dagsim_rect(n, 1, causal, schedule, heads, workers, placement, c, r, e, makespan, wait_time,
                            busy_time);
}

// ---------------------------------------------------------------------------
// Schedule selection and cost calibration on the DAG model
// ---------------------------------------------------------------------------
extern "C" int attn_sched_select(int n, int causal, int heads, int workers, int placement, double c, double r,
                                 double e, int* schedule, double* makespan) {
    return attn::guarded([&]() -> int {
        if (n <= 0 || heads <= 0 || workers <= 0 || placement < 0 || placement > 2 || !(c >= 0) || !(r >= 0) ||
            !(e >= 0))
            return attn::fail(ATTN_ERR_INVALID_ARG, "attn_sched_select: invalid arguments");
        int best = -1;
        double best_t = 0;
        for (int s : {ATTN_SCHED_NAIVE, ATTN_SCHED_DESCENDING, ATTN_SCHED_SHIFT, ATTN_SCHED_SYMMETRIC_SHIFT}) {
            attn::Schedule sc;
            if (attn::build_schedule(n, causal != 0, s, sc) != ATTN_OK) continue;  // e.g. odd n, fold
            if (attn::min_workers(sc) > workers) continue;                          // cannot be co-scheduled
            double t = 0;
            if (attn::simulate(sc, heads, workers, placement, c, r, e, &t, nullptr, nullptr) != ATTN_OK) continue;
            if (best < 0 || t < best_t * (1 - 1e-12)) {
                best = s;
                best_t = t;
            }
        }
        if (best < 0) return attn::fail(ATTN_ERR_UNSUPPORTED, "attn_sched_select: no schedule runs on this many workers");
        if (schedule) *schedule = best;
        if (makespan) *makespan = best_t;
        return ATTN_OK;
    });
}

namespace {
struct FitData {
    int count, placement;
    const int *n, *causal, *schedule, *heads, *workers;
    const double* measured;
};

// RMS relative error of the model with c = 1, r = rho, e = eps scaled by the
// best c (for fixed rho and eps every makespan is proportional to c, and
// the c minimising sum (c m_k / T_k - 1)^2 is sum(x) / sum(x^2) with
// x_k = m_k / T_k).  Negative when a sample cannot be simulated.
double fit_error(const FitData& f, double rho, double eps, double* c_out) {
    double sx = 0, sxx = 0;
    std::vector<double> x(f.count);
    for (int k = 0; k < f.count; ++k) {
        attn::Schedule sc;
        double m = 0;
        if (attn::build_schedule(f.n[k], f.causal[k] != 0, f.schedule[k], sc) != ATTN_OK) return -1;
        if (attn::simulate(sc, f.heads[k], f.workers[k], f.placement, 1.0, rho, eps, &m, nullptr, nullptr) != ATTN_OK)
            return -1;
        x[k] = m / f.measured[k];
        sx += x[k];
        sxx += x[k] * x[k];
    }
    const double c = sxx > 0 ? sx / sxx : 0;
    double err = 0;
    for (int k = 0; k < f.count; ++k) err += (c * x[k] - 1) * (c * x[k] - 1);
    if (c_out) *c_out = c;
    return std::sqrt(err / f.count);
}
}  // namespace

extern "C" int attn_sched_fit(int count, const int* n, const int* causal, const int* schedule, const int* heads,
                              const int* workers, int placement, const double* measured, double* c, double* r,
                              double* e, double* rms) {
    return attn::guarded([&]() -> int {
        if (count <= 0 || !n || !causal || !schedule || !heads || !workers || !measured || placement < 0 ||
            placement > 2)
            return attn::fail(ATTN_ERR_INVALID_ARG, "attn_sched_fit: invalid arguments");
        for (int k = 0; k < count; ++k)
            if (!(measured[k] > 0) || n[k] <= 0 || heads[k] <= 0 || workers[k] <= 0)
                return attn::fail(ATTN_ERR_INVALID_ARG, "attn_sched_fit: invalid sample");
        const FitData f{count, placement, n, causal, schedule, heads, workers, measured};
        // search in u = log(r/c) in [log 1e-4, log 1e2] and v = log(e/c) in
        // [log 1e-4, log 1e2], with v at its lower end standing for e = 0
        const double ulo = std::log(1e-4), uhi = std::log(1e2), vlo = std::log(1e-4), vhi = std::log(1e2);
        auto eval = [&](double u, double v) {
            return fit_error(f, std::exp(u), v <= vlo ? 0.0 : std::exp(v), nullptr);
        };
        // 1. r/c alone on a grid (e = 0)
        double bu = ulo, bv = vlo, be = -1;
        for (int i = 0; i <= 30; ++i) {
            const double u = ulo + (uhi - ulo) * i / 30, er = eval(u, vlo);
            if (er < 0) return attn::fail(ATTN_ERR_UNSUPPORTED, "attn_sched_fit: a sample cannot be simulated");
            if (be < 0 || er < be) { be = er; bu = u; }
        }
        // 2. e/c on a grid at that r/c
        for (int j = 1; j <= 15; ++j) {
            const double v = vlo + (vhi - vlo) * j / 15, er = eval(bu, v);
            if (er < be) { be = er; bv = v; }
        }
        // 3. pattern search in (u, v), halving the step when no neighbour helps
        double step = (uhi - ulo) / 30;
        while (step > 1e-4) {
            bool moved = false;
            const double du[4] = {step, -step, 0, 0}, dv[4] = {0, 0, step, -step};
            for (int d = 0; d < 4; ++d) {
                const double u = std::min(uhi, std::max(ulo, bu + du[d]));
                const double v = std::min(vhi, std::max(vlo, bv + dv[d]));
                const double er = eval(u, v);
                if (er >= 0 && er < be * (1 - 1e-12)) { be = er; bu = u; bv = v; moved = true; }
            }
            if (!moved) step *= 0.5;
        }
        double cc = 0;
        fit_error(f, std::exp(bu), bv <= vlo ? 0.0 : std::exp(bv), &cc);
        if (c) *c = cc;
        if (r) *r = cc * std::exp(bu);
        if (e) *e = bv <= vlo ? 0.0 : cc * std::exp(bv);
        if (rms) *rms = be;
        return ATTN_OK;
    });
}
