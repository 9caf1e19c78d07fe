"""Oracle for the scheduling side of the deterministic attention backward.

TEST INFRASTRUCTURE ONLY: only tests, the smoke check and the benchmark's CPU
baseline leg may import this module.  It shares no code with the product's
schedule generator or simulator.

What it follows (DASH paper, as summarised on the pith.science review page):
  * "What carries the argument": each (KV_i, Q_j) task is a chain of a
    compute phase C(i,j) of cost c and a reduction phase R(i,j) of cost r;
    zero-weight edges impose the fixed dQ accumulation order; the objective
    is the critical path (the makespan).
  * Axiom ledger: all operations of one KV tile run contiguously on one SM;
    the number of KV tiles equals the number of SMs n; heads are handled by
    aggregation.
  * The schedules: the FlashAttention-3 baseline (Fig. 3), Descending Q-Tile
    Iteration (Fig. 4), Shift Scheduling (Fig. 6, cyclic order), Symmetric
    Shift Scheduling with two-phase workload folding (Fig. 7 caption).

Everything here is plain Python: explicit node/edge lists and a longest-path
over a topological order (Kahn), so that a reader can check it by eye.

Readings taken where the pages are silent (each also listed in the design
notes):
  * Baseline: the SM owning KV_i visits Q tiles in ascending order and dQ_j
    is accumulated in ascending KV order.
  * Descending: Q tiles visited in descending order; the dQ order stays the
    baseline's ascending KV order.
  * Shift: the SM owning KV_i visits Q_{(i+t) mod n}, t = 0..n-1, and dQ_j is
    accumulated by KV j, j-1, ..., j+1 (mod n), i.e. in the order the tasks
    occur.  Under the causal mask the same cyclic order is kept and masked
    tiles are skipped.
  * Shift with more KV tiles than SMs (Axiom ledger: the case KV tiles != SMs
    is handled by refining heads): the KV tiles of a head are cut into
    consecutive rounds of at most `round_size` tiles; every item keeps
    Shift's cyclic visiting order, and dQ_j is accumulated round by round,
    inside a round in the order the round's tasks occur.  With one round
    (round_size >= n) this is Shift.
  * Symmetric Shift (causal, n even, h = n/2): the SM p < h owns KV_p and then
    KV_{n-1-p}.  Phase 1 (steps t < h): (KV_p, Q_{h + (p+t) mod h}), the dense
    lower-left rectangle.  Phase 2 (steps h+u, u = 0..h): (KV_p, Q_{p+u})
    while u < h-p (upper-left triangle from the diagonal), then
    (KV_{n-1-p}, Q_{n-1+h-p-u}) (lower-right triangle from the bottom row up
    to the diagonal).  dQ_j is accumulated in step order.  Under the full
    mask the fold is empty and the schedule is Shift.
"""
from __future__ import annotations

from fractions import Fraction
from itertools import permutations, product

SCHEDULES = ("naive", "descending", "shift", "symmetric_shift")


def allowed(causal: bool, kv: int, q: int) -> bool:
    """Task (KV_kv, Q_q) exists unless the causal mask removes it (square
    tiles, query tile q sees key tiles 0..q)."""
    return (not causal) or kv <= q


# --------------------------------------------------------------------------
# Schedule definitions for one head: work items and dQ accumulation orders.
# --------------------------------------------------------------------------
def head_items(name: str, n: int, causal: bool):
    """Work items of one head, each an ordered list of (kv, q) tasks.  An item
    runs start to finish on one SM; a KV tile never spans two items."""
    if name == "symmetric_shift" and not causal:
        name = "shift"
    if name == "naive":
        return [[(i, j) for j in range(n) if allowed(causal, i, j)] for i in range(n)]
    if name == "descending":
        return [[(i, j) for j in reversed(range(n)) if allowed(causal, i, j)] for i in range(n)]
    if name == "shift":
        return [[(i, (i + t) % n) for t in range(n) if allowed(causal, i, (i + t) % n)]
                for i in range(n)]
    if name == "symmetric_shift":
        if n % 2:
            raise ValueError("symmetric shift needs an even number of tiles")
        h = n // 2
        items = []
        for p in range(h):
            tasks = [(p, h + (p + t) % h) for t in range(h)]
            for u in range(h + 1):
                if u < h - p:
                    tasks.append((p, p + u))
                else:
                    tasks.append((n - 1 - p, n - 1 + h - p - u))
            items.append(tasks)
        return items
    raise ValueError(f"unknown schedule {name!r}")


def dq_orders(name: str, n: int, causal: bool, round_size=None):
    """For each Q tile, the list of KV tiles in dQ accumulation order.
    round_size (Shift only): KV tiles per round; None means one round."""
    if name == "symmetric_shift" and not causal:
        name = "shift"
    if name in ("naive", "descending"):
        return [[i for i in range(n) if allowed(causal, i, j)] for j in range(n)]
    if name == "shift":
        w = round_size or n
        # round first (KV tile i is in round i // w), then the step at which
        # KV tile i reaches Q tile j: (j - i) mod n
        return [sorted((i for i in range(n) if allowed(causal, i, j)), key=lambda i: (i // w, (j - i) % n))
                for j in range(n)]
    if name == "symmetric_shift":
        # step order: position of each task inside its item
        step = {}
        for tasks in head_items(name, n, causal):
            for t, (kv, q) in enumerate(tasks):
                step[(kv, q)] = t
        return [sorted((i for i in range(n) if allowed(causal, i, j)),
                       key=lambda i: step[(i, j)]) for j in range(n)]
    raise ValueError(f"unknown schedule {name!r}")


def rank_table(name: str, n: int, causal: bool, round_size=None):
    """rank[kv][q] = position of KV tile kv in dQ_q's accumulation order, or
    -1 for a masked task."""
    rank = [[-1] * n for _ in range(n)]
    for q, order in enumerate(dq_orders(name, n, causal, round_size)):
        for pos, kv in enumerate(order):
            rank[kv][q] = pos
    return rank


# --------------------------------------------------------------------------
# DAG and critical path.
# --------------------------------------------------------------------------
def build_dag(sm_tasks, orders, c, r):
    """Node-weighted DAG of a schedule.

    sm_tasks: per SM, the ordered list of tasks (head, kv, q) it runs.
    orders:   dict (head, q) -> list of kv in dQ accumulation order.
    Nodes are ("C", head, kv, q) with weight c and ("R", head, kv, q) with
    weight r.  Edges: C -> R of each task; R of a task -> C of the next task
    on the same SM (the SM runs one phase at a time); and a zero-weight edge
    R(prev contributor) -> R(next contributor) for every dQ order.
    """
    weight, edges = {}, []
    for tasks in sm_tasks:
        prev = None
        for (hd, kv, q) in tasks:
            cn, rn = ("C", hd, kv, q), ("R", hd, kv, q)
            weight[cn], weight[rn] = c, r
            edges.append((cn, rn))
            if prev is not None:
                edges.append((prev, cn))
            prev = rn
    for (hd, q), kvs in orders.items():
        for a, b in zip(kvs, kvs[1:]):
            edges.append((("R", hd, a, q), ("R", hd, b, q)))
    return weight, edges


def longest_path(weight, edges):
    """ASAP start and finish of every node; None if the graph has a cycle
    (a deadlocked schedule).  Returns (makespan, start, finish)."""
    succ = {u: [] for u in weight}
    indeg = {u: 0 for u in weight}
    for a, b in edges:
        succ[a].append(b)
        indeg[b] += 1
    start = {u: 0 for u in weight}
    ready = [u for u in weight if indeg[u] == 0]
    finish, done = {}, 0
    while ready:
        u = ready.pop()
        finish[u] = start[u] + weight[u]
        done += 1
        for v in succ[u]:
            if finish[u] > start[v]:
                start[v] = finish[u]
            indeg[v] -= 1
            if indeg[v] == 0:
                ready.append(v)
    if done != len(weight):
        return None
    return max(finish.values(), default=0), start, finish


def place_static(name, n, causal, heads, sms, round_size=None):
    """Head-major items dealt round-robin to `sms` SMs, each SM running its
    items in increasing item order (one head's items are numbered in the
    order head_items lists them)."""
    items = head_items(name, n, causal)
    sm_tasks = [[] for _ in range(sms)]
    g = 0
    for hd in range(heads):
        for tasks in items:
            sm_tasks[g % sms].extend((hd, kv, q) for kv, q in tasks)
            g += 1
    orders = {(hd, q): kvs for hd in range(heads)
              for q, kvs in enumerate(dq_orders(name, n, causal, round_size))}
    return sm_tasks, orders


def makespan(name, n, causal, heads=1, sms=None, c=1, r=1, round_size=None):
    """Critical path of a schedule under static head-major placement on `sms`
    SMs (default n).  None means deadlock."""
    sm_tasks, orders = place_static(name, n, causal, heads, sms or n, round_size)
    res = longest_path(*build_dag(sm_tasks, orders, c, r))
    return None if res is None else res[0]


def brute_force_optimum(n, causal, c, r):
    """Smallest makespan over every schedule of one head on n SMs with KV_i on
    SM i: every visiting order of each SM and every dQ accumulation order of
    each Q tile (tiny n only)."""
    per_sm = [[q for q in range(n) if allowed(causal, i, q)] for i in range(n)]
    per_q = [[i for i in range(n) if allowed(causal, i, q)] for q in range(n)]
    best = None
    for visit in product(*(list(permutations(x)) for x in per_sm)):
        sm_tasks = [[(0, i, q) for q in visit[i]] for i in range(n)]
        for red in product(*(list(permutations(x)) for x in per_q)):
            orders = {(0, q): list(red[q]) for q in range(n)}
            res = longest_path(*build_dag(sm_tasks, orders, c, r))
            if res is not None and (best is None or res[0] < best):
                best = res[0]
    return best


def closed_form_full(m, n, c, r):
    """Optimal full-mask makespan m*n*(c+r) stated for Shift Scheduling
    ("What would settle it" on the review page)."""
    return m * n * (c + r)


def closed_form_full_rounds(m, n, w, c, r):
    """Full-mask Shift in rounds of w KV tiles on w SMs (w divides n): each
    round is n steps of c + r on every SM, and a round's first contribution
    to a Q tile comes no earlier than the previous round's last, so the
    makespan is the total work over w SMs, m*(n/w)*n*(c+r); with w = n it
    is the pages' m*n*(c+r)."""
    return m * (n // w) * n * (c + r)


def closed_form_causal(m, n, c, r):
    """m*(n+1)*(c+r)/2, the causal figure the paper states for Symmetric Shift
    (review page, major comment 1: a load-balancing bound)."""
    return Fraction(m * (n + 1)) * (c + r) / 2
