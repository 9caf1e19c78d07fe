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
  * Rectangular tiles (Br != Bc; the pages draw square tiles only), with
    r = Bc / Br (`ratio` in the code): a KV tile of Bc rows and Q tiles of
    Br rows, so a head
    has n KV tiles and r*n Q tiles.  Q tile j sees KV tile i under the causal
    mask when some key of the KV tile is at or before some query of the Q
    tile: r*i <= j.  Naive and Descending keep their orders.  Shift: KV tile
    i visits Q tiles (r*i + t) mod r*n, so at every step the items of a head
    are on distinct Q tiles, and dQ_j is accumulated in visiting order.
    Symmetric Shift (causal, n even, h = n/2): item p pairs KV p (Q tiles
    r*p .. r*n-1) with KV n-1-p (Q tiles r*(n-1-p) .. r*n-1), n*r + r tasks
    in all; phase 1 (t < r*h): (KV p, Q r*h + (r*p + t) mod r*h); phase 2
    (u < r*h + r), with x = r*p + u: (KV p, Q x) while x < r*h, then
    (KV n-1-p, Q 3*r*h - 1 - x).  At a fixed step x differs between items
    and maps to distinct Q tiles, so the fold stays conflict-free; with r = 1
    every rule above is the square one.
"""
from __future__ import annotations

from fractions import Fraction
from itertools import permutations, product

SCHEDULES = ("naive", "descending", "shift", "symmetric_shift")


def allowed(causal: bool, kv: int, q: int, ratio: int = 1) -> bool:
    """Task (KV_kv, Q_q) exists unless the causal mask removes it: with
    `ratio` Q tiles per KV tile, query tile q sees key tiles
    0..floor(q/ratio) (square tiles, ratio 1: key tiles 0..q)."""
    return (not causal) or ratio * kv <= q


# --------------------------------------------------------------------------
# Schedule definitions for one head: work items and dQ accumulation orders.
# --------------------------------------------------------------------------
def head_items(name: str, n: int, causal: bool, ratio: int = 1):
    """Work items of one head, each an ordered list of (kv, q) tasks, for n KV
    tiles and ratio*n Q tiles.  An item runs start to finish on one SM; a KV tile
    never spans two items."""
    if name == "symmetric_shift" and not causal:
        name = "shift"
    nq = ratio * n
    if name == "naive":
        return [[(i, j) for j in range(nq) if allowed(causal, i, j, ratio)] for i in range(n)]
    if name == "descending":
        return [[(i, j) for j in reversed(range(nq)) if allowed(causal, i, j, ratio)] for i in range(n)]
    if name == "shift":
        return [[(i, (ratio * i + t) % nq) for t in range(nq) if allowed(causal, i, (ratio * i + t) % nq, ratio)]
                for i in range(n)]
    if name == "symmetric_shift":
        if n % 2:
            raise ValueError("symmetric shift needs an even number of KV tiles")
        h = n // 2
        items = []
        for p in range(h):
            tasks = [(p, ratio * h + (ratio * p + t) % (ratio * h)) for t in range(ratio * h)]
            for u in range(ratio * h + ratio):
                x = ratio * p + u
                if x < ratio * h:
                    tasks.append((p, x))
                else:
                    tasks.append((n - 1 - p, 3 * ratio * h - 1 - x))
            items.append(tasks)
        return items
    raise ValueError(f"unknown schedule {name!r}")


def dq_orders(name: str, n: int, causal: bool, round_size=None, ratio: int = 1):
    """For each of the ratio*n Q tiles, the list of KV tiles in dQ accumulation
    order.  round_size (Shift, square tiles only): KV tiles per round; None
    means one round."""
    if name == "symmetric_shift" and not causal:
        name = "shift"
    nq = ratio * n
    if name in ("naive", "descending"):
        return [[i for i in range(n) if allowed(causal, i, j, ratio)] for j in range(nq)]
    if name == "shift":
        if round_size and ratio != 1:
            raise ValueError("Shift in rounds is defined for square tiles")
        w = round_size or n
        # round first (KV tile i is in round i // w), then the step at which
        # KV tile i reaches Q tile j: (j - ratio*i) mod ratio*n
        return [sorted((i for i in range(n) if allowed(causal, i, j, ratio)), key=lambda i: (i // w, (j - ratio * i) % nq))
                for j in range(nq)]
    if name == "symmetric_shift":
        # step order: position of each task inside its item
        step = {}
        for tasks in head_items(name, n, causal, ratio):
            for t, (kv, q) in enumerate(tasks):
                step[(kv, q)] = t
        return [sorted((i for i in range(n) if allowed(causal, i, j, ratio)),
                       key=lambda i: step[(i, j)]) for j in range(nq)]
    raise ValueError(f"unknown schedule {name!r}")


def rank_table(name: str, n: int, causal: bool, round_size=None, ratio: int = 1):
    """rank[kv][q] = position of KV tile kv in dQ_q's accumulation order, or
    -1 for a masked task (n rows, ratio*n columns)."""
    rank = [[-1] * (ratio * n) for _ in range(n)]
    for q, order in enumerate(dq_orders(name, n, causal, round_size, ratio)):
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


def place_static(name, n, causal, heads, sms, round_size=None, ratio=1):
    """Head-major items dealt round-robin to `sms` SMs, each SM running its
    items in increasing item order (one head's items are numbered in the
    order head_items lists them)."""
    items = head_items(name, n, causal, ratio)
    sm_tasks = [[] for _ in range(sms)]
    g = 0
    for hd in range(heads):
        for tasks in items:
            sm_tasks[g % sms].extend((hd, kv, q) for kv, q in tasks)
            g += 1
    orders = {(hd, q): kvs for hd in range(heads)
              for q, kvs in enumerate(dq_orders(name, n, causal, round_size, ratio))}
    return sm_tasks, orders


def makespan(name, n, causal, heads=1, sms=None, c=1, r=1, round_size=None, ratio=1):
    """Critical path of a schedule under static head-major placement on `sms`
    SMs (default n), with `ratio` Q tiles per KV tile.  None means
    deadlock.  (r is the reduction cost, as in the pages' notation.)"""
    sm_tasks, orders = place_static(name, n, causal, heads, sms or n, round_size, ratio)
    res = longest_path(*build_dag(sm_tasks, orders, c, r))
    return None if res is None else res[0]


def brute_force_optimum(n, causal, c, r, ratio=1):
    """Smallest makespan over every schedule of one head on n SMs with KV_i on
    SM i: every visiting order of each SM and every dQ accumulation order of
    each of the ratio*n Q tiles (tiny n only)."""
    nq = ratio * n
    per_sm = [[q for q in range(nq) if allowed(causal, i, q, ratio)] for i in range(n)]
    per_q = [[i for i in range(n) if allowed(causal, i, q, ratio)] for q in range(nq)]
    best = None
    for visit in product(*(list(permutations(x)) for x in per_sm)):
        sm_tasks = [[(0, i, q) for q in visit[i]] for i in range(n)]
        for red in product(*(list(permutations(x)) for x in per_q)):
            orders = {(0, q): list(red[q]) for q in range(nq)}
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


def closed_form_full_rect(m, n, ratio, c, r):
    """Full-mask Shift with `ratio` Q tiles per KV tile on n SMs: each SM
    runs m*ratio*n tasks, and every Q tile's contributors arrive `ratio`
    steps apart, so nothing waits: the total work per SM, m*ratio*n*(c+r)."""
    return m * ratio * n * (c + r)


def closed_form_causal_rect(m, n, ratio, c, r):
    """Causal Symmetric Shift with `ratio` Q tiles per KV tile, m even, on n
    SMs: every folded item has ratio*n + ratio tasks and each SM runs m/2 of
    them, so the total work per SM is m*(ratio*n + ratio)*(c+r)/2 (ratio 1:
    the pages' m*(n+1)*(c+r)/2)."""
    return Fraction(m * (ratio * n + ratio)) * (c + r) / 2


def closed_form_causal(m, n, c, r):
    """m*(n+1)*(c+r)/2, the causal figure the paper states for Symmetric Shift
    (review page, major comment 1: a load-balancing bound)."""
    return Fraction(m * (n + 1)) * (c + r) / 2
