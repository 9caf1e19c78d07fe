"""Pins of the schedule/DAG oracle against what the pages state and against
brute force: the optimal full-mask critical path m*n*(c+r), the causal figure
m*(n+1)*(c+r)/2, the n = 2, m = 1 counterexample from the review page,
Lemma 1's depth condition on isomorphic chains, and hand-derived closed forms
of the baseline schedules."""
import json
import os
import random
from fractions import Fraction

import pytest

from oracle import dag

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "dag_closed_forms.json")
COSTS = [(1, 1), (3, 1), (1, 3), (Fraction(5, 2), Fraction(1, 3))]


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def test_golden_fixture_has_citations():
    g = _golden()
    for key in ("full_mask_optimum", "causal_claim", "causal_counterexample"):
        assert "citation" in g[key] and g[key]["citation"]


@pytest.mark.parametrize("name", dag.SCHEDULES)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n", [1, 2, 3, 4, 6, 8])
def test_schedule_covers_every_task_once_and_contiguously(name, causal, n):
    if name == "symmetric_shift" and causal and n % 2:
        with pytest.raises(ValueError):
            dag.head_items(name, n, causal)
        return
    items = dag.head_items(name, n, causal)
    tasks = [t for it in items for t in it]
    want = {(i, j) for i in range(n) for j in range(n) if dag.allowed(causal, i, j)}
    assert sorted(tasks) == sorted(want)
    # contiguity: the tasks of one KV tile form one unbroken run in one item
    owner = {}
    for x, it in enumerate(items):
        runs = [kv for p, (kv, _) in enumerate(it) if p == 0 or it[p - 1][0] != kv]
        assert len(runs) == len(set(runs))
        for kv in runs:
            assert kv not in owner
            owner[kv] = x
    orders = dag.dq_orders(name, n, causal)
    for j, kvs in enumerate(orders):
        assert sorted(kvs) == [i for i in range(n) if dag.allowed(causal, i, j)]


@pytest.mark.parametrize("n", [2, 3, 4, 8, 16])
def test_shift_is_conflict_free(n):
    """No two SMs touch the same Q tile at the same step (Fig. 6 caption)."""
    for causal in (False,):
        items = dag.head_items("shift", n, causal)
        for t in range(n):
            qs = [it[t][1] for it in items]
            assert len(set(qs)) == n


@pytest.mark.parametrize("n", [2, 4, 8, 16, 64])
def test_symmetric_shift_is_conflict_free_and_balanced(n):
    items = dag.head_items("symmetric_shift", n, True)
    assert len(items) == n // 2
    assert all(len(it) == n + 1 for it in items)
    for t in range(n + 1):
        qs = [it[t][1] for it in items]
        assert len(set(qs)) == len(qs)


@pytest.mark.parametrize("c,r", COSTS)
@pytest.mark.parametrize("n", [1, 2, 3, 4, 8, 16])
@pytest.mark.parametrize("m", [1, 2, 3])
def test_shift_reaches_full_mask_optimum(m, n, c, r):
    assert dag.makespan("shift", n, False, heads=m, sms=n, c=c, r=r) == dag.closed_form_full(m, n, c, r)


@pytest.mark.parametrize("c,r", COSTS)
@pytest.mark.parametrize("n", [2, 4, 8, 16])
@pytest.mark.parametrize("m", [2, 4])
def test_symmetric_shift_reaches_causal_figure(m, n, c, r):
    got = dag.makespan("symmetric_shift", n, True, heads=m, sms=n, c=c, r=r)
    assert got == dag.closed_form_causal(m, n, c, r)


@pytest.mark.parametrize("c,r", COSTS[:3])
def test_counterexample_n2_m1(c, r):
    g = _golden()["causal_counterexample"]
    best = dag.brute_force_optimum(2, True, c, r)
    assert best == Fraction(g["minimum_multiple_of_c_plus_r"]) * (c + r)
    assert best > Fraction(g["claimed_multiple_of_c_plus_r"]) * (c + r)
    assert dag.closed_form_causal(1, 2, c, r) == Fraction(3, 2) * (c + r)


@pytest.mark.parametrize("c,r", [(1, 1), (2, 1)])
def test_brute_force_full_mask_optimum_matches_shift(c, r):
    for n in (2, 3):
        assert dag.brute_force_optimum(n, False, c, r) == n * (c + r)
        assert dag.makespan("shift", n, False, c=c, r=r) == n * (c + r)


def test_brute_force_causal_n3():
    # KV0 feeds three Q tiles, so 3(c+r) is a lower bound; Descending meets it.
    assert dag.brute_force_optimum(3, True, 1, 1) == 6
    assert dag.makespan("descending", 3, True) == 6


@pytest.mark.parametrize("c,r", COSTS)
@pytest.mark.parametrize("n", [1, 2, 5, 8])
def test_baseline_closed_forms(n, c, r):
    """Hand-derived for one head on n SMs: with the ascending dQ order,
    R(i, j) of the full-mask baseline ends at (j+1)(c+r) + i*r, so the
    makespan is n(c+r) + (n-1)r; causal baseline: R(i, j) ends at
    (j+1)c + (i+j+1)r, makespan nc + (2n-1)r; Descending: SM i ends at
    (n-i)(c+r) + i*r <= n(c+r); causal Shift has no waits, n(c+r)."""
    assert dag.makespan("naive", n, False, c=c, r=r) == n * (c + r) + (n - 1) * r
    assert dag.makespan("naive", n, True, c=c, r=r) == n * c + (2 * n - 1) * r
    assert dag.makespan("descending", n, True, c=c, r=r) == n * (c + r)
    assert dag.makespan("shift", n, True, c=c, r=r) == n * (c + r)


def test_shift_with_too_few_sms_deadlocks():
    """Shift's cyclic dependencies need every KV tile of a head resident at
    once: with fewer SMs than tiles the DAG has a cycle."""
    assert dag.makespan("shift", 4, False, sms=3) is None
    assert dag.makespan("naive", 4, False, sms=3) is not None


def test_lemma1_depth_condition_on_isomorphic_chains():
    """Lemma 1 (review page, 'What carries the argument'): on n isomorphic
    parallel chains, an added zero-weight edge u -> v keeps the critical path
    iff u finishes no later than v starts in the schedule without the edge."""
    rng = random.Random(5)
    for _ in range(300):
        n, length = rng.randint(2, 4), rng.randint(1, 4)
        c, r = rng.randint(1, 4), rng.randint(1, 4)
        sm_tasks = [[(0, i, j) for j in range(length)] for i in range(n)]
        weight, edges = dag.build_dag(sm_tasks, {}, c, r)
        base, start, finish = dag.longest_path(weight, edges)
        nodes = list(weight)
        u, v = rng.sample(nodes, 2)
        if u[2] == v[2]:
            continue  # same chain: not the case the lemma covers
        res = dag.longest_path(weight, edges + [(u, v)])
        assert res is not None
        assert (res[0] == base) == (finish[u] <= start[v])


def test_rank_table_matches_orders():
    for name in dag.SCHEDULES:
        for causal in (False, True):
            n = 6
            rank = dag.rank_table(name, n, causal)
            for j, kvs in enumerate(dag.dq_orders(name, n, causal)):
                assert [rank[i][j] for i in kvs] == list(range(len(kvs)))
                for i in range(n):
                    if not dag.allowed(causal, i, j):
                        assert rank[i][j] == -1


# ------------------------------------------------ Shift in rounds (refining)
@pytest.mark.parametrize("n,w", [(4, 2), (6, 2), (6, 3), (8, 4), (9, 3), (8, 8), (5, 2)])
@pytest.mark.parametrize("causal", [False, True])
def test_shift_rounds_orders_are_round_major_and_conflict_free(n, w, causal):
    """Every dQ order lists its contributors round by round (round of KV tile
    i = i // w), inside a round in the order they reach the Q tile; inside a
    round no two SMs touch one Q tile at one step; one round is plain Shift."""
    orders = dag.dq_orders("shift", n, causal, round_size=w)
    items = dag.head_items("shift", n, causal)
    step = {(kv, q): t for it in items for t, (kv, q) in enumerate(it)}
    for j, kvs in enumerate(orders):
        assert sorted(kvs) == [i for i in range(n) if dag.allowed(causal, i, j)]
        rounds = [i // w for i in kvs]
        assert rounds == sorted(rounds)
        for a, b in zip(kvs, kvs[1:]):
            if a // w == b // w:
                assert (j - a) % n < (j - b) % n
    if not causal:
        for r0 in range(0, n, w):
            for t in range(n):
                qs = [(i + t) % n for i in range(r0, min(n, r0 + w))]
                assert len(qs) == len(set(qs))
    if w >= n:
        assert orders == dag.dq_orders("shift", n, causal)


@pytest.mark.parametrize("n,w", [(4, 2), (6, 2), (6, 3), (8, 4), (8, 2)])
def test_shift_rounds_reach_the_total_work_bound(n, w):
    """Full mask, w SMs, rounds of w tiles: the critical path equals the work
    per SM, m*(n/w)*n*(c+r) (m*n*(c+r) when w = n, the review page's
    T_full^opt), for several cost ratios and two heads."""
    for c, r in COSTS:
        for m in (1, 2):
            got = dag.makespan("shift", n, False, heads=m, sms=w, c=c, r=r, round_size=w)
            assert got == dag.closed_form_full_rounds(m, n, w, c, r), (n, w, c, r, m)
    assert dag.closed_form_full_rounds(3, 8, 8, 2, 1) == dag.closed_form_full(3, 8, 2, 1)


@pytest.mark.parametrize("n,w", [(4, 2), (6, 3), (8, 4)])
def test_shift_rounds_need_a_whole_round_resident(n, w):
    """Waits inside a round wrap around the round (as in Shift), so a round's
    w items must run at once: w SMs finish, w - 1 SMs deadlock."""
    assert dag.makespan("shift", n, False, sms=w, round_size=w) is not None
    assert dag.makespan("shift", n, False, sms=w - 1, round_size=w) is None


# --------------------------------------------------------------------------
# Rectangular tiles: `ratio` Q tiles of Br = Bc/ratio rows per KV tile of Bc
# rows (Br != Bc).  The pins are coverage, KV contiguity, conflict-freedom,
# the total-work bounds (each SM's task count times c + r) and brute force.
# --------------------------------------------------------------------------
RATIOS = [2, 3, 4]


@pytest.mark.parametrize("ratio", RATIOS)
@pytest.mark.parametrize("name", dag.SCHEDULES)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n", [1, 2, 3, 4, 6])
def test_rect_schedule_covers_every_task_once_and_contiguously(ratio, name, causal, n):
    if name == "symmetric_shift" and causal and n % 2:
        with pytest.raises(ValueError):
            dag.head_items(name, n, causal, ratio)
        return
    items = dag.head_items(name, n, causal, ratio)
    tasks = [t for it in items for t in it]
    # the causal mask by hand: KV tile i holds keys i*Bc .. i*Bc+Bc-1, Q tile
    # j holds queries j*Br .. j*Br+Br-1 with Bc = ratio*Br; the task exists
    # when the first key is at or before the last query
    br = 4
    bc = ratio * br
    want = {(i, j) for i in range(n) for j in range(ratio * n) if not causal or i * bc <= j * br + br - 1}
    assert len(tasks) == len(set(tasks)) and set(tasks) == want
    for it in items:  # each KV tile's tasks are one contiguous run
        kvs = [kv for kv, _ in it]
        runs = [k for i, k in enumerate(kvs) if i == 0 or kvs[i - 1] != k]
        assert len(runs) == len(set(runs))


@pytest.mark.parametrize("ratio", RATIOS)
@pytest.mark.parametrize("n", [2, 3, 5, 8])
def test_rect_shift_is_conflict_free_with_contributions_ratio_steps_apart(ratio, n):
    items = dag.head_items("shift", n, False, ratio)
    for t in range(ratio * n):
        qs = [it[t][1] for it in items]
        assert len(qs) == len(set(qs))
    step = {(kv, q): t for it in items for t, (kv, q) in enumerate(it)}
    for q, order in enumerate(dag.dq_orders("shift", n, False, None, ratio)):
        steps = [step[(kv, q)] for kv in order]
        assert steps == sorted(steps) and all(b - a == ratio for a, b in zip(steps, steps[1:]))


@pytest.mark.parametrize("ratio", RATIOS)
@pytest.mark.parametrize("n", [2, 4, 6, 8])
def test_rect_symmetric_shift_is_conflict_free_and_balanced(ratio, n):
    items = dag.head_items("symmetric_shift", n, True, ratio)
    assert len(items) == n // 2
    assert all(len(it) == ratio * n + ratio for it in items)
    for t in range(ratio * n + ratio):
        qs = [it[t][1] for it in items]
        assert len(qs) == len(set(qs))


def test_rect_symmetric_shift_with_ratio_one_is_the_square_fold():
    for n in (2, 4, 6, 8):
        h = n // 2
        square = []
        for p in range(h):
            tasks = [(p, h + (p + t) % h) for t in range(h)]
            tasks += [(p, p + u) if u < h - p else (n - 1 - p, n - 1 + h - p - u) for u in range(h + 1)]
            square.append(tasks)
        assert dag.head_items("symmetric_shift", n, True, 1) == square


@pytest.mark.parametrize("ratio", RATIOS)
@pytest.mark.parametrize("m,n", [(1, 2), (2, 4), (3, 6)])
@pytest.mark.parametrize("c,r", COSTS)
def test_rect_shift_reaches_the_total_work_bound(ratio, m, n, c, r):
    got = dag.makespan("shift", n, False, heads=m, sms=n, c=c, r=r, ratio=ratio)
    assert got == dag.closed_form_full_rect(m, n, ratio, c, r) == m * ratio * n * (c + r)


@pytest.mark.parametrize("ratio", RATIOS)
@pytest.mark.parametrize("m,n", [(2, 2), (2, 4), (4, 6)])
@pytest.mark.parametrize("c,r", COSTS)
def test_rect_symmetric_shift_reaches_the_total_work_bound(ratio, m, n, c, r):
    got = dag.makespan("symmetric_shift", n, True, heads=m, sms=n, c=c, r=r, ratio=ratio)
    assert got == dag.closed_form_causal_rect(m, n, ratio, c, r)
    # ratio 1 is the pages' causal figure
    assert dag.closed_form_causal_rect(m, n, 1, c, r) == dag.closed_form_causal(m, n, c, r)


@pytest.mark.parametrize("c,r", [(1, 1), (3, 1), (1, 3)])
def test_rect_brute_force_full_mask_optimum_is_shift(c, r):
    # n = 2 KV tiles, 4 Q tiles: every visiting and reduction order
    best = dag.brute_force_optimum(2, False, c, r, ratio=2)
    assert best == 4 * (c + r) == dag.makespan("shift", 2, False, c=c, r=r, ratio=2)


def test_rect_brute_force_causal_n2():
    # KV 0 sees Q 0..3, KV 1 sees Q 2..3: six tasks on two SMs, at least
    # four on one of them
    best = dag.brute_force_optimum(2, True, 1, 1, ratio=2)
    assert best == 8
    assert dag.makespan("naive", 2, True, c=1, r=1, ratio=2) >= best
