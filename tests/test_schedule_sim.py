"""Host-side schedule generator and DAG simulator of the library, checked
bit for bit against the oracle's schedule definitions and DAG critical path,
and against the closed forms the pages state (CPU only)."""
from fractions import Fraction

import numpy as np
import pytest

import tile_scheduling_attn_amd as tsa
from oracle import dag

SCHEDS = ("naive", "descending", "shift", "symmetric_shift")


@pytest.mark.parametrize("name", SCHEDS)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 8, 16, 64, 128])
def test_tables_match_oracle(name, causal, n):
    if name == "symmetric_shift" and causal and n % 2:
        with pytest.raises(tsa.AttnError) as e:
            tsa.attn_sched_get(n, causal, name)
        assert e.value.code == -2
        return
    got = tsa.attn_sched_get(n, causal, name)
    items = dag.head_items(name, n, causal)
    assert len(got["item_begin"]) == len(items) + 1
    for x, tasks in enumerate(items):
        a, b = got["item_begin"][x], got["item_begin"][x + 1]
        assert list(zip(got["task_kv"][a:b].tolist(), got["task_q"][a:b].tolist())) == tasks
    assert got["rank"].tolist() == dag.rank_table(name, n, causal)
    assert got["count"].tolist() == [len(o) for o in dag.dq_orders(name, n, causal)]


def test_atomic_has_no_order():
    got = tsa.attn_sched_get(8, True, "atomic")
    assert (got["rank"] == -1).all()
    assert got["count"].tolist() == [j + 1 for j in range(8)]


@pytest.mark.parametrize("name", SCHEDS)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,heads,workers", [(1, 1, 1), (2, 1, 2), (4, 2, 4), (4, 3, 4), (6, 2, 6),
                                             (8, 4, 8), (8, 3, 12), (16, 2, 16), (4, 5, 7)])
@pytest.mark.parametrize("c,r", [(1, 1), (3, 1), (1, 3), (2.5, 0.25)])
def test_simulator_matches_oracle_critical_path(name, causal, n, heads, workers, c, r):
    if name == "symmetric_shift" and causal and n % 2:
        return
    want = dag.makespan(name, n, causal, heads=heads, sms=workers, c=Fraction(c), r=Fraction(r))
    if want is None:
        with pytest.raises(tsa.AttnError) as e:
            tsa.attn_dagsim(n, causal, name, heads, workers, 0, c, r)
        assert e.value.code == -7
        return
    got, wait, busy = tsa.attn_dagsim(n, causal, name, heads, workers, 0, c, r)
    assert got == float(want)
    ntasks = heads * sum(1 for i in range(n) for j in range(n) if dag.allowed(causal, i, j))
    assert busy == pytest.approx(ntasks * (c + r))


@pytest.mark.parametrize("placement", [0, 1, 2])
@pytest.mark.parametrize("m,n", [(1, 4), (2, 8), (3, 16), (4, 64)])
def test_simulator_closed_form_full(placement, m, n):
    for c, r in ((1, 1), (3, 1), (0.5, 2)):
        got = tsa.attn_dagsim(n, False, "shift", m, n, placement, c, r)[0]
        assert got == m * n * (c + r)


@pytest.mark.parametrize("placement", [0, 1, 2])
@pytest.mark.parametrize("m,n", [(2, 2), (2, 8), (4, 16), (6, 64)])
def test_simulator_closed_form_causal(placement, m, n):
    for c, r in ((1, 1), (3, 1), (0.5, 2)):
        got = tsa.attn_dagsim(n, True, "symmetric_shift", m, n, placement, c, r)[0]
        assert got == m * (n + 1) * (c + r) / 2


def test_min_workers():
    assert tsa.attn_sched_min_workers(64, False, "naive") == 1
    assert tsa.attn_sched_min_workers(64, True, "descending") == 1
    assert tsa.attn_sched_min_workers(64, False, "shift") == 64
    assert tsa.attn_sched_min_workers(64, True, "symmetric_shift") == 32
    assert tsa.attn_sched_min_workers(64, False, "symmetric_shift") == 64
    assert tsa.attn_sched_min_workers(64, False, "atomic") == 1


@pytest.mark.parametrize("name,causal", [("shift", False), ("symmetric_shift", True), ("naive", False),
                                         ("descending", True)])
def test_ticket_queue_progresses_with_min_workers(name, causal):
    """With items handed out in increasing order, the minimum worker count
    never deadlocks, for any head count."""
    n = 8
    w = tsa.attn_sched_min_workers(n, causal, name)
    for heads in (1, 2, 3, 5):
        tsa.attn_dagsim(n, causal, name, heads, w, 1, 1.0, 1.0)


def test_shift_below_min_workers_deadlocks():
    with pytest.raises(tsa.AttnError) as e:
        tsa.attn_dagsim(8, False, "shift", 1, 7, 1, 1.0, 1.0)
    assert e.value.code == -7


def test_schedule_argument_errors():
    with pytest.raises(tsa.AttnError):
        tsa.attn_sched_size(-1, False, "naive")
    with pytest.raises(tsa.AttnError):
        tsa.attn_sched_size(4, False, 9)
    with pytest.raises(tsa.AttnError):
        tsa.attn_dagsim(4, False, "naive", 1, 0, 0, 1.0, 1.0)


# ---------------------------------------------------------------- selection
@pytest.mark.parametrize("m,n", [(1, 4), (2, 8), (4, 16)])
@pytest.mark.parametrize("c,r", [(1, 1), (3, 1), (1, 0.25)])
def test_select_full_mask_picks_shift_at_the_bound(m, n, c, r):
    name, t = tsa.attn_sched_select(n, False, m, n, c, r)
    assert name == "shift"
    assert t == float(dag.closed_form_full(m, n, Fraction(c), Fraction(r)))


@pytest.mark.parametrize("m,n", [(2, 4), (2, 8), (4, 16)])
@pytest.mark.parametrize("c,r", [(1, 1), (3, 1), (1, 0.25)])
def test_select_causal_picks_symmetric_shift_at_the_bound(m, n, c, r):
    """With at least two heads the workers Symmetric Shift leaves free are
    used by the next head, and it reaches m(n+1)(c+r)/2."""
    name, t = tsa.attn_sched_select(n, True, m, n, c, r)
    assert name == "symmetric_shift"
    assert t == float(dag.closed_form_causal(m, n, Fraction(c), Fraction(r)))


def test_select_causal_single_head_prefers_descending():
    """One head on n workers: the fold leaves half the workers idle, and
    Descending (tied with the causal Shift; the lower id wins) is faster."""
    name, t = tsa.attn_sched_select(8, True, 1, 8, 1.0, 1.0)
    assert name == "descending"
    assert t == tsa.attn_dagsim(8, True, "descending", 1, 8, 1, 1.0, 1.0)[0]
    assert t < tsa.attn_dagsim(8, True, "symmetric_shift", 1, 8, 1, 1.0, 1.0)[0]


def test_select_skips_schedules_that_cannot_run():
    # Shift needs n resident workers; with fewer the baseline orders remain
    name, t = tsa.attn_sched_select(8, False, 2, 4, 1.0, 1.0)
    assert name in ("naive", "descending")
    assert t == tsa.attn_dagsim(8, False, name, 2, 4, 1, 1.0, 1.0)[0]
    # the fold needs an even tile count
    name, _ = tsa.attn_sched_select(5, True, 4, 5, 1.0, 1.0)
    assert name != "symmetric_shift"
    with pytest.raises(tsa.AttnError):
        tsa.attn_sched_select(0, False, 1, 1, 1.0, 1.0)


# ---------------------------------------------------------------- calibration
def _samples(c, r, e=0.0, scale=None):
    cases = [(8, False, "shift", 2, 8), (8, False, "naive", 2, 8), (8, True, "descending", 2, 8),
             (8, True, "symmetric_shift", 2, 8), (16, True, "naive", 3, 16)]
    out = []
    for k, (n, causal, name, heads, workers) in enumerate(cases):
        t = tsa.attn_dagsim_edge(n, causal, name, heads, workers, 1, c, r, e)[0]
        out.append((n, causal, name, heads, workers, t * (scale[k] if scale else 1.0)))
    return out


@pytest.mark.parametrize("c,r,e", [(2.0, 0.7, 0.0), (1.0, 1.0, 0.0), (0.3, 2.5, 0.0), (5.0, 0.05, 0.0),
                                   (2.0, 0.7, 0.4), (1.0, 0.5, 1.5)])
def test_fit_reproduces_simulated_timings(c, r, e):
    """Timings pin down c + r (a worker's time per task) and r + e (a link of
    a reduction chain), not the three costs one by one, so the check is on
    what the fitted model predicts: every sample, to the fit's tolerance."""
    samples = _samples(c, r, e)
    fc, fr, fe, rms = tsa.attn_sched_fit(samples)
    assert rms < 1e-4
    assert fc + fr == pytest.approx(c + r, rel=1e-3)
    assert fr + fe == pytest.approx(r + e, rel=1e-2, abs=1e-3)
    for (n, causal, name, heads, workers, t) in samples:
        assert tsa.attn_dagsim_edge(n, causal, name, heads, workers, 1, fc, fr, fe)[0] == pytest.approx(t, rel=1e-3)


def test_fit_tolerates_noise():
    noise = [1.02, 0.98, 1.01, 0.99, 1.015]
    fc, fr, fe, rms = tsa.attn_sched_fit(_samples(2.0, 0.7, 0.0, noise))
    assert fc == pytest.approx(2.0, rel=0.1)
    assert rms < 0.03
    for (n, causal, name, heads, workers, t) in _samples(2.0, 0.7, 0.0, noise):
        pred = tsa.attn_dagsim_edge(n, causal, name, heads, workers, 1, fc, fr, fe)[0]
        assert pred == pytest.approx(t, rel=0.06)


def test_edge_cost_of_zero_is_the_pages_model():
    for name, causal in (("naive", False), ("shift", False), ("descending", True), ("symmetric_shift", True)):
        assert tsa.attn_dagsim_edge(8, causal, name, 2, 8, 1, 1.5, 0.5, 0.0) == \
            tsa.attn_dagsim(8, causal, name, 2, 8, 1, 1.5, 0.5)


def test_edge_cost_delays_the_serial_chain_but_not_shift():
    """Naive full: every contributor waits on the previous one, so each edge
    adds to the critical path; Shift staggers the contributors by a whole
    task, so an edge shorter than the compute phase costs nothing."""
    c, r = 1.0, 0.5
    base = tsa.attn_dagsim(8, False, "naive", 1, 8, 1, c, r)[0]
    assert tsa.attn_dagsim_edge(8, False, "naive", 1, 8, 1, c, r, 0.25)[0] > base
    assert tsa.attn_dagsim_edge(8, False, "shift", 1, 8, 1, c, r, 0.25)[0] == \
        float(dag.closed_form_full(1, 8, Fraction(c), Fraction(r)))


def test_xcd_placement_keeps_whole_heads_on_one_xcd():
    """Placement 2 models the kernel's per-XCD queues.  With at least eight
    heads a naive or Descending head runs on one XCD, so no hand-off crosses
    XCDs and the edge cost changes nothing; under one global queue it delays
    the serial chains."""
    c, r, e = 1.0, 0.5, 0.75
    for name, causal in (("naive", False), ("descending", True)):
        base = tsa.attn_dagsim_edge(16, causal, name, 16, 64, 2, c, r, 0.0)[0]
        assert tsa.attn_dagsim_edge(16, causal, name, 16, 64, 2, c, r, e)[0] == base
        assert tsa.attn_dagsim_edge(16, causal, name, 16, 64, 1, c, r, e)[0] > \
            tsa.attn_dagsim_edge(16, causal, name, 16, 64, 1, c, r, 0.0)[0]


def test_xcd_placement_charges_edges_only_between_xcds():
    """Shift at n = 64 on 256 workers: a head's 64 items run as two chunks of
    32 on two XCDs, so 2 of a tile's 63 hand-offs cross XCDs.  With an edge
    longer than a task those crossings delay the launch, but by less than
    when every hand-off pays it, and never below the edge-free makespan."""
    c, r, e = 1.0, 1.0, 2.5
    free = tsa.attn_dagsim_edge(64, False, "shift", 32, 256, 2, c, r, 0.0)[0]
    xcd = tsa.attn_dagsim_edge(64, False, "shift", 32, 256, 2, c, r, e)[0]
    every = tsa.attn_dagsim_edge(64, False, "shift", 32, 256, 1, c, r, e)[0]
    # 32 heads on four groups of 64 workers: 8 heads per group
    assert free == float(dag.closed_form_full(8, 64, Fraction(c), Fraction(r)))
    assert free < xcd < every


def test_placement_argument_is_checked():
    with pytest.raises(tsa.AttnError):
        tsa.attn_dagsim(8, False, "shift", 1, 8, 3, 1.0, 1.0)
    with pytest.raises(tsa.AttnError):
        tsa.attn_sched_select(8, False, 1, 8, 1.0, 1.0, 0.0, placement=-1)
    with pytest.raises(tsa.AttnError):
        tsa.attn_sched_fit([(8, False, "shift", 1, 8, 1.0)], placement=5)


def test_fit_argument_errors():
    with pytest.raises(tsa.AttnError):
        tsa.attn_sched_fit([])
    with pytest.raises(tsa.AttnError):
        tsa.attn_sched_fit([(8, False, "shift", 1, 8, 0.0)])
    with pytest.raises(tsa.AttnError):  # Shift on fewer workers than it needs deadlocks
        tsa.attn_sched_fit([(8, False, "shift", 1, 4, 1.0)])


# ------------------------------------------------ Shift in rounds (n > 256)
@pytest.mark.parametrize("n", [257, 300, 513])
@pytest.mark.parametrize("causal", [False, True])
def test_shift_rounds_match_the_oracle(n, causal):
    """With more than 256 KV tiles Shift runs in rounds of
    ceil(n / ceil(n / 256)) tiles: items, rank table and contributor counts
    equal the oracle's definition with that round size, and the resident
    work groups it needs are one round."""
    rounds = -(-n // 256)
    w = -(-n // rounds)
    got = tsa.attn_sched_get(n, causal, "shift")
    want_items = dag.head_items("shift", n, causal)
    ib = got["item_begin"]
    assert len(ib) == n + 1
    for i, tasks in enumerate(want_items):
        assert list(zip(got["task_kv"][ib[i]:ib[i + 1]], got["task_q"][ib[i]:ib[i + 1]])) == tasks
    assert got["rank"].tolist() == dag.rank_table("shift", n, causal, round_size=w)
    assert tsa.attn_sched_min_workers(n, causal, "shift") == w
    if n <= 256:
        assert w == n


def test_shift_up_to_256_tiles_is_one_round():
    for n in (2, 64, 255, 256):
        assert tsa.attn_sched_min_workers(n, False, "shift") == n
        assert tsa.attn_sched_get(n, False, "shift")["rank"].tolist() == dag.rank_table("shift", n, False)


def test_shift_rounds_simulate_to_the_total_work_bound():
    """n = 512 full mask on 256 workers: two rounds of 256, no waits, the
    critical path is the work per worker, 2 * 512 * (c + r), as the oracle's
    closed form for rounds states; one worker fewer than a round deadlocks."""
    c, r = 3.0, 1.0
    mk, wait, _ = tsa.attn_dagsim(512, False, "shift", 1, 256, 1, c, r)
    assert mk == pytest.approx(dag.closed_form_full_rounds(1, 512, 256, c, r))
    assert wait == pytest.approx(0.0)
    with pytest.raises(tsa.AttnError) as e:
        tsa.attn_dagsim(512, False, "shift", 1, 255, 1, c, r)
    assert e.value.code == -7


# --------------------------------------------------------------------------
# Rectangular tiles (n KV tiles, ratio Q tiles per KV tile)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("ratio", [2, 3, 4])
@pytest.mark.parametrize("name", SCHEDS + ("atomic",))
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n", [1, 2, 3, 4, 6, 8, 16, 64])
def test_rect_tables_match_oracle(ratio, name, causal, n):
    if name == "symmetric_shift" and causal and n % 2:
        with pytest.raises(tsa.AttnError) as e:
            tsa.attn_sched_get_rect(n, ratio, causal, name)
        assert e.value.code == -2
        return
    got = tsa.attn_sched_get_rect(n, ratio, causal, name)
    items = dag.head_items("naive" if name == "atomic" else name, n, causal, ratio)
    assert len(got["item_begin"]) == len(items) + 1
    for x, tasks in enumerate(items):
        a, b = got["item_begin"][x], got["item_begin"][x + 1]
        assert list(zip(got["task_kv"][a:b].tolist(), got["task_q"][a:b].tolist())) == tasks
    if name == "atomic":
        assert (got["rank"] == -1).all()
    else:
        assert got["rank"].tolist() == dag.rank_table(name, n, causal, None, ratio)
    assert got["count"].tolist() == [len(o) for o in dag.dq_orders("naive", n, causal, None, ratio)]
    want_workers = 1 if name in ("naive", "descending", "atomic") else len(items)
    assert tsa.lib.attn_sched_min_workers_rect(n, ratio, int(causal), tsa._sched_id(name)) == want_workers


@pytest.mark.parametrize("ratio", [2, 4])
@pytest.mark.parametrize("name", SCHEDS)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,heads,workers", [(2, 1, 2), (4, 2, 4), (4, 3, 5), (6, 2, 6), (8, 4, 8)])
@pytest.mark.parametrize("c,r", [(1, 1), (3, 1), (2.5, 0.25)])
def test_rect_simulator_matches_oracle_critical_path(ratio, name, causal, n, heads, workers, c, r):
    want = dag.makespan(name, n, causal, heads=heads, sms=workers, c=Fraction(c), r=Fraction(r), ratio=ratio)
    if want is None:
        with pytest.raises(tsa.AttnError) as e:
            tsa.attn_dagsim_rect(n, ratio, causal, name, heads, workers, 0, c, r)
        assert e.value.code == -7
        return
    got, wait, busy = tsa.attn_dagsim_rect(n, ratio, causal, name, heads, workers, 0, c, r)
    assert got == float(want)
    ntasks = heads * sum(1 for i in range(n) for j in range(ratio * n) if dag.allowed(causal, i, j, ratio))
    assert busy == pytest.approx(ntasks * (c + r))


def test_rect_shapes_outside_the_supported_range_are_refused():
    assert tsa.lib.attn_sched_size_rect(4, 0, 0, 0, None, None) == -1       # ratio < 1
    assert tsa.lib.attn_sched_size_rect(4, 9, 0, 0, None, None) == -2       # ratio > 8
    assert tsa.lib.attn_sched_size_rect(300, 2, 0, 2, None, None) == -2     # Shift rounds are square only
    assert tsa.lib.attn_sched_size_rect(1025, 2, 0, 0, None, None) == -2    # more than 2048 Q tiles
    assert tsa.lib.attn_sched_size_rect(300, 2, 0, 0, None, None) == 0      # naive has no rounds
