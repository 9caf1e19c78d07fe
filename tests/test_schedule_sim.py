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


@pytest.mark.parametrize("placement", [0, 1])
@pytest.mark.parametrize("m,n", [(1, 4), (2, 8), (3, 16), (4, 64)])
def test_simulator_closed_form_full(placement, m, n):
    for c, r in ((1, 1), (3, 1), (0.5, 2)):
        got = tsa.attn_dagsim(n, False, "shift", m, n, placement, c, r)[0]
        assert got == m * n * (c + r)


@pytest.mark.parametrize("placement", [0, 1])
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
