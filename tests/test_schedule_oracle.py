"""Pins of the schedule and DAG oracles.

The schedules are pinned to the N=4 instantiation of the pages' prose
(tests/golden/schedules_n4.json) and to the properties the pages state:
every task once, a fixed order per dQ tile, shift lockstep without conflicts,
symmetric pairs of N+1 tasks, descending order from N-1 to 0.  The DAG oracle
is pinned to closed-form critical paths derived by hand for one group with one
worker per item, and to Lemma 1's condition.
"""

import itertools
import json
import os

import pytest

from oracle import dag
from oracle import schedule as sch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "schedules_n4.json")

NAMES = {"naive": sch.NAIVE, "descending": sch.DESCENDING_Q, "shift": sch.SHIFT,
         "symmetric": sch.SYMMETRIC_SHIFT}
MASKS = {"full": sch.FULL, "causal": sch.CAUSAL}


def _combos(Ns=(1, 2, 3, 4, 5, 8, 16)):
    for name, s in NAMES.items():
        for mname, m in MASKS.items():
            for N in Ns:
                if s == sch.SYMMETRIC_SHIFT and (m != sch.CAUSAL or N % 2):
                    continue
                yield s, m, N


def test_golden_n4():
    gold = json.load(open(GOLDEN))
    N = gold["N"]
    for key, chains in gold["chains"].items():
        name, mname = key.split("_")
        s, m = NAMES[name], MASKS[mname]
        got = [[j for (_, _, j) in it] for it in sch.items(s, m, N)]
        assert got == chains, key
    for key, orders in gold["dq_order"].items():
        name, mname = key.split("_")
        s, m = NAMES[name], MASKS[mname]
        rk = sch.ranks(s, m, N)
        for j, order in enumerate(orders):
            got = sorted((r, i) for (g, i, jj), r in rk.items() if jj == j)
            assert [i for _, i in got] == order, (key, j)
    pairs = sch.items(sch.SYMMETRIC_SHIFT, sch.CAUSAL, N)
    assert [[[i, j] for (_, i, j) in it] for it in pairs] == gold["symmetric_pairs"]
    for step, tiles in enumerate(gold["symmetric_step_tiles"]):
        assert [it[step][2] for it in pairs] == tiles


@pytest.mark.parametrize("s,m,N", list(_combos()))
@pytest.mark.parametrize("G", [1, 3])
def test_every_task_once_and_ranks_permute(s, m, N, G):
    its = sch.items(s, m, N, G)
    tasks = [t for it in its for t in it]
    want = {(g, i, j) for g in range(G) for i in range(N) for j in range(N)
            if sch.valid(m, i, j)}
    assert len(tasks) == len(want) and set(tasks) == want
    rk = sch.ranks(s, m, N, G)
    for g in range(G):
        for j in range(N):
            rs = sorted(rk[(g, i, j)] for i in sch.contributors(m, N, j))
            assert rs == list(range(len(sch.contributors(m, N, j))))


@pytest.mark.parametrize("s,m,N", list(_combos()))
def test_chains_are_contiguous(s, m, N):
    # the work of one KV tile is an unbroken run inside its item
    for it in sch.items(s, m, N, 2):
        seen = []
        for (_, i, _) in it:
            if not seen or seen[-1] != i:
                assert i not in seen
                seen.append(i)


@pytest.mark.parametrize("N", [1, 2, 3, 4, 5, 8, 16, 32])
@pytest.mark.parametrize("G", [1, 4])
def test_shift_lockstep_conflict_free(N, G):
    for s, m in ((sch.SHIFT, sch.FULL), (sch.SHIFT, sch.CAUSAL),
                 (sch.SYMMETRIC_SHIFT, sch.CAUSAL)):
        if s == sch.SYMMETRIC_SHIFT and N % 2:
            continue
        its = sch.items(s, m, N, G)
        L = max(len(it) for it in its)
        for step in range(L):
            tiles = [(it[step][0], it[step][2]) for it in its if step < len(it)]
            assert len(tiles) == len(set(tiles))
        # arrival order == rank order, and every rank's predecessor arrives
        # strictly earlier (no waiting in lockstep)
        for (g, j), lst in sch.lockstep_steps(s, m, N, G).items():
            lst = sorted(lst)
            rk = sch.ranks(s, m, N, G)
            assert [rk[(g, i, j)] for _, i in lst] == list(range(len(lst)))


@pytest.mark.parametrize("N", [2, 4, 6, 8, 32, 128])
def test_symmetric_pairs_balanced(N):
    for p, it in enumerate(sch.items(sch.SYMMETRIC_SHIFT, sch.CAUSAL, N)):
        assert len(it) == N + 1
        assert {i for (_, i, _) in it} == ({p, N - 1 - p})


def test_descending_order():
    for N in (1, 4, 7):
        assert sch.chain_q_order(sch.DESCENDING_Q, sch.FULL, N, 0) == list(range(N - 1, -1, -1))
        assert sch.chain_q_order(sch.DESCENDING_Q, sch.CAUSAL, N, 2 % N) == \
            list(range(N - 1, (2 % N) - 1, -1))


def test_symmetric_rejects():
    with pytest.raises(ValueError):
        sch.items(sch.SYMMETRIC_SHIFT, sch.FULL, 4)
    with pytest.raises(ValueError):
        sch.items(sch.SYMMETRIC_SHIFT, sch.CAUSAL, 5)


def test_dispatch_order_dependencies():
    # naive and descending only ever wait on earlier chains; the shift family
    # needs the whole group resident
    for N in (2, 4, 8):
        for m in (sch.FULL, sch.CAUSAL):
            assert sch.dispatch_order_ok(sch.NAIVE, m, N, 2)
            assert sch.dispatch_order_ok(sch.DESCENDING_Q, m, N, 2)
        assert not sch.dispatch_order_ok(sch.SHIFT, sch.FULL, N, 1)


# --- DAG oracle ------------------------------------------------------------

CLOSED = [
    # schedule, mask, makespan(N, c, r), violations(N), deficit(c, r)
    (sch.SHIFT, sch.FULL, lambda N, c, r: N * (c + r), lambda N: 0, None),
    (sch.NAIVE, sch.FULL, lambda N, c, r: N * (c + r) + (N - 1) * r,
     lambda N: N * (N - 1), lambda c, r: r),
    (sch.DESCENDING_Q, sch.FULL, lambda N, c, r: N * (c + r) + (N - 1) * r,
     lambda N: N * (N - 1), lambda c, r: r),
    (sch.NAIVE, sch.CAUSAL, lambda N, c, r: N * (c + r) + (N - 1) * r,
     lambda N: N * (N - 1) // 2, lambda c, r: c + 2 * r),
    (sch.DESCENDING_Q, sch.CAUSAL, lambda N, c, r: N * (c + r),
     lambda N: N * (N - 1) // 2, lambda c, r: r),
    (sch.SHIFT, sch.CAUSAL, lambda N, c, r: N * (c + r), lambda N: 0, None),
    (sch.SYMMETRIC_SHIFT, sch.CAUSAL, lambda N, c, r: (N + 1) * (c + r),
     lambda N: 0, None),
]


@pytest.mark.parametrize("case", CLOSED, ids=lambda c: "%d-%d" % (c[0], c[1]))
@pytest.mark.parametrize("N", [2, 4, 8])
@pytest.mark.parametrize("cr", [(4.0, 1.0), (3.0, 2.0)])
def test_dag_closed_forms(case, N, cr):
    s, m, mk, nv, dfc = case
    c, r = cr
    res = dag.simulate(s, m, N, c=c, r=r)
    assert not res["deadlock"]
    assert res["makespan"] == mk(N, c, r)
    assert res["replay_makespan"] == res["makespan"]
    assert res["violations"] == nv(N)
    if dfc is not None and nv(N):
        assert res["max_deficit"] == dfc(c, r)


def test_causal_chain_end_times():
    N, c, r = 6, 5.0, 1.0
    rep = dag.replay(sch.NAIVE, sch.CAUSAL, N, 1, 1, N, "static", c, c, r)
    for i in range(N):
        assert rep["times"][(0, 0, i, N - 1)][3] == N * (c + r) + i * r
    rep = dag.replay(sch.DESCENDING_Q, sch.CAUSAL, N, 1, 1, N, "static", c, c, r)
    for i in range(N):
        assert rep["times"][(0, 0, i, i)][3] == (N - i) * (c + r) + i * r
    rep = dag.replay(sch.SHIFT, sch.CAUSAL, N, 1, 1, N, "static", c, c, r)
    for i in range(N):
        assert rep["times"][(0, 0, i, N - 1)][3] == (N - i) * (c + r)


@pytest.mark.parametrize("s,m", [(sch.NAIVE, sch.FULL), (sch.NAIVE, sch.CAUSAL),
                                 (sch.DESCENDING_Q, sch.CAUSAL),
                                 (sch.SHIFT, sch.FULL), (sch.SHIFT, sch.CAUSAL),
                                 (sch.SYMMETRIC_SHIFT, sch.CAUSAL)])
@pytest.mark.parametrize("P,groups,G", [(3, 2, 1), (8, 3, 2), (5, 4, 3)])
@pytest.mark.parametrize("dispatch", ["static", "dynamic"])
def test_replay_equals_dag_and_lower_bounds(s, m, P, groups, G, dispatch):
    N = 4
    res = dag.simulate(s, m, N, G=G, groups=groups, P=P, dispatch=dispatch,
                       c=3.0, c_diag=2.0, r=1.0)
    items_per_group = len(sch.items(s, m, N, G))
    if res["deadlock"]:
        # only the shift family can stall, and only when a group does not fit
        assert s in (sch.SHIFT, sch.SYMMETRIC_SHIFT) and items_per_group > P
        return
    assert res["makespan"] == res["replay_makespan"]
    longest = max(sum(dag.task_cost(m, i, j, 3.0, 2.0) + 1.0 for (_, i, j) in it)
                  for it in sch.items(s, m, N, G))
    assert res["makespan"] >= longest
    assert res["makespan"] >= res["total_work"] / P - 1e-9
    assert res["makespan"] >= res["base_makespan"]
    if res["violations"] == 0:
        # Lemma 1 (sufficient direction): no violated edge keeps the path
        assert res["makespan"] == res["base_makespan"]


def test_cyclic_rank_override_deadlocks():
    # shift, full mask, N=2: chain 0 visits Q tiles 0 then 1, chain 1 visits
    # 1 then 0.  Reversing both dQ orders makes each chain's first task wait
    # for the other chain's second task: a cycle.
    assert sch.items(sch.SHIFT, sch.FULL, 2) == [[(0, 0, 0), (0, 0, 1)],
                                               [(0, 1, 1), (0, 1, 0)]]
    ok = dag.simulate(sch.SHIFT, sch.FULL, 2, c=1.0, r=1.0)
    assert not ok["deadlock"]
    bad = {(0, 1, 0): 0, (0, 0, 0): 1, (0, 0, 1): 0, (0, 1, 1): 1}
    res = dag.simulate(sch.SHIFT, sch.FULL, 2, rank_map=bad, c=1.0, r=1.0)
    assert res["deadlock"]


def test_lemma1_violation_changes_critical_path():
    # an order edge whose source is deeper than its target lengthens the path
    res = dag.simulate(sch.NAIVE, sch.FULL, 4, c=4.0, r=1.0)
    assert res["violations"] > 0 and res["makespan"] > res["base_makespan"]


def test_oracle_selection_closed_forms():
    # selection = the schedule of least critical path; pinned on shapes whose
    # critical paths have closed forms (one group, one chain per worker)
    from oracle import dag
    N, c, r = 8, 4.0, 1.0
    s, res = dag.select(sch.FULL, N, P=N, c=c, r=r)
    assert s == sch.SHIFT and res["makespan"] == N * (c + r)
    s, res = dag.select(sch.CAUSAL, N, P=N // 2, c=c, r=r)
    assert s == sch.SYMMETRIC_SHIFT and res["makespan"] == (N + 1) * (c + r)
    # odd N, causal: the symmetric shift does not apply
    s, _ = dag.select(sch.CAUSAL, 5, P=5, c=c, r=r)
    assert s != sch.SYMMETRIC_SHIFT
    # a deadlocked candidate is never chosen
    s, _ = dag.select(sch.FULL, N, P=N // 2, dispatch="dynamic", c=c, r=r)
    assert s in (sch.NAIVE, sch.DESCENDING_Q)
    # ties go to the earlier candidate: with r = 0 every order of a full mask
    # on one chain per worker takes N c
    s, res = dag.select(sch.FULL, N, P=N, c=c, r=0.0)
    assert s == sch.SHIFT and res["makespan"] == N * c


# ---------------------------------------------------------------------------
# Grouped-query items: the hand-written G = 2, N = 4 table pins the task order
# inside an item (step outer, head inner; part by part for the symmetric pair).

GOLDEN_G2 = os.path.join(os.path.dirname(__file__), "golden", "schedules_n4_g2.json")
G2_KEYS = {"naive": sch.NAIVE, "descending": sch.DESCENDING_Q, "shift": sch.SHIFT,
           "symmetric": sch.SYMMETRIC_SHIFT, "atomic": sch.ATOMIC}


def _parse_item(text):
    return [tuple(int(v) for v in t.split(",")) for t in text.split()]


def _g2_mismatches(items_fn, ranks_fn):
    """Keys of the G = 2 table whose items or ranks differ from the given
    item and rank functions (an empty list when all agree)."""
    gold = json.load(open(GOLDEN_G2))
    N, G = gold["N"], gold["G"]
    bad = []
    for key, rows in gold["items"].items():
        name, mname = key.split("_")
        s, m = G2_KEYS[name], MASKS[mname]
        want = [_parse_item(r) for r in rows]
        its = items_fn(s, m, N, G)
        rk = ranks_fn(s, m, N, G)
        got = [[(g, i, j, rk[(g, i, j)]) for (g, i, j) in it] for it in its]
        if got != want:
            bad.append(key)
    return bad


def test_golden_n4_g2():
    assert _g2_mismatches(sch.items, sch.ranks) == []


def test_planted_head_outer_order_is_caught():
    # the earlier head-outer order (each walk for one head, then the next)
    # covers the same tasks with the same ranks; only the table tells it apart
    def head_outer(s, m, N, G):
        return [sorted(it, key=lambda t: t[0]) for it in sch.items(s, m, N, G)]
    bad = _g2_mismatches(head_outer, sch.ranks)
    assert len(bad) == len(json.load(open(GOLDEN_G2))["items"])


# ---------------------------------------------------------------------------
# The causal diagonal weight.  With c_diag != c the closed forms of one group
# with a worker per item (derived by hand from the event graph):
#   causal SHIFT: chain i starts on its diagonal tile and never waits, so it
#     ends at c_diag + (N-1-i) c + (N-i) r; the critical path is chain 0's,
#     c_diag + (N-1) c + N r;
#   SYMMETRIC_SHIFT: every pair meets its two diagonal tiles at the same two
#     lockstep steps (the first of phase 2 and the last), so the lockstep
#     holds and the critical path is 2 c_diag + (N-1) c + (N+1) r;
#   total work: N diagonal tiles, N(N-1)/2 others, one reduction per task.

DIAG_CASES = [(2, 5.0, 2.0, 1.0), (4, 5.0, 2.0, 1.0), (8, 3.0, 7.0, 0.5), (6, 4.0, 1.0, 0.0)]


@pytest.mark.parametrize("N,c,cd,r", DIAG_CASES)
def test_dag_causal_diagonal_weight(N, c, cd, r):
    res = dag.simulate(sch.SHIFT, sch.CAUSAL, N, c=c, c_diag=cd, r=r)
    assert not res["deadlock"]
    assert res["makespan"] == cd + (N - 1) * c + N * r
    assert res["total_work"] == N * cd + N * (N - 1) // 2 * c + N * (N + 1) // 2 * r
    assert res["violations"] == 0
    rep = dag.replay(sch.SHIFT, sch.CAUSAL, N, 1, 1, N, "static", c, cd, r)
    for i in range(N):
        assert rep["times"][(0, 0, i, N - 1)][3] == cd + (N - 1 - i) * c + (N - i) * r
    res = dag.simulate(sch.SYMMETRIC_SHIFT, sch.CAUSAL, N, c=c, c_diag=cd, r=r)
    assert not res["deadlock"]
    assert res["makespan"] == 2 * cd + (N - 1) * c + (N + 1) * r
    assert res["violations"] == 0


def test_planted_diagonal_weight_off_by_one_is_caught(monkeypatch):
    # the diagonal weight moved to the tile next to the diagonal
    def shifted(mask, i, j, c, c_diag):
        return c_diag if (mask == sch.CAUSAL and i == j + 1) else c
    monkeypatch.setattr(dag, "task_cost", shifted)
    N, c, cd, r = DIAG_CASES[1]
    res = dag.simulate(sch.SHIFT, sch.CAUSAL, N, c=c, c_diag=cd, r=r)
    assert res["makespan"] != cd + (N - 1) * c + N * r


def test_golden_n4_g2_split_parts():
    # a group's heads split over two parts: the hand-written table
    gold = json.load(open(GOLDEN_G2))
    N, G = gold["N"], gold["G"]
    for key, rows in gold["items_parts2"].items():
        name, mname = key.split("_")
        s, m = G2_KEYS[name], MASKS[mname]
        rk = sch.ranks(s, m, N, G)
        got = [[(g, i, j, rk[(g, i, j)]) for (g, i, j) in it] for it in sch.items(s, m, N, G, parts=2)]
        assert got == [_parse_item(r) for r in rows], key


@pytest.mark.parametrize("s,m,N", list(_combos((2, 4, 5))))
@pytest.mark.parametrize("G,parts", [(2, 2), (4, 2), (6, 3), (7, 7)])
def test_split_parts_cover_every_task_once(s, m, N, G, parts):
    its = sch.items(s, m, N, G, parts)
    assert len(its) == parts * len(sch.items(s, m, N, G))
    tasks = [t for it in its for t in it]
    assert sorted(tasks) == sorted(t for it in sch.items(s, m, N, G) for t in it)
    # each item serves the heads of one part only, and the parts come in order
    n_base = len(its) // parts
    for n, it in enumerate(its):
        k = n // n_base
        assert all(k * (G // parts) <= g < (k + 1) * (G // parts) for (g, _, _) in it)
