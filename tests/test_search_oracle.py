"""Pins of the oracle's task tables, deadlock check and schedule search
(oracle/search.py) against things fixed outside it: the hand-written golden
task lists (tests/golden/schedules_n4_g2.json), a closed-form critical path,
an independent replay of the kernels' hand-off program
(tests/test_reduction_protocol.py) on every table of tiny shapes, and an
exhaustive exploration of dispatch and interleavings on P workers.
"""

import itertools
import json
import os

import pytest

from oracle import dag
from oracle import schedule as sch
from oracle import search as se

from test_reduction_protocol import program

GOLDEN_G2 = os.path.join(os.path.dirname(__file__), "golden", "schedules_n4_g2.json")


def _golden_table(name):
    items = json.load(open(GOLDEN_G2))["items"][name]
    offs, tasks = [0], []
    for text in items:
        for tok in text.split():
            tasks.append(tuple(int(x) for x in tok.split(",")))
        offs.append(len(tasks))
    return offs, tasks


# (golden name, mask, kind, order, block) -- members of the family that are
# the closed forms (N = 4, G = 2)
MEMBERS = [
    ("shift_full", sch.FULL, se.SHIFT, 0, 4),
    ("shift_causal", sch.CAUSAL, se.SHIFT, 0, 4),
    ("symmetric_causal", sch.CAUSAL, se.SYMMETRIC, 0, 2),
    ("descending_full", sch.FULL, se.DESCENDING, 0, 4),
    ("descending_causal", sch.CAUSAL, se.DESCENDING, 0, 4),
    ("naive_full", sch.FULL, se.ASCENDING, 0, 1),
    ("naive_causal", sch.CAUSAL, se.SHIFT, 0, 1),
]


@pytest.mark.parametrize("name,mask,kind,order,block", MEMBERS)
def test_family_holds_the_golden_closed_forms(name, mask, kind, order, block):
    offs, tasks = se.family_table(mask, 4, 2, kind, order, block)
    g_offs, g_tasks = _golden_table(name)
    assert offs == g_offs
    assert tasks == g_tasks
    assert se.structure_ok(mask, 4, 2, offs, tasks)


@pytest.mark.parametrize("N,P,G,r", [(8, 1, 1, 0.0), (8, 2, 1, 0.25), (8, 4, 1, 0.25),
                                     (8, 8, 1, 0.5), (12, 4, 2, 0.125), (16, 4, 1, 0.1)])
def test_blocked_shift_critical_path(N, P, G, r):
    # blocks of P chains in lockstep, one block after another: every worker
    # runs G * N tasks per block back to back and no wait is exposed, so the
    # critical path is G * N * N / P * (c + r)
    offs, tasks = se.family_table(sch.FULL, N, G, se.SHIFT, 0, P)
    rep = se.simulate_table(sch.FULL, N, G, 1, P, offs, tasks, c=1.0, r=r)
    assert not rep["deadlock"]
    assert rep["makespan"] == pytest.approx(G * N * N / P * (1.0 + r))
    assert se.protocol_ok(sch.FULL, N, offs, tasks, 8, P) == (True, N // P, P)


def test_two_chain_cycle_needs_the_pipeline_model():
    # KV 0 reduces first into Q tile 0, KV 1 first into Q tile 1, and both
    # walk Q tile 0 then 1.  As a task DAG this is acyclic; but a unit
    # publishes the last pass of a task only after taking the turn of the next
    # task's first pass, so with two or more passes per task each unit waits
    # for the other: KV 0 cannot publish tile 0's last pass before KV 1 hands
    # over tile 1, which KV 1 reaches only after tile 0.
    offs = [0, 2, 4]
    tasks = [(0, 0, 0, 0), (0, 0, 1, 1), (0, 1, 0, 1), (0, 1, 1, 0)]
    assert se.structure_ok(sch.FULL, 2, 1, offs, tasks)
    rep = se.simulate_table(sch.FULL, 2, 1, 1, 2, offs, tasks)
    assert not rep["deadlock"]
    assert se.events_acyclic(offs, tasks, 1)
    assert not se.events_acyclic(offs, tasks, 2)
    assert se.protocol_ok(sch.FULL, 2, offs, tasks, 8, 2)[0] is False


@pytest.mark.parametrize("schedule,mask", [(sch.NAIVE, sch.FULL), (sch.NAIVE, sch.CAUSAL),
                                           (sch.DESCENDING_Q, sch.FULL), (sch.DESCENDING_Q, sch.CAUSAL),
                                           (sch.SHIFT, sch.FULL), (sch.SHIFT, sch.CAUSAL),
                                           (sch.SYMMETRIC_SHIFT, sch.CAUSAL)])
@pytest.mark.parametrize("N", [2, 4, 6])
@pytest.mark.parametrize("G", [1, 3])
@pytest.mark.parametrize("passes", [2, 4, 8])
def test_closed_forms_pass_when_a_group_fits(schedule, mask, N, G, passes):
    offs, tasks = se.closed_form_table(schedule, mask, N, G)
    assert se.structure_ok(mask, N, G, offs, tasks)
    items = len(offs) - 1
    ok, nb, widest = se.protocol_ok(mask, N, offs, tasks, passes, items)
    assert ok
    # the rigid ascending order waits only on earlier items: blocks of one
    if schedule in (sch.NAIVE, sch.DESCENDING_Q):
        assert widest == 1
        assert se.protocol_ok(mask, N, offs, tasks, passes, 1)[0]
    # the full-mask shift is one cyclic block: it needs every chain at once
    if schedule == sch.SHIFT and mask == sch.FULL:
        assert widest == N
        assert not se.protocol_ok(mask, N, offs, tasks, passes, N - 1)[0]


def _bad_tables():
    offs, tasks = se.closed_form_table(sch.SHIFT, sch.CAUSAL, 4, 2)
    out = []
    t = list(tasks)
    t[0] = (t[0][0], t[0][1], t[0][2], 1)           # duplicate rank
    out.append((offs, t))
    t = list(tasks)
    t[0], t[-1] = t[-1], t[0]                        # KV 3's run split from item 3
    out.append((offs, t))
    out.append(([0, 4, 4, len(tasks)], tasks))      # empty item
    t = list(tasks)
    t[1] = (t[1][0], t[1][1], t[1][2] - 1, t[1][3])  # a masked tile, a tile missing
    out.append((offs, t))
    t = list(tasks)
    t[2] = (5, t[2][1], t[2][2], t[2][3])            # head out of range
    out.append((offs, t))
    return out


@pytest.mark.parametrize("k", range(5))
def test_structure_rejects(k):
    offs, tasks = _bad_tables()[k]
    assert not se.structure_ok(sch.CAUSAL, 4, 2, offs, tasks)


# ---- every table of tiny shapes ---------------------------------------------

def _all_tables(mask, N):
    """Every valid table of one head: run orders, ranks, item cuts."""
    walks = [list(itertools.permutations([j for j in range(N) if sch.valid(mask, i, j)]))
             for i in range(N)]
    rank_choices = [list(itertools.permutations(sch.contributors(mask, N, j))) for j in range(N)]
    for walk in itertools.product(*walks):
        for orders in itertools.product(*rank_choices):
            rank = {}
            for j, order in enumerate(orders):
                for r, i in enumerate(order):
                    rank[(i, j)] = r
            for perm in itertools.permutations(range(N)):
                for cuts in itertools.product((0, 1), repeat=N - 1):
                    offs, tasks = [0], []
                    for pos, i in enumerate(perm):
                        tasks.extend((0, i, j, rank[(i, j)]) for j in walk[i])
                        if pos == N - 1 or cuts[pos]:
                            offs.append(len(tasks))
                    yield offs, tasks


def _programs(offs, tasks, passes, split=False):
    ranks = {(g, i, j): r for (g, i, j, r) in tasks}
    return [program([(g, i, j) for (g, i, j, _) in tasks[offs[k]:offs[k + 1]]], ranks, passes,
                    split=split)
            for k in range(len(offs) - 1)]


def _deadlock_reachable(progs, P):
    """Explores every order of steps and of dispatch (items taken in order by
    idle workers): True if some reachable state can make no step."""
    n = len(progs)
    start = (0, (), ())
    seen = {start}
    stack = [start]
    while stack:
        nxt, run, cnt = stack.pop()
        cd = dict(cnt)
        moves = []
        if len(run) < P and nxt < n:
            moves.append((nxt + 1, tuple(sorted(run + ((nxt, 0),))), cnt))
        for x, (k, pc) in enumerate(run):
            kind, (sl, rank) = progs[k][pc]
            if kind == "acquire" and cd.get(sl, 0) != rank:
                continue
            c2 = dict(cd)
            if kind == "release":
                c2[sl] = rank + 1
            rest = run[:x] + run[x + 1:]
            if pc + 1 < len(progs[k]):
                rest = tuple(sorted(rest + ((k, pc + 1),)))
            moves.append((nxt, rest, tuple(sorted(c2.items()))))
        if not moves:
            if nxt < n or run:
                return True
            continue
        for m in moves:
            if m not in seen:
                seen.add(m)
                stack.append(m)
    return False


def _complete_alone(progs):
    """One worker per item: replays until no step is possible (the outcome
    does not depend on the order: steps only ever enable others)."""
    cnt, pcs = {}, [0] * len(progs)
    moved = True
    while moved:
        moved = False
        for w, prog in enumerate(progs):
            while pcs[w] < len(prog):
                kind, (sl, rank) = prog[pcs[w]]
                if kind == "acquire" and cnt.get(sl, 0) != rank:
                    break
                if kind == "release":
                    cnt[sl] = rank + 1
                pcs[w] += 1
                moved = True
    return all(pc == len(p) for pc, p in zip(pcs, progs))


@pytest.mark.parametrize("mask,N", [(sch.FULL, 2), (sch.CAUSAL, 3)])
@pytest.mark.parametrize("passes", [1, 2, 3])
def test_event_graph_matches_the_replayed_program(mask, N, passes):
    # all items resident: the check's acyclic waits-for graph is exactly the
    # set of tables whose hand-off programs all run to completion
    n = agree = 0
    for offs, tasks in _all_tables(mask, N):
        progs = _programs(offs, tasks, passes)
        assert se.events_acyclic(offs, tasks, passes) == _complete_alone(progs)
        n += 1
        agree += _complete_alone(progs)
    assert n > 0 and 0 < agree < n


@pytest.mark.parametrize("mask,N,P", [(sch.FULL, 2, 1), (sch.CAUSAL, 3, 1), (sch.CAUSAL, 3, 2)])
def test_check_is_sound_on_fewer_workers(mask, N, P):
    # every table the check accepts on P workers finishes under every order
    # of dispatch and steps; the full-mask shift on one worker is refused and
    # can in fact deadlock
    passes = 2
    accepted = 0
    for offs, tasks in _all_tables(mask, N):
        if len(offs) - 1 <= P or not se.protocol_ok(mask, N, offs, tasks, passes, P)[0]:
            continue
        accepted += 1
        assert not _deadlock_reachable(_programs(offs, tasks, passes), P)
    assert accepted > 0
    offs, tasks = se.closed_form_table(sch.SHIFT, mask, N)
    if mask == sch.FULL:
        assert not se.protocol_ok(mask, N, offs, tasks, passes, P)[0]
        assert _deadlock_reachable(_programs(offs, tasks, passes), P)


# ---- the search -------------------------------------------------------------

@pytest.mark.parametrize("mask", [sch.FULL, sch.CAUSAL])
@pytest.mark.parametrize("N,G,groups,P", [(4, 1, 1, 4), (4, 2, 2, 2), (6, 1, 1, 3), (8, 1, 2, 8),
                                          (8, 2, 1, 3)])
def test_search_never_loses_to_a_closed_form(mask, N, G, groups, P):
    c, cd, r = 1.0, 0.5, 0.125
    offs, tasks, fam, rep = se.search(mask, N, G, groups, P, 8, c, cd, r)
    assert se.structure_ok(mask, N, G, offs, tasks)
    assert se.protocol_ok(mask, N, offs, tasks, 8, P)[0]
    for s in (sch.NAIVE, sch.DESCENDING_Q, sch.SHIFT, sch.SYMMETRIC_SHIFT):
        if s == sch.SYMMETRIC_SHIFT and (mask != sch.CAUSAL or N % 2):
            continue
        co, ct = se.closed_form_table(s, mask, N, G)
        if not se.protocol_ok(mask, N, co, ct, 8, P)[0]:
            continue
        cr = dag.simulate(s, mask, N, G=G, groups=groups, P=P, dispatch="dynamic", c=c,
                          c_diag=cd, r=r)
        assert rep["makespan"] <= cr["makespan"] + 1e-12


def test_search_reaches_more_chains_than_workers():
    # N = 16 chains on 4 workers: the shift family's closed form needs all 16
    # at once; the search runs the shift in blocks of 4 at the work bound
    N, P = 16, 4
    offs, tasks, fam, rep = se.search(sch.FULL, N, 1, 1, P, 8, 1.0, 1.0, 0.25)
    assert fam == (se.SHIFT, 0, P)
    assert rep["makespan"] == pytest.approx(N * N / P * 1.25)
    co, ct = se.closed_form_table(sch.SHIFT, sch.FULL, N)
    assert not se.protocol_ok(sch.FULL, N, co, ct, 8, P)[0]


# ---- per-head tables and the packed kind -------------------------------------

def _head_tables(mask, N, G, rng, n):
    """Seeded random tables whose runs are (head, KV tile) pairs: shuffled
    walks, ranks and run order, random item cuts."""
    out = []
    for _ in range(n):
        chains = []
        for g in range(G):
            for i in range(N):
                js = [j for j in range(N) if sch.valid(mask, i, j)]
                rng.shuffle(js)
                chains.append([(g, i, j) for j in js])
        rng.shuffle(chains)
        rank = {}
        for g in range(G):
            for j in range(N):
                cs = list(sch.contributors(mask, N, j))
                rng.shuffle(cs)
                for r, i in enumerate(cs):
                    rank[(g, i, j)] = r
        offs, tasks = [0], []
        for x, ch in enumerate(chains):
            tasks.extend(t + (rank[t],) for t in ch)
            if x == len(chains) - 1 or rng.random() < 0.4:
                offs.append(len(tasks))
        out.append((offs, tasks))
    return out


@pytest.mark.parametrize("mask,N", [(sch.FULL, 2), (sch.CAUSAL, 3), (sch.FULL, 3)])
@pytest.mark.parametrize("passes", [1, 2, 3])
def test_event_graph_matches_the_replayed_program_per_head(mask, N, passes):
    # per-head runs: the check's waits-for graph agrees with the replayed
    # hand-off programs whose runs end where the head or the tile changes
    import random
    rng = random.Random(1000 * N + passes)
    tables = _head_tables(mask, N, 2, rng, 300) + [se.packed_table(mask, N, 2, b) for b in (2, 3, 4)]
    heads = agree = 0
    for offs, tasks in tables:
        assert se.structure_ok(mask, N, 2, offs, tasks)
        split = se.table_form(offs, tasks) == "head"
        heads += split
        done = _complete_alone(_programs(offs, tasks, passes, split))
        assert se.events_acyclic(offs, tasks, passes, split) == done
        agree += done
    assert heads > 0 and 0 < agree < len(tables)


def test_check_is_sound_on_fewer_workers_per_head():
    import random
    rng = random.Random(7)
    passes, P, accepted = 2, 2, 0
    for offs, tasks in _head_tables(sch.FULL, 2, 2, rng, 200):
        if se.table_form(offs, tasks) != "head" or len(offs) - 1 <= P:
            continue
        if not se.protocol_ok(sch.FULL, 2, offs, tasks, passes, P)[0]:
            continue
        accepted += 1
        assert not _deadlock_reachable(_programs(offs, tasks, passes, True), P)
    assert accepted > 0


def test_a_split_head_run_is_neither_form():
    # head 0 of KV tile 0 in two pieces: not one run per tile, nor per head
    offs = [0, 1, 3, 4]
    tasks = [(0, 0, 0, 0), (0, 1, 0, 1), (0, 1, 1, 0), (0, 0, 1, 1)]
    assert se.table_form(offs, tasks) is None
    assert not se.structure_ok(sch.FULL, 2, 1, offs, tasks)


PACKED_CASES = [(m, N, G, b) for m in (sch.FULL, sch.CAUSAL)
                for (N, G, b) in ((1, 1, 1), (2, 3, 4), (4, 2, 3), (5, 3, 4), (8, 4, 6), (3, 2, 100),
                                  (16, 7, 16))]


@pytest.mark.parametrize("mask,N,G,bins", PACKED_CASES)
def test_packed_table(mask, N, G, bins):
    offs, tasks = se.packed_table(mask, N, G, bins)
    assert se.structure_ok(mask, N, G, offs, tasks)
    items = len(offs) - 1
    assert items == min(bins, G * N)
    # each (head, KV tile) is one run that walks its Q tiles from the
    # diagonal on, wrapping round under the full mask
    for k in range(items):
        chunk = tasks[offs[k]:offs[k + 1]]
        x = 0
        while x < len(chunk):
            g, i = chunk[x][0], chunk[x][1]
            js = [j for (gg, ii, j, _) in chunk if (gg, ii) == (g, i)]
            want = [(i + s) % N for s in range(N)] if mask == sch.FULL else list(range(i, N))
            assert js == want
            assert chunk[x:x + len(js)] == [t for t in chunk if (t[0], t[1]) == (g, i)]
            x += len(js)
    # greedy placement: the fullest item holds at most the mean of the rest
    # plus the longest walk
    loads = [offs[k + 1] - offs[k] for k in range(items)]
    longest = N
    total = len(tasks)
    assert max(loads) <= (total - longest) / items + longest
    # all items resident, equal task costs and no reduction cost: no wait
    # is exposed, every item ends at its own length
    rep = se.simulate_table(mask, N, G, 1, items, offs, tasks, 1.0, 1.0, 0.0)
    assert not rep["deadlock"]
    assert rep["makespan"] == max(loads)
    split = se.table_form(offs, tasks) == "head"
    for passes in (2, 4, 8):      # the kernels run 2 to 8 passes per task
        assert se.protocol_ok(mask, N, offs, tasks, passes, items)[0]
    if N <= 5:
        assert _complete_alone(_programs(offs, tasks, 2, split))


def test_search_packs_grouped_heads():
    # causal, seven heads per group: the packed kind spreads the G * N walks
    # over the grid share of each group and wins; kept out when per-head
    # tables cannot run
    m, N, G, groups, P = sch.CAUSAL, 8, 7, 2, 16
    offs, tasks, fam, rep = se.search(m, N, G, groups, P, 8, 1.0, 0.5, 0.125)
    assert fam == (se.PACKED, 0, se.packed_bins(N, G, groups, P))
    assert se.table_form(offs, tasks) == "head"
    offs2, tasks2, fam2, rep2 = se.search(m, N, G, groups, P, 8, 1.0, 0.5, 0.125, head_form_ok=False)
    assert fam2[0] != se.PACKED
    assert rep["makespan"] < rep2["makespan"]


GOLDEN_PACKED = os.path.join(os.path.dirname(__file__), "golden", "packed_tables.json")


def _golden_items(items):
    offs, tasks = [0], []
    for text in items:
        tasks.extend(tuple(int(x) for x in tok.split(",")) for tok in text.split())
        offs.append(len(tasks))
    return offs, tasks


@pytest.mark.parametrize("k", range(2))
def test_packed_kind_equals_the_hand_written_tables(k):
    case = json.load(open(GOLDEN_PACKED))["cases"][k]
    mask = sch.CAUSAL if case["mask"] == "causal" else sch.FULL
    offs, tasks = se.packed_table(mask, case["N"], case["G"], case["bins"])
    assert (offs, tasks) == _golden_items(case["items"])
    assert se.structure_ok(mask, case["N"], case["G"], offs, tasks)
