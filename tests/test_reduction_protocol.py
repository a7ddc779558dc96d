"""Deadlock freedom of the backward kernel's ordered-reduction pipeline (host model).

The persistent kernel reduces the dQ slice of pass x in three stages: during
pass x+1 it waits for the slice's turn and loads the partial sum; during pass
x+2 it adds and stores; during pass x+3 it publishes rank + 1 on the slice's
counter (right after the pass's opening barrier, or after its S/dP products
when a task has four or more passes) -- in both cases before that pass's own
turn wait, which is the order the model below replays.  The last pass of a key/value tile's run
stores the pending slices, publishes them, and only then waits for its own
turn.  This test replays that order of operations for every item of every
schedule (one worker per item, as the shift family requires) and checks that
all of them finish; the counters' semantics (a wait blocks until the counter
equals the rank, a release sets it to rank + 1) make the outcome independent
of how the workers interleave.  It also checks that holding the pending
slices across the last pass's wait -- the order the kernel must not use --
is caught as a deadlock.
"""

import pytest

from oracle import schedule as sch


def program(tasks, ranks, NP, release_before_wait=True, split=False):
    # split: runs end where the head or the KV tile changes (per-head tables),
    # else only where the KV tile changes
    ops = []
    prev = fin = rel = None
    key = (lambda t: (t[0], t[1])) if split else (lambda t: t[1])
    for k, (g, i, j) in enumerate(tasks):
        seg_begin = k == 0 or key(tasks[k - 1]) != key(tasks[k])
        seg_end = k == len(tasks) - 1 or key(tasks[k + 1]) != key(tasks[k])
        if seg_begin:
            prev = fin = None
        for hp in range(NP):
            cur = ((g, j, hp), ranks[(g, i, j)])
            if rel is not None:          # after the barrier that opens the pass
                ops.append(("release", rel))
                rel = None
            if prev is not None and prev[1] > 0:
                ops.append(("acquire", prev))
            stored, fin = fin, prev      # fin stored in this pass; prev loaded
            if hp == NP - 1 and seg_end:
                held = [x for x in (stored, fin) if x is not None]
                if release_before_wait:
                    ops += [("release", x) for x in held]
                if cur[1] > 0:
                    ops.append(("acquire", cur))
                if not release_before_wait:
                    ops += [("release", x) for x in held]
                ops.append(("release", cur))
                prev = fin = None
            else:
                rel, prev = stored, cur
    return ops


def completes(schedule, mask, N, G, NP, release_before_wait=True):
    ranks = sch.ranks(schedule, mask, N, G)
    progs = [program(it, ranks, NP, release_before_wait)
             for it in sch.items(schedule, mask, N, G)]
    cnt, pcs = {}, [0] * len(progs)
    while True:
        moved = False
        for w, prog in enumerate(progs):
            while pcs[w] < len(prog):
                kind, (sl, rank) = prog[pcs[w]]
                if kind == "acquire" and cnt.get(sl, 0) != rank:
                    break
                if kind == "release":
                    assert cnt.get(sl, 0) == rank
                    cnt[sl] = rank + 1
                pcs[w] += 1
                moved = True
        if all(pc == len(p) for pc, p in zip(pcs, progs)):
            return True
        if not moved:
            return False


CASES = [(s, m) for s in (sch.NAIVE, sch.DESCENDING_Q, sch.SHIFT) for m in (sch.FULL, sch.CAUSAL)]
CASES.append((sch.SYMMETRIC_SHIFT, sch.CAUSAL))


@pytest.mark.parametrize("s,m", CASES)
@pytest.mark.parametrize("N", [2, 3, 4, 6, 8])
@pytest.mark.parametrize("G", [1, 2, 3])
@pytest.mark.parametrize("NP", [2, 4])
def test_pipeline_completes(s, m, N, G, NP):
    if s == sch.SYMMETRIC_SHIFT and N % 2:
        return
    assert completes(s, m, N, G, NP)


def test_holding_pending_slices_across_the_wait_deadlocks():
    # every chain of the full-mask shift reaches its last pass together
    assert not completes(sch.SHIFT, sch.FULL, 4, 1, 2, release_before_wait=False)
