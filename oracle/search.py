"""Task tables and the schedule search, in plain Python (oracle).

TEST INFRASTRUCTURE ONLY: tests import this to check the library's host-side
table checks and search; no product code uses it.

What this follows.  The DASH technical summary frames the choice of schedule
as minimising the critical path of the backward DAG (section 2.1), under the
constraint that the work of one key/value tile is an unbroken chain on one
unit, and leaves the choice per shape and hardware to the practitioner
(section 2; section 5 on the trade-offs).  The pages give no search
procedure.  The reading used here (a family of block-wise lockstep walks that
holds the closed forms of section 2.2 as members):

* units: the chains of KV tiles 0..N-1, or (SYMMETRIC kind: causal, N even)
  the pairs p = 0..N/2-1 of section 2.2 B, in ascending or descending order;
* a unit's walk over its Q tiles for one head: SHIFT -- the cyclic walk from
  the diagonal (full) or the walk upward from the diagonal (causal);
  DESCENDING -- from the last Q tile down; ASCENDING -- from Q tile 0 up (full
  masks; on causal masks it is the SHIFT walk); SYMMETRIC -- the three parts of
  schedule.symmetric_pair_parts;
* G heads: every step of the walk is taken for all heads in turn;
* the units are cut into dispatch blocks of `block` consecutive units, and dQ
  tile (g, j) is reduced in the order of (block, step at which the unit
  reaches j, unit position): lockstep arrival inside a block, and the blocks
  one after another;
* candidates: every kind that applies, ascending then descending unit order,
  blocks of min(units, P), half that and 1; the shortest simulated critical
  path (oracle.dag, dynamic dispatch) wins, ties to the earlier candidate.

A fifth kind, PACKED, drops the lockstep walk for load balance: each
(head, KV tile) is a chain of its own (walk as SHIFT), chains go longest first
to the least loaded of `bins` bins (lowest bin on ties; bins = the workgroups
one group gets, min(G*N, P // groups)), the non-empty bins in order are the
items, and dQ tile (g, j) is reduced in the order (position of the task in its
item, item).  With G > 1 the chains of one KV tile then sit in different
items: a table in the per-head form, where each (head, KV tile)'s tasks are
one run (its dK/dV leave the unit as that head's partial); tables whose KV
tiles each form one run are in the whole-tile form, taken when both hold.

Deadlock freedom.  A table is run by persistent workgroups that take items in
order and keep them; a dQ hand-off waits for the previous rank.  The kernels
pipeline each hand-off: within a key/value tile's run, in pass m the turn of
pass m-1 is taken (at the end of the pass) and the slice of pass m-3 is
published (before that); after the run's last pass L the slices L-2 and L-1
are published, then the turn of L is taken and L published.  The check used:
the waits-for graph of those events has no cycle, and the items split into
consecutive dispatch blocks of at most P items with no item waiting on a
later block (then the earliest unfinished block can always progress).

Tables are (offs, tasks): item k is tasks[offs[k]:offs[k+1]], a task is
(g, i, j, rank).
"""

from . import dag
from . import schedule as sch

SYMMETRIC, SHIFT, DESCENDING, ASCENDING, PACKED = 0, 1, 2, 3, 4


def tiles(mask, N):
    return N * (N + 1) // 2 if mask == sch.CAUSAL else N * N


def closed_form_table(schedule, mask, N, G=1):
    """A closed-form schedule of oracle.schedule written as a table."""
    rk = sch.ranks(schedule, mask, N, G)
    offs, tasks = [0], []
    for it in sch.items(schedule, mask, N, G):
        tasks.extend((g, i, j, rk[(g, i, j)]) for (g, i, j) in it)
        offs.append(len(tasks))
    return offs, tasks


def run_key(task, split):
    g, i = task[0], task[1]
    return (g, i) if split else i


def one_run_each(offs, tasks, split):
    """Whether every run key occurs in one unbroken stretch of one item."""
    seen = set()
    for k in range(len(offs) - 1):
        prev = None
        for t in tasks[offs[k]:offs[k + 1]]:
            key = run_key(t, split)
            if key != prev:
                if key in seen:
                    return False
                seen.add(key)
                prev = key
    return True


def table_form(offs, tasks):
    """'tile' (each KV tile one run), else 'head' (each (head, KV tile) one
    run), else None."""
    if one_run_each(offs, tasks, False):
        return "tile"
    if one_run_each(offs, tasks, True):
        return "head"
    return None


def structure_ok(mask, N, G, offs, tasks):
    """Every unmasked (g, i, j) exactly once; ranks of each dQ tile a
    permutation; each KV tile's tasks one contiguous run inside one item, or
    each (head, KV tile)'s tasks."""
    items = len(offs) - 1
    if items < 1 or items > G * N or offs[0] != 0 or offs[-1] != len(tasks):
        return False
    if any(offs[k + 1] <= offs[k] for k in range(items)):
        return False
    want = {(g, i, j) for g in range(G) for j in range(N) for i in sch.contributors(mask, N, j)}
    got = [(g, i, j) for (g, i, j, _) in tasks]
    if len(got) != len(set(got)) or set(got) != want:
        return False
    for g in range(G):
        for j in range(N):
            rs = sorted(r for (gg, _, jj, r) in tasks if gg == g and jj == j)
            if rs != list(range(len(sch.contributors(mask, N, j)))):
                return False
    return table_form(offs, tasks) is not None


def runs(offs, tasks, split=False):
    """[(item, first task index, last task index)] of every run."""
    out = []
    for k in range(len(offs) - 1):
        t = offs[k]
        while t < offs[k + 1]:
            u = t
            while u + 1 < offs[k + 1] and run_key(tasks[u + 1], split) == run_key(tasks[t], split):
                u += 1
            out.append((k, t, u))
            t = u + 1
    return out


def run_events(first, last, passes):
    """The kernel's hand-off events of one run, in program order: ("A", t, p)
    takes the turn of pass p of task t, ("R", t, p) publishes it."""
    L = (last - first + 1) * passes - 1

    def at(m):
        return first + m // passes, m % passes

    ev = []
    for m in range(1, L + 1):
        if m >= 3:
            ev.append(("R",) + at(m - 3))
        ev.append(("A",) + at(m - 1))
    if L >= 2:
        ev.append(("R",) + at(L - 2))
    if L >= 1:
        ev.append(("R",) + at(L - 1))
    ev.append(("A",) + at(L))
    ev.append(("R",) + at(L))
    return ev


def predecessors(offs, tasks):
    """Task index of the previous rank in each task's dQ tile (None for 0)."""
    by = {(g, j, r): t for t, (g, _, j, r) in enumerate(tasks)}
    return [by[(g, j, r - 1)] if r > 0 else None for (g, _, j, r) in tasks]


def dispatch_blocks(offs, tasks):
    """Sizes of the consecutive dispatch blocks: the smallest cut in which no
    item waits on an item of a later block."""
    owner = {}
    for k in range(len(offs) - 1):
        for t in range(offs[k], offs[k + 1]):
            owner[t] = k
    pred = predecessors(offs, tasks)
    sizes, start, end = [], 0, 0
    for k in range(len(offs) - 1):
        reach = max([k] + [owner[pred[t]] for t in range(offs[k], offs[k + 1]) if pred[t] is not None])
        end = max(end, reach)
        if k == end:
            sizes.append(k - start + 1)
            start = k + 1
    return sizes


def events_acyclic(offs, tasks, passes, split=False):
    """Whether the waits-for graph of the hand-off events has no cycle."""
    succ = {}
    indeg = {}

    def node(x):
        succ.setdefault(x, [])
        indeg.setdefault(x, 0)

    def edge(u, v):
        node(u)
        node(v)
        succ[u].append(v)
        indeg[v] += 1

    for k in range(len(offs) - 1):
        prev_last = None
        for (kk, a, b) in runs(offs, tasks, split):
            if kk != k:
                continue
            ev = run_events(a, b, passes)
            for x in ev:
                node(x)
            if prev_last is not None:
                edge(prev_last, ev[0])
            for u, v in zip(ev, ev[1:]):
                edge(u, v)
            prev_last = ev[-1]
    for t, pr in enumerate(predecessors(offs, tasks)):
        if pr is not None:
            for p in range(passes):
                edge(("R", pr, p), ("A", t, p))
    ready = [x for x in indeg if indeg[x] == 0]
    seen = 0
    while ready:
        u = ready.pop()
        seen += 1
        for v in succ[u]:
            indeg[v] -= 1
            if indeg[v] == 0:
                ready.append(v)
    return seen == len(indeg)


def protocol_ok(mask, N, offs, tasks, passes, P):
    """(ok, number of dispatch blocks, widest block) on P workgroups."""
    sizes = dispatch_blocks(offs, tasks)
    split = table_form(offs, tasks) == "head"
    ok = max(sizes) <= P and events_acyclic(offs, tasks, passes, split)
    return ok, len(sizes), max(sizes)


def unit_walk(mask, N, kind, u):
    """(i, j) per step of unit u's walk for one head."""
    if kind == SYMMETRIC:
        ph1, ph2a, ph2b = sch.symmetric_pair_parts(N, u)
        return ph1 + ph2a + ph2b
    if kind == SHIFT:
        js = [(u + s) % N for s in range(N)] if mask == sch.FULL else list(range(u, N))
    elif kind == DESCENDING:
        js = list(range(N - 1, -1, -1))
    else:
        js = list(range(N))
    return [(u, j) for j in js if sch.valid(mask, u, j)]


def family_applies(mask, N, kind):
    if kind == SYMMETRIC:
        return mask == sch.CAUSAL and N % 2 == 0
    if kind == ASCENDING:
        return mask == sch.FULL
    return kind in (SHIFT, DESCENDING, PACKED)


def packed_bins(N, G, groups, P):
    return max(1, min(G * N, P // groups))


def packed_table(mask, N, G, bins):
    """The PACKED kind (module docstring) with `bins` bins."""
    chains = []
    for g in range(G):
        for i in range(N):
            walk = [j for (_, j) in unit_walk(mask, N, SHIFT, i)]
            chains.append((-len(walk), g, i, walk))
    chains.sort(key=lambda c: c[:3])
    loads = [0] * bins
    content = [[] for _ in range(bins)]
    for (neg, g, i, walk) in chains:
        b = min(range(bins), key=lambda x: (loads[x], x))
        content[b].append((g, i, walk))
        loads[b] -= neg
    item_tasks = []
    for b in range(bins):
        if content[b]:
            item_tasks.append([(g, i, j) for (g, i, walk) in content[b] for j in walk])
    order = {}
    for k, lst in enumerate(item_tasks):
        for pos, (g, i, j) in enumerate(lst):
            order.setdefault((g, j), []).append((pos, k, i))
    rank = {}
    for (g, j), lst in order.items():
        for r, (_, _, i) in enumerate(sorted(lst)):
            rank[(g, i, j)] = r
    offs, tasks = [0], []
    for lst in item_tasks:
        tasks.extend((g, i, j, rank[(g, i, j)]) for (g, i, j) in lst)
        offs.append(len(tasks))
    return offs, tasks


def family_table(mask, N, G, kind, order, block):
    if kind == PACKED:
        return packed_table(mask, N, G, block)
    units = N // 2 if kind == SYMMETRIC else N
    seq = list(range(units)) if order == 0 else list(range(units - 1, -1, -1))
    walks = [unit_walk(mask, N, kind, u) for u in seq]
    keys = {}   # j -> [(block, step, position)]
    for pos, w in enumerate(walks):
        for s, (i, j) in enumerate(w):
            keys.setdefault(j, []).append((pos // block, s, pos))
    rank = {}
    for j, lst in keys.items():
        for r, (_, s, pos) in enumerate(sorted(lst)):
            rank[(pos, s)] = r
    offs, tasks = [0], []
    for pos, w in enumerate(walks):
        for s, (i, j) in enumerate(w):
            for g in range(G):
                tasks.append((g, i, j, rank[(pos, s)]))
        offs.append(len(tasks))
    return offs, tasks


def family_blocks(units, P):
    m = min(units, P)
    out = [m]
    if m // 2 >= 1 and m // 2 != m:
        out.append(m // 2)
    if out[-1] != 1:
        out.append(1)
    return out


def simulate_table(mask, N, G, groups, P, offs, tasks, c=1.0, c_diag=None, r=0.0,
                   dispatch="dynamic"):
    item_lists = [[(g, i, j) for (g, i, j, _) in tasks[offs[k]:offs[k + 1]]]
                  for k in range(len(offs) - 1)]
    rank_map = {(g, i, j): rk for (g, i, j, rk) in tasks}
    return dag.simulate(None, mask, N, G=G, groups=groups, P=P, dispatch=dispatch, c=c,
                        c_diag=c_diag, r=r, rank_map=rank_map, item_lists=item_lists)


def search(mask, N, G, groups, P, passes, c=1.0, c_diag=None, r=0.0, head_form_ok=True):
    """(offs, tasks, (kind, order, block), report) of the best candidate.
    head_form_ok: whether tables in the per-head form can run (the kernels
    of 256-key tiles); without it PACKED is tried only for G = 1."""
    best = None
    for kind in (SYMMETRIC, SHIFT, DESCENDING, ASCENDING, PACKED):
        if not family_applies(mask, N, kind):
            continue
        if kind == PACKED and G > 1 and not head_form_ok:
            continue
        units = N // 2 if kind == SYMMETRIC else N
        orders = (0,) if kind == PACKED else (0, 1)
        blocks = [packed_bins(N, G, groups, P)] if kind == PACKED else family_blocks(units, P)
        for order in orders:
            for b in blocks:
                offs, tasks = family_table(mask, N, G, kind, order, b)
                if not protocol_ok(mask, N, offs, tasks, passes, P)[0]:
                    continue
                rep = simulate_table(mask, N, G, groups, P, offs, tasks, c, c_diag, r)
                if rep["deadlock"]:
                    continue
                if best is None or rep["makespan"] < best[3]["makespan"]:
                    best = (offs, tasks, (kind, order, b), rep)
    return best
