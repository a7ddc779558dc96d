"""The DASH backward DAG in plain Python (oracle; test infrastructure only).

DASH technical summary, section 2.1: nodes are compute phases (tile work) and
reduction phases; edges are data dependencies and the mandatory accumulation
order; the objective is the critical-path length; the work of one KV tile runs
as an unbroken chain on one unit.  Section 2.2 B states Lemma 1: adding a
zero-weight edge (u, v) keeps the critical path iff depth(u) <= depth(v).

The pages give no weights and no definition of depth.  Reading used here:

* every task has four events S (compute start), E (compute end), R (reduction
  start), F (reduction end), with edges S->E of weight c (c_diag for a causal
  diagonal tile), E->R of weight 0 and R->F of weight r;
* consecutive tasks of an item: F(prev) -> S(next), weight 0;
* consecutive items on one worker: F(last task) -> S(first task), weight 0;
* the accumulation order of a dQ tile: F(rank q) -> R(rank q+1), weight 0 --
  these are the zero-weight edges that Lemma 1 adds;
* depth(x) = longest weighted path from any source to x (the earliest time
  at which x can happen); critical path = largest depth.

Workers: ``static`` dispatch gives item k to worker k mod P; ``dynamic``
dispatch gives the next item to the first worker to become idle (ties to the
lower worker index), which needs the timed replay below to decide.

Two independent computations are provided so that tests can compare them:
``replay`` (event-driven, advances workers in time order) and ``build_dag`` +
``longest_path`` (explicit graph, topological order).
"""

import heapq

from . import schedule as sch


def group_items(schedule, mask, N, G, groups, item_lists=None):
    """All items of all groups, in global dispatch order: list of task lists.

    A task is (group, g, i, j).  item_lists, when given, are one group's items
    (lists of (g, i, j)) written out directly -- a schedule given as a table --
    and replace the closed form of `schedule`.
    """
    out = []
    base = sch.items(schedule, mask, N, G) if item_lists is None else item_lists
    for grp in range(groups):
        for it in base:
            out.append([(grp, g, i, j) for (g, i, j) in it])
    return out


def task_cost(mask, i, j, c, c_diag):
    return c_diag if (mask == sch.CAUSAL and i == j) else c


def replay(schedule, mask, N, G, groups, P, dispatch, c, c_diag, r, rank_map=None,
           item_lists=None):
    """Event-driven replay.  Returns dict with makespan, assignment, times,
    deadlock flag."""
    its = group_items(schedule, mask, N, G, groups, item_lists)
    rk = sch.ranks(schedule, mask, N, G) if rank_map is None else rank_map
    # F time of (group, g, j, rank) once known
    done = {}
    waiting = {}   # (group, g, j, rank) -> list of (worker, E, task)
    assign = {}
    times = {}
    state = {}     # worker -> [item index, position]; None = must take an item
    last = {}      # worker -> index of its last item (static dispatch)
    next_item = [0]
    heap = []      # (time, worker): the worker is free at that time

    def take_item(w):
        if dispatch == "static":
            k = last[w] + P if w in last else w
        else:
            k = next_item[0]
            next_item[0] += 1
        if k >= len(its):
            return False
        last[w] = k
        state[w] = [k, 0]
        assign[k] = w
        return True

    def finish_task(w, task, E, Rt):
        F = Rt + r
        grp, g, i, j = task
        times[task] = (E - task_cost(mask, i, j, c, c_diag), E, Rt, F)
        done[(grp, g, j, rk[(g, i, j)])] = F
        st = state[w]
        st[1] += 1
        if st[1] >= len(its[st[0]]):
            state[w] = None
        # the worker is free again at F (a new item is taken when that
        # event is popped, so items are handed out in time order)
        heapq.heappush(heap, (F, w))
        for (w2, E2, task2) in waiting.pop((grp, g, j, rk[(g, i, j)]), []):
            finish_task(w2, task2, E2, max(E2, F))

    for w in range(P):
        state[w] = None
        heapq.heappush(heap, (0.0, w))
    while heap:
        t, w = heapq.heappop(heap)
        if state[w] is None and not take_item(w):
            continue
        k, pos = state[w]
        task = its[k][pos]
        grp, g, i, j = task
        E = t + task_cost(mask, i, j, c, c_diag)
        q = rk[(g, i, j)]
        if q == 0:
            finish_task(w, task, E, E)
        elif (grp, g, j, q - 1) in done:
            finish_task(w, task, E, max(E, done[(grp, g, j, q - 1)]))
        else:
            waiting.setdefault((grp, g, j, q - 1), []).append((w, E, task))
    ntasks = sum(len(it) for it in its)
    deadlock = len(times) != ntasks
    makespan = max((v[3] for v in times.values()), default=0.0)
    return {"makespan": makespan, "assign": assign, "times": times,
            "deadlock": deadlock}


def build_dag(schedule, mask, N, G, groups, P, assign, c, c_diag, r, rank_map=None,
              item_lists=None):
    """Explicit event graph.  Returns (nodes, base_edges, order_edges) where an
    edge is (u, v, weight) and a node is (task, kind)."""
    its = group_items(schedule, mask, N, G, groups, item_lists)
    rk = sch.ranks(schedule, mask, N, G) if rank_map is None else rank_map
    nodes = []
    base = []
    order = []
    for it in its:
        for task in it:
            grp, g, i, j = task
            for kind in "SERF":
                nodes.append((task, kind))
            base.append(((task, "S"), (task, "E"), task_cost(mask, i, j, c, c_diag)))
            base.append(((task, "E"), (task, "R"), 0.0))
            base.append(((task, "R"), (task, "F"), r))
        for a, b in zip(it, it[1:]):
            base.append(((a, "F"), (b, "S"), 0.0))
    per_worker = {}
    for k in sorted(assign):
        per_worker.setdefault(assign[k], []).append(k)
    for w, ks in per_worker.items():
        for a, b in zip(ks, ks[1:]):
            base.append(((its[a][-1], "F"), (its[b][0], "S"), 0.0))
    by_tile = {}
    for it in its:
        for task in it:
            grp, g, i, j = task
            by_tile.setdefault((grp, g, j), {})[rk[(g, i, j)]] = task
    for key, d in by_tile.items():
        for q in range(1, len(d)):
            order.append(((d[q - 1], "F"), (d[q], "R"), 0.0))
    return nodes, base, order


def longest_path(nodes, edges):
    """Depth of every node (longest path from a source); None on a cycle."""
    succ = {n: [] for n in nodes}
    indeg = {n: 0 for n in nodes}
    for u, v, w in edges:
        succ[u].append((v, w))
        indeg[v] += 1
    depth = {n: 0.0 for n in nodes}
    ready = [n for n in nodes if indeg[n] == 0]
    seen = 0
    while ready:
        u = ready.pop()
        seen += 1
        for v, w in succ[u]:
            if depth[u] + w > depth[v]:
                depth[v] = depth[u] + w
            indeg[v] -= 1
            if indeg[v] == 0:
                ready.append(v)
    if seen != len(nodes):
        return None
    return depth


def simulate(schedule, mask, N, G=1, groups=1, P=None, dispatch="static",
             c=1.0, c_diag=None, r=0.0, rank_map=None, item_lists=None):
    """Replay, DAG, Lemma-1 check.  Returns a dict like the library's report.
    A schedule given as a table passes item_lists and rank_map (schedule is
    then ignored)."""
    if c_diag is None:
        c_diag = c
    its = group_items(schedule, mask, N, G, groups, item_lists)
    n_items = len(its)
    if P is None:
        P = n_items
    rep = replay(schedule, mask, N, G, groups, P, dispatch, c, c_diag, r, rank_map, item_lists)
    total = sum(task_cost(mask, i, j, c, c_diag) + r
                for it in its for (_, _, i, j) in it)
    res = {"total_work": total, "deadlock": bool(rep["deadlock"]),
           "replay_makespan": rep["makespan"]}
    if rep["deadlock"]:
        # The assignment is incomplete; report the cycle test on the static
        # assignment instead.
        assign = {k: k % P for k in range(len(its))}
    else:
        assign = rep["assign"]
    nodes, base, order = build_dag(schedule, mask, N, G, groups, P, assign,
                                   c, c_diag, r, rank_map, item_lists)
    d_base = longest_path(nodes, base)
    d_full = longest_path(nodes, base + order)
    res["order_edges"] = len(order)
    if d_full is None:
        res["deadlock"] = True
        res["makespan"] = float("inf")
    else:
        res["makespan"] = max(d_full.values()) if d_full else 0.0
    viol = 0
    worst = 0.0
    for u, v, _ in order:
        deficit = d_base[u] - d_base[v]
        if deficit > 0:
            viol += 1
            worst = max(worst, deficit)
    res["violations"] = viol
    res["max_deficit"] = worst
    res["base_makespan"] = max(d_base.values()) if d_base else 0.0
    used = min(P, n_items) if n_items else 1
    res["efficiency"] = (total / (used * res["makespan"])
                         if res["makespan"] not in (0.0, float("inf")) else 0.0)
    return res


# Candidates of the schedule selection, in the order that breaks ties (the
# first one wins on an equal critical path).
SELECT_ORDER = (sch.SYMMETRIC_SHIFT, sch.SHIFT, sch.DESCENDING_Q, sch.NAIVE)


def select(mask, N, G=1, groups=1, P=None, dispatch="static", c=1.0, c_diag=None, r=0.0):
    """The deterministic schedule with the shortest critical path for this
    shape and worker count (DASH technical summary, section 2: the schedule
    is chosen to minimise the DAG's critical path; the pages leave the choice
    per shape and hardware to the practitioner).  Schedules that deadlock on P
    workers, or do not apply to the mask and tile count, are skipped.
    Returns (schedule, simulate() result)."""
    best = None
    for s in SELECT_ORDER:
        if s == sch.SYMMETRIC_SHIFT and (mask != sch.CAUSAL or N % 2):
            continue
        res = simulate(s, mask, N, G=G, groups=groups, P=P, dispatch=dispatch,
                       c=c, c_diag=c_diag, r=r)
        if res["deadlock"]:
            continue
        if best is None or res["makespan"] < best[1]["makespan"]:
            best = (s, res)
    return best
