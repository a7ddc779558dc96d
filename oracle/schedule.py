"""Tile schedules of the deterministic backward, as explicit task lists (oracle).

TEST INFRASTRUCTURE ONLY.

Vocabulary.  The key/value sequence is cut into N tiles (index i) and the query
sequence into N tiles (index j).  A *task* (i, j) is the work of KV tile i
against Q tile j; with a causal mask only j >= i exists.  The work of one KV
tile runs contiguously on one compute unit so that its dK/dV stay in
registers (DASH technical summary, section 2.1, constraints): that ordered
list is a *chain*.  The dQ tile j receives one reduction from each KV tile
that meets it, and the order of those reductions is fixed: the *rank* of KV
tile i in dQ tile j is its position in that order.

Schedules (DASH technical summary, section 2.2):

* NAIVE -- the baseline the pages improve on: each chain walks its Q tiles
  upward and dQ tiles are reduced in the rigid ascending-KV order
  (section 1, the predetermined accumulation order).
* DESCENDING_Q -- the same chains walk their Q tiles from the last one down
  to the first (section 2.2 A); the reduction order is unchanged.
* SHIFT -- full mask: the unit working on KV tile i visits Q tiles
  i, i+1, ..., N-1, 0, ..., i-1 (section 2.2 B).  The page words the cycle as
  one over KV blocks; since a KV tile's work must stay on one unit (section
  2.1) the cycle is read as running over the Q tiles of chain i.  The
  reduction order of each dQ tile is the order in which the chains reach it
  when all chains advance in lockstep, which the page describes as an order
  that arises by itself with no two chains meeting one dQ tile at once.
  With a causal mask the same cycle is used with the masked tiles left out.
* SYMMETRIC_SHIFT -- causal mask, N even: one unit takes the KV tiles p and
  N-1-p (section 2.2 B, symmetric shift), which together have N+1 tasks.
  Phase 1 is the dense block {KV < N/2} x {Q >= N/2}, walked as a cyclic
  shift; phase 2 is the remaining two triangles, folded so that pair p first
  takes Q tiles p..N/2-1 of KV p and then Q tiles N-1 down to N-1-p of KV
  N-1-p.  Reduction order = lockstep arrival order.
* ATOMIC -- the non-deterministic counterpart (section 1: unordered atomic
  adds into dQ).  The pages give it no order, and its result does not depend
  on one.  Reading used here: it takes the best-balanced items for the mask,
  the symmetric pairs on causal masks with an even tile count and one chain
  per KV tile otherwise, so that a comparison with the ordered schedules
  isolates the reduction; its ranks are listed in ascending KV order.

Grouped-query attention: Hq/Hkv = G query heads read one KV head.  One item
serves one KV tile (or pair) for all G query heads so that dK/dV stay
resident across the group; the task list of an item takes every step of the
single-head list for all G heads in turn (step outer, head inner), part by
part for the symmetric shift (phase 1, the KV-p part of phase 2, the
KV-(N-1-p) part).  Ranks are defined per (query head, dQ tile).

Everything here is deliberately naive: task lists are materialised, and the
arrival ranks are obtained by sorting the contributors of each dQ tile by the
lockstep step at which they reach it.
"""

NAIVE = 0
DESCENDING_Q = 1
SHIFT = 2
SYMMETRIC_SHIFT = 3
ATOMIC = 4

FULL = 0
CAUSAL = 1

SCHEDULE_NAMES = {NAIVE: "naive", DESCENDING_Q: "descending_q", SHIFT: "shift",
                  SYMMETRIC_SHIFT: "symmetric_shift", ATOMIC: "atomic"}


def valid(mask, i, j):
    """Whether KV tile i and Q tile j meet (causal: keys not after queries)."""
    return True if mask == FULL else j >= i


def contributors(mask, N, j):
    """KV tiles that reduce into dQ tile j, ascending."""
    return [i for i in range(N) if valid(mask, i, j)]


def chain_q_order(schedule, mask, N, i):
    """Q tiles visited by the chain of KV tile i, in visiting order."""
    if schedule in (NAIVE, ATOMIC):
        seq = list(range(N))
    elif schedule == DESCENDING_Q:
        seq = list(range(N - 1, -1, -1))
    elif schedule == SHIFT:
        seq = [(i + t) % N for t in range(N)]
    else:
        raise ValueError("not a chain schedule")
    return [j for j in seq if valid(mask, i, j)]


def symmetric_pair_parts(N, p):
    """The three parts of symmetric pair p for one head, as (i, j) lists.

    phase 1: KV p against Q tiles N/2 .. N-1, cyclically from N/2 + p;
    phase 2a: KV p against Q tiles p .. N/2-1 (ascending);
    phase 2b: KV N-1-p against Q tiles N-1 .. N-1-p (descending).
    """
    if N % 2:
        raise ValueError("symmetric shift needs an even tile count")
    h = N // 2
    ph1 = [(p, h + (p + t) % h) for t in range(h)]
    ph2a = [(p, j) for j in range(p, h)]
    ph2b = [(N - 1 - p, j) for j in range(N - 1, N - 2 - p, -1)]
    return ph1, ph2a, ph2b


def items(schedule, mask, N, G=1, parts=1):
    """Items of one (batch, KV head) group, in dispatch order.

    Each item is a list of tasks (g, i, j): query head g of the group, KV
    tile i, Q tile j.  With parts > 1 (a divisor of G) the query heads are
    split into `parts` consecutive runs of G / parts heads, and each part has
    its own copy of every item, serving only its heads; the parts follow one
    another in dispatch order (part 0's items first).  dK/dV of a key/value
    tile are then the sum of the parts' sums, added in ascending part order.
    """
    if parts != 1:
        if parts < 1 or G % parts:
            raise ValueError("parts must divide G")
        Gp = G // parts
        return [[(k * Gp + g, i, j) for (g, i, j) in it]
                for k in range(parts) for it in items(schedule, mask, N, Gp)]
    out = []
    # the atomic reference's result does not depend on its order; on causal
    # masks with an even tile count it takes the symmetric pairs (the
    # best-balanced items), else one chain per KV tile
    paired = schedule == SYMMETRIC_SHIFT or (schedule == ATOMIC and mask == CAUSAL and N % 2 == 0)
    if paired:
        if mask != CAUSAL:
            raise ValueError("symmetric shift is defined for causal masks")
        for p in range(N // 2):
            ph1, ph2a, ph2b = symmetric_pair_parts(N, p)
            it = []
            for part in (ph1, ph2a, ph2b):
                for (i, j) in part:
                    it.extend((g, i, j) for g in range(G))
            out.append(it)
        return out
    for i in range(N):
        js = chain_q_order(schedule, mask, N, i)
        out.append([(g, i, j) for j in js for g in range(G)])
    return out


def lockstep_steps(schedule, mask, N, G=1):
    """{(g, j): [(step, i), ...]} when all items of a group start together."""
    arrivals = {}
    for it in items(schedule, mask, N, G):
        for step, (g, i, j) in enumerate(it):
            arrivals.setdefault((g, j), []).append((step, i))
    return arrivals


def ranks(schedule, mask, N, G=1):
    """{(g, i, j): rank} -- the fixed reduction order of every dQ tile.

    NAIVE / DESCENDING_Q: ascending KV index (the rigid order).
    SHIFT / SYMMETRIC_SHIFT: lockstep arrival order; a tie (two chains at
    one dQ tile in the same step) raises, since the schedule is meant to be
    conflict free.
    """
    out = {}
    if schedule in (NAIVE, DESCENDING_Q, ATOMIC):
        for g in range(G):
            for j in range(N):
                for r, i in enumerate(contributors(mask, N, j)):
                    out[(g, i, j)] = r
        return out
    for (g, j), lst in lockstep_steps(schedule, mask, N, G).items():
        lst = sorted(lst)
        steps = [s for s, _ in lst]
        if len(set(steps)) != len(steps):
            raise ValueError("lockstep conflict at dQ tile (%d, %d)" % (g, j))
        for r, (_, i) in enumerate(lst):
            out[(g, i, j)] = r
    return out


def dispatch_order_ok(schedule, mask, N, G=1):
    """Every wait of an item targets an item at or before it in dispatch order,
    or the whole group must be resident at once (returned as False)."""
    rk = ranks(schedule, mask, N, G)
    owner = {}
    for n, it in enumerate(items(schedule, mask, N, G)):
        for (g, i, j) in it:
            owner[(g, i, j)] = n
    by_tile = {}
    for (g, i, j), r in rk.items():
        by_tile.setdefault((g, j), {})[r] = (g, i, j)
    for (g, j), d in by_tile.items():
        for r in range(1, len(d)):
            if owner[d[r - 1]] > owner[d[r]]:
                return False
    return True
