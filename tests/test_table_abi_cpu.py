"""Host-side tests of the task-table part of libdash_attn.so (no GPU needed):
the library's closed-form tables, table checks, table simulation and
schedule search against the oracle (oracle/search.py), the packed device
form, and the argument checks of dash_attn_bwd_table before any device
call."""

import ctypes
import random
import struct

import numpy as np
import pytest

import scheduling_persistent_attn_amd as dash
from oracle import schedule as sch
from oracle import search as se


def _lists(offs, tasks):
    return [int(x) for x in offs], [tuple(int(v) for v in t) for t in np.asarray(tasks).tolist()]


# (S, D) -> (N, passes per task) of the kernel that runs it
SHAPES = {(256, 64): (4, 2), (512, 64): (8, 2), (1024, 64): (4, 4), (384, 128): (3, 4),
          (512, 128): (4, 4), (768, 128): (3, 8), (1024, 128): (4, 8), (1536, 128): (6, 8),
          (2048, 128): (8, 8), (4096, 128): (16, 8)}


def test_shapes_table():
    for (S, D), (N, passes) in SHAPES.items():
        T = dash.dash_attn_tile_size(S, D)
        assert (S + T - 1) // T == N


@pytest.mark.parametrize("s,m", [(sch.NAIVE, sch.FULL), (sch.NAIVE, sch.CAUSAL),
                                 (sch.DESCENDING_Q, sch.FULL), (sch.DESCENDING_Q, sch.CAUSAL),
                                 (sch.SHIFT, sch.FULL), (sch.SHIFT, sch.CAUSAL),
                                 (sch.SYMMETRIC_SHIFT, sch.CAUSAL)])
@pytest.mark.parametrize("N,G", [(1, 1), (2, 3), (4, 2), (7, 1), (8, 3)])
def test_closed_form_tables_equal_oracle(s, m, N, G):
    if s == sch.SYMMETRIC_SHIFT and N % 2:
        with pytest.raises(dash.DashError):
            dash.dash_schedule_table_closed_form(m, s, N, G)
        return
    got = _lists(*dash.dash_schedule_table_closed_form(m, s, N, G))
    assert got == se.closed_form_table(s, m, N, G)
    assert dash.dash_schedule_table_tasks(m, N, G) == G * se.tiles(m, N)


def _mutations(offs, tasks, rng, n):
    """Seeded random edits: swapped ranks, reordered tasks inside an item,
    moved item boundaries, swapped items."""
    out = []
    for _ in range(n):
        o, t = list(offs), list(tasks)
        kind = rng.randrange(4)
        if kind == 0:
            a, b = rng.randrange(len(t)), rng.randrange(len(t))
            if t[a][0] == t[b][0] and t[a][2] == t[b][2]:   # same dQ tile: a valid rank swap
                t[a], t[b] = t[a][:3] + (t[b][3],), t[b][:3] + (t[a][3],)
        elif kind == 1:
            k = rng.randrange(len(o) - 1)
            seg = t[o[k]:o[k + 1]]
            rng.shuffle(seg)
            t[o[k]:o[k + 1]] = seg
        elif kind == 2 and len(o) > 2:
            k = rng.randrange(1, len(o) - 1)
            o[k] = rng.randrange(o[k - 1], o[k + 1] + 1)
        else:
            k1, k2 = rng.randrange(len(o) - 1), rng.randrange(len(o) - 1)
            items = [t[o[k]:o[k + 1]] for k in range(len(o) - 1)]
            items[k1], items[k2] = items[k2], items[k1]
            t = [x for it in items for x in it]
            o = [0]
            for it in items:
                o.append(o[-1] + len(it))
        out.append((o, t))
    return out


@pytest.mark.parametrize("S,D", [(256, 64), (384, 128), (1024, 128), (1536, 128)])
@pytest.mark.parametrize("m", [sch.FULL, sch.CAUSAL])
@pytest.mark.parametrize("G", [1, 2])
def test_table_check_equals_oracle(S, D, m, G):
    N, passes = SHAPES[(S, D)]
    rng = random.Random(1000 * S + 10 * G + m)
    cands = []
    for s in (sch.NAIVE, sch.DESCENDING_Q, sch.SHIFT, sch.SYMMETRIC_SHIFT):
        if s == sch.SYMMETRIC_SHIFT and (m != sch.CAUSAL or N % 2):
            continue
        cands.append(se.closed_form_table(s, m, N, G))
    for kind in (se.SYMMETRIC, se.SHIFT, se.DESCENDING, se.ASCENDING):
        if not se.family_applies(m, N, kind):
            continue
        units = N // 2 if kind == se.SYMMETRIC else N
        for order in (0, 1):
            for b in se.family_blocks(units, units):
                cands.append(se.family_table(m, N, G, kind, order, b))
    muts = []
    for offs, tasks in cands:
        muts.extend(_mutations(offs, tasks, rng, 6))
    n_ok = n_bad = 0
    for offs, tasks in cands + muts:
        for P in (1, 2, N):
            want = se.structure_ok(m, N, G, offs, tasks) and \
                se.protocol_ok(m, N, offs, tasks, passes, P)[0]
            got = dash.dash_schedule_table_check(S, D, m, G, P, offs, tasks)
            assert got == (dash.DASH_OK if want else dash.DASH_ERR_TABLE), (offs, tasks, P)
            n_ok += want
            n_bad += not want
    assert n_ok > 0 and n_bad > 0


@pytest.mark.parametrize("m", [sch.FULL, sch.CAUSAL])
@pytest.mark.parametrize("N,G,groups,P", [(4, 1, 1, 4), (4, 2, 3, 2), (6, 1, 2, 3), (8, 2, 1, 5)])
def test_table_simulation_equals_oracle(m, N, G, groups, P):
    c, cd, r = 5.0, 3.0, 1.0
    for kind in (se.SYMMETRIC, se.SHIFT, se.DESCENDING, se.ASCENDING):
        if not se.family_applies(m, N, kind):
            continue
        units = N // 2 if kind == se.SYMMETRIC else N
        for b in se.family_blocks(units, P):
            offs, tasks = se.family_table(m, N, G, kind, 1, b)
            ref = se.simulate_table(m, N, G, groups, P, offs, tasks, c, cd, r)
            got = dash.dash_sim_table(m, N, G, groups, P, 1, offs, tasks, c, cd, r)
            assert bool(got["deadlock"]) == ref["deadlock"]
            assert got["total_work"] == ref["total_work"]
            assert got["base_makespan"] == ref["base_makespan"]
            if not ref["deadlock"]:
                assert got["makespan"] == ref["makespan"]
                assert got["violations"] == ref["violations"]


SEARCH_CASES = [(S, D, m, G, groups, P)
                for (S, D) in ((256, 64), (384, 128), (1024, 128), (1536, 128), (4096, 128))
                for m in (sch.FULL, sch.CAUSAL)
                for (G, groups, P) in ((1, 1, 2), (2, 3, 4), (1, 2, 16), (3, 1, 3))]


@pytest.mark.parametrize("S,D,m,G,groups,P", SEARCH_CASES)
def test_search_equals_oracle(S, D, m, G, groups, P):
    # binary fractions keep both simulators exact, so ties break alike
    N, passes = SHAPES[(S, D)]
    c, cd, r = 1.0, 0.5, 0.125
    got = dash.dash_schedule_search(S, D, m, G, groups, P, c, cd, r)
    head_form_ok = dash.dash_attn_tile_size(S, D) == 256
    offs, tasks, fam, rep = se.search(m, N, G, groups, P, passes, c, cd, r, head_form_ok)
    assert _lists(got["item_offsets"], got["tasks"]) == (offs, tasks)
    assert got["family"] == fam
    assert got["report"]["makespan"] == rep["makespan"]
    assert dash.dash_schedule_table_check(S, D, m, G, P, offs, tasks) == dash.DASH_OK


def test_search_beyond_the_grid():
    # 16 chains on 4 workgroups: the closed-form shift is refused, the search
    # runs it in blocks at the work bound
    got = dash.dash_schedule_search(4096, 128, sch.FULL, 1, 1, 4, 1.0, 1.0, 0.25)
    assert got["family"] == (dash.FAMILY_SHIFT, 0, 4)
    assert got["report"]["makespan"] == pytest.approx(16 * 16 / 4 * 1.25)
    offs, tasks = dash.dash_schedule_table_closed_form(sch.FULL, sch.SHIFT, 16, 1)
    assert dash.dash_schedule_table_check(4096, 128, sch.FULL, 1, 4, offs, tasks) == dash.DASH_ERR_TABLE
    assert dash.dash_schedule_table_check(4096, 128, sch.FULL, 1, 16, offs, tasks) == dash.DASH_OK


def test_pack_layout():
    S, D, m, G = 1024, 128, sch.CAUSAL, 2
    offs, tasks = dash.dash_schedule_table_closed_form(m, sch.SYMMETRIC_SHIFT, 4, G)
    raw = dash.dash_schedule_table_pack(S, D, m, G, offs, tasks)
    items, n = len(offs) - 1, len(tasks)
    tw = 8 + ((items + 2) & ~1)
    assert len(raw) == 4 * (tw + 2 * n)
    w = struct.unpack("<%dI" % (len(raw) // 4), raw)
    # magic, N, G, mask, passes, items, widest block (the pairs wait on each
    # other: one block of both), tasks
    assert w[:8] == (0x54485344, 4, G, m, 8, items, items, n)
    assert list(w[8:8 + items + 1]) == [int(x) for x in offs]
    tl = [tuple(int(v) for v in t) for t in np.asarray(tasks).tolist()]
    for t, (g, i, j, r) in enumerate(tl):
        w0, w1 = w[tw + 2 * t], w[tw + 2 * t + 1]
        assert (w0 & 0xffff, w0 >> 16) == (i, j)
        assert (w1 & 0xffff, (w1 >> 16) & 0x3fff) == (g, r)
        k = max(x for x in range(items) if offs[x] <= t)
        begin = t == offs[k] or tl[t - 1][1] != i
        end = t == offs[k + 1] - 1 or tl[t + 1][1] != i
        assert ((w1 >> 30) & 1, w1 >> 31) == (begin, end)
    # invalid tables and short buffers are refused
    bad = np.array(tasks, dtype=np.int32)
    bad[0, 3] = 1 - bad[0, 3] if bad[0, 3] < 2 else 0
    with pytest.raises(dash.DashError) as e:
        dash.dash_schedule_table_pack(S, D, m, G, offs, bad)
    assert e.value.status == dash.DASH_ERR_TABLE
    o = np.ascontiguousarray(offs, dtype=np.int32)
    tk = np.ascontiguousarray(tasks, dtype=np.int32)
    st = ctypes.c_int()
    buf = ctypes.create_string_buffer(16)
    dash.lib().dash_schedule_table_pack(S, D, m, G, items, dash._iptr(o), dash._iptr(tk), buf, 16,
                                        ctypes.byref(st))
    assert st.value == dash.DASH_ERR_WORKSPACE


def _bwd_table(**kw):
    args = dict(B=1, Hq=2, Hkv=1, S=1024, D=128, mask=0, table=1 << 12, tb=1 << 20, items=4,
                grid=0, ws=1 << 12, wsb=1 << 30, q=1 << 12)
    args.update(kw)
    p = ctypes.c_void_p
    a = p(1 << 12)
    return dash.lib().dash_attn_bwd_table(
        p(args["q"]), a, a, a, a, a, a, a, a, args["B"], args["Hq"], args["Hkv"], args["S"],
        args["D"], args["mask"], p(args["table"]), args["tb"], args["items"], args["grid"],
        p(args["ws"]), args["wsb"], None)


def test_bwd_table_validation_before_device():
    assert _bwd_table(table=None) == dash.DASH_ERR_NULL
    assert _bwd_table(table=(1 << 12) + 2) == dash.DASH_ERR_SHAPE
    assert _bwd_table(items=0) == dash.DASH_ERR_TABLE
    assert _bwd_table(items=9) == dash.DASH_ERR_TABLE          # more items than G * N runs
    assert _bwd_table(tb=64) == dash.DASH_ERR_TABLE            # shorter than the table
    assert _bwd_table(Hq=3, Hkv=2) == dash.DASH_ERR_SHAPE
    assert _bwd_table(D=96) == dash.DASH_ERR_UNSUPPORTED
    assert _bwd_table(S=0, table=None) == dash.DASH_OK         # empty: nothing to launch
    # the plain entry points need the table
    p = ctypes.c_void_p
    a = p(1 << 12)
    assert dash.lib().dash_attn_bwd(a, a, a, a, a, a, a, a, a, 1, 2, 2, 256, 64, 0, dash.TABLE, a,
                                    1 << 30, None) == dash.DASH_ERR_SCHEDULE_MASK
    assert dash.lib().dash_attn_bwd_run(a, a, a, a, a, a, a, 1, 2, 2, 256, 64, 0, dash.TABLE, a,
                                        1 << 30, None) == dash.DASH_ERR_SCHEDULE_MASK


def _bwd_table_run(**kw):
    args = dict(B=1, Hq=2, Hkv=1, S=1024, D=128, mask=0, table=1 << 12, tb=1 << 20, items=4,
                grid=0, ws=1 << 12, wsb=1 << 30, q=1 << 12, dq=1 << 12)
    args.update(kw)
    p = ctypes.c_void_p
    a = p(1 << 12)
    return dash.lib().dash_attn_bwd_table_run(
        p(args["q"]), a, a, a, p(args["dq"]), a, a, args["B"], args["Hq"], args["Hkv"], args["S"],
        args["D"], args["mask"], p(args["table"]), args["tb"], args["items"], args["grid"],
        p(args["ws"]), args["wsb"], None)


def test_bwd_table_run_validation_before_device():
    # the run phase alone checks like the one-call form (no o, lse needed)
    assert _bwd_table_run(table=None) == dash.DASH_ERR_NULL
    assert _bwd_table_run(table=(1 << 12) + 2) == dash.DASH_ERR_SHAPE
    assert _bwd_table_run(items=0) == dash.DASH_ERR_TABLE
    assert _bwd_table_run(items=9) == dash.DASH_ERR_TABLE
    assert _bwd_table_run(tb=64) == dash.DASH_ERR_TABLE
    assert _bwd_table_run(Hq=3, Hkv=2) == dash.DASH_ERR_SHAPE
    assert _bwd_table_run(D=96) == dash.DASH_ERR_UNSUPPORTED
    assert _bwd_table_run(S=0, table=None) == dash.DASH_OK


def test_table_workspace_holds_per_head_partials():
    # with 256-key tiles and grouped heads a table may be in the per-head
    # form: the workspace keeps one fp32 dK/dV partial per query head, the
    # most any closed form splits into
    for (B, Hq, Hkv, S) in ((1, 8, 1, 4096), (2, 4, 2, 2048)):
        G = Hq // Hkv
        assert dash.dash_attn_bwd_head_parts(B, Hq, Hkv, S, 128, 0, dash.TABLE) == G
        n_t = dash.dash_attn_bwd_workspace_size(B, Hq, Hkv, S, 128, 0, dash.TABLE)
        assert dash.dash_attn_bwd_head_parts(B, Hq, Hkv, S, 128, 0, dash.SHIFT) > 1
        assert n_t >= dash.dash_attn_bwd_workspace_size(B, Hq, Hkv, S, 128, 0, dash.SHIFT)
    # one head per group, or small tiles: no partials
    assert dash.dash_attn_bwd_head_parts(1, 4, 4, 4096, 128, 0, dash.TABLE) == 1
    assert dash.dash_attn_bwd_head_parts(1, 4, 2, 512, 128, 0, dash.TABLE) == 1
    # beyond the closed forms' workspace: room for the largest table (the one
    # AUTO may resolve to), 8 header words, 6 offset words and 2 words per
    # task of the 16 full-mask tasks, rounded to 256 bytes
    words = 8 + ((4 + 2) & ~1) + 2 * 16
    assert dash.dash_attn_bwd_workspace_size(1, 2, 2, 256, 64, 0, dash.TABLE) == \
        dash.dash_attn_bwd_workspace_size(1, 2, 2, 256, 64, 0, dash.NAIVE) + ((4 * words + 255) & ~255)


FAMILY_CASES = [(m, N, G, kind, order, block)
                for m in (sch.FULL, sch.CAUSAL)
                for (N, G) in ((1, 1), (2, 3), (4, 2), (6, 1), (8, 3))
                for kind in (se.SYMMETRIC, se.SHIFT, se.DESCENDING, se.ASCENDING, se.PACKED)
                for order in ((0,) if kind == se.PACKED else (0, 1))
                for block in (1, 2, 3, 5, 64)
                if se.family_applies(m, N, kind) and (kind == se.PACKED or block <= max(1, N))]


@pytest.mark.parametrize("m,N,G,kind,order,block", FAMILY_CASES)
def test_family_tables_equal_oracle(m, N, G, kind, order, block):
    got = _lists(*dash.dash_schedule_table_family(m, N, G, kind, order, block))
    assert got == tuple(se.family_table(m, N, G, kind, order, block))


def test_family_arguments():
    with pytest.raises(ValueError):
        dash.dash_schedule_table_family(sch.CAUSAL, 4, 2, dash.FAMILY_PACKED, 1, 4)
    o, t = dash._table_out(8, 8)
    items = ctypes.c_int()
    f = dash.lib().dash_schedule_table_family
    # symmetric pairs need the causal mask and even N; blocks start at 1
    assert f(sch.FULL, 4, 1, dash.FAMILY_SYMMETRIC, 0, 1, ctypes.byref(items), dash._iptr(o),
             dash._iptr(t)) != dash.DASH_OK
    assert f(sch.CAUSAL, 4, 1, dash.FAMILY_SHIFT, 0, 0, ctypes.byref(items), dash._iptr(o),
             dash._iptr(t)) != dash.DASH_OK
    assert f(sch.CAUSAL, 4, 1, 9, 0, 1, ctypes.byref(items), dash._iptr(o),
             dash._iptr(t)) != dash.DASH_OK
    # the packed kind has one order; a bin count beyond the walks gives the
    # table of one walk per item (and allocates nothing for the rest)
    assert f(sch.CAUSAL, 4, 2, dash.FAMILY_PACKED, 1, 2, ctypes.byref(items), dash._iptr(o),
             dash._iptr(t)) == dash.DASH_ERR_SHAPE
    big = _lists(*dash.dash_schedule_table_family(sch.CAUSAL, 4, 2, dash.FAMILY_PACKED, 0, 1 << 30))
    assert big == _lists(*dash.dash_schedule_table_family(sch.CAUSAL, 4, 2, dash.FAMILY_PACKED, 0, 8))
    assert big == tuple(se.packed_table(sch.CAUSAL, 4, 2, 8))
    assert len(big[0]) - 1 == 8


def test_per_head_tables_on_256_key_tiles_only():
    # a packed table of two heads is in the per-head form: accepted with
    # 256-key tiles (S = 1024, D = 128 gives 4 tiles), refused with 128-key
    # tiles (S = 512, D = 128 gives 4 tiles as well)
    m, N, G = sch.CAUSAL, 4, 2
    offs, tasks = dash.dash_schedule_table_family(m, N, G, dash.FAMILY_PACKED, 0, 3)
    ol, tl = _lists(offs, tasks)
    assert se.table_form(ol, tl) == "head"
    assert dash.dash_attn_tile_size(1024, 128) == 256 and dash.dash_attn_tile_size(512, 128) == 128
    assert dash.dash_schedule_table_check(1024, 128, m, G, 3, offs, tasks) == dash.DASH_OK
    assert dash.dash_schedule_table_check(512, 128, m, G, 3, offs, tasks) == dash.DASH_ERR_UNSUPPORTED
    with pytest.raises(dash.DashError) as e:
        dash.dash_schedule_table_pack(512, 128, m, G, offs, tasks)
    assert e.value.status == dash.DASH_ERR_UNSUPPORTED
    raw = dash.dash_schedule_table_pack(1024, 128, m, G, offs, tasks)
    w = struct.unpack("<%dI" % (len(raw) // 4), raw)
    items, n = len(ol) - 1, len(tl)
    assert w[3] == m | 0x100                 # the per-head form's flag beside the mask
    assert w[5] == items and w[7] == n
    tw = 8 + ((items + 2) & ~1)
    for t, (g, i, j, r) in enumerate(tl):
        w1 = w[tw + 2 * t + 1]
        k = max(x for x in range(items) if ol[x] <= t)
        begin = t == ol[k] or tl[t - 1][:2] != (g, i)
        end = t == ol[k + 1] - 1 or tl[t + 1][:2] != (g, i)
        assert ((w1 >> 30) & 1, w1 >> 31) == (begin, end)
    # a tile-form table keeps the bare mask
    offs2, tasks2 = dash.dash_schedule_table_closed_form(m, sch.SHIFT, N, G)
    raw2 = dash.dash_schedule_table_pack(1024, 128, m, G, offs2, tasks2)
    assert struct.unpack("<4I", raw2[:16])[3] == m


def test_table_in_neither_form_is_refused():
    # head 0 of KV tile 0 in two pieces on either side of another run
    offs = [0, 1, 3, 4]
    tasks = [(0, 0, 0, 0), (0, 1, 0, 1), (0, 1, 1, 0), (0, 0, 1, 1)]
    assert dash.dash_schedule_table_check(512, 128, sch.FULL, 1, 4, offs, tasks) == dash.DASH_ERR_TABLE
    # more items than (head, tile) runs
    offs, tasks = dash.dash_schedule_table_family(sch.FULL, 2, 1, dash.FAMILY_PACKED, 0, 2)
    assert len(offs) == 3
    assert dash.dash_schedule_table_check(512, 256, sch.FULL, 1, 4, offs, tasks) in (
        dash.DASH_OK, dash.DASH_ERR_UNSUPPORTED)


def test_search_packs_grouped_heads():
    # 8 tiles of 256 keys, 7 heads per group, 2 groups on 16 workgroups: the
    # search picks the packed kind, as the oracle does
    S, D, m, G, groups, P = 2048, 128, sch.CAUSAL, 7, 2, 16
    c, cd, r = 1.0, 0.5, 0.125
    got = dash.dash_schedule_search(S, D, m, G, groups, P, c, cd, r)
    offs, tasks, fam, rep = se.search(m, 8, G, groups, P, 8, c, cd, r)
    assert got["family"] == fam == (dash.FAMILY_PACKED, 0, se.packed_bins(8, G, groups, P))
    assert _lists(got["item_offsets"], got["tasks"]) == (offs, tasks)
    assert got["report"]["makespan"] == rep["makespan"]
    # with 128-key tiles (S = 512) the per-head form cannot run
    assert dash.dash_attn_tile_size(512, 128) == 128
    got2 = dash.dash_schedule_search(512, 128, m, G, groups, P, c, cd, r)
    assert got2["family"][0] != dash.FAMILY_PACKED


AUTO_CASES = [
    # B, Hq, Hkv, S, D, mask, grid
    (1, 28, 4, 4096, 128, sch.CAUSAL, 256),   # closed forms split 7 heads into 7 parts
    (2, 14, 2, 4096, 128, sch.CAUSAL, 256),
    (1, 28, 4, 2048, 128, sch.CAUSAL, 256),
    (2, 6, 2, 4096, 128, sch.CAUSAL, 256),
    (4, 32, 8, 4096, 128, sch.CAUSAL, 256),   # whole-tile items only
    (1, 8, 4, 8192, 128, sch.CAUSAL, 256),
    (1, 4, 4, 2048, 128, sch.FULL, 64),
    (1, 28, 4, 512, 128, sch.CAUSAL, 256),    # 128-key tiles
    (1, 14, 2, 4096, 64, sch.CAUSAL, 128),
]


@pytest.mark.parametrize("B,Hq,Hkv,S,D,m,grid", AUTO_CASES)
def test_auto_choice_equals_oracle(B, Hq, Hkv, S, D, m, grid):
    # the closed forms simulated by the oracle with the library's head parts,
    # then the oracle's search where the table needs no more workspace; the
    # table wins only with a strictly shorter critical path
    from oracle import dag
    T = dash.dash_attn_tile_size(S, D)
    N = (S + T - 1) // T
    G = Hq // Hkv
    groups = B * Hkv
    passes = 8 if (T, D) == (256, 128) else 4 if T == 256 or (T, D) == (128, 128) else 2
    best = None
    for s in (sch.SYMMETRIC_SHIFT, sch.SHIFT, sch.DESCENDING_Q, sch.NAIVE):
        if s == sch.SYMMETRIC_SHIFT and (m != sch.CAUSAL or N % 2):
            continue
        parts = dash.dash_attn_bwd_head_parts(B, Hq, Hkv, S, D, m, s)
        rep = dag.simulate(s, m, N, G=G // parts, groups=groups * parts, P=grid, dispatch="dynamic",
                           c=1.0, c_diag=1.0, r=0.1)
        if rep["deadlock"]:
            continue
        if best is None or rep["makespan"] < best[1]:
            best = (s, rep["makespan"])
    want = best[0]
    same_ws = T != 256 or G == 1 or dash.dash_attn_bwd_head_parts(B, Hq, Hkv, S, D, m, dash.AUTO) == G
    if same_ws and groups * G * se.tiles(m, N) <= 1 << 18:
        found = se.search(m, N, G, groups, grid, passes, 1.0, 1.0, 0.1, T == 256)
        if found is not None:
            # a tie (the search returning a closed form) keeps the closed form
            if found[3]["makespan"] < best[1] - 1e-9:
                want = dash.TABLE
    assert dash.dash_attn_bwd_auto_schedule_on(B, Hq, Hkv, S, D, m, grid) == want


def test_auto_choice_picks_the_table_where_the_closed_forms_leave_units_idle():
    # on 256 workgroups: the 16k causal layer with 7 heads per KV head runs the
    # packed per-head table, the 8B layer the symmetric shift, the full-mask
    # 16k layer the shift; no table where it would need more workspace
    assert dash.dash_attn_bwd_auto_schedule_on(1, 28, 4, 16384, 128, 1, 256) == dash.TABLE
    assert dash.dash_attn_bwd_auto_schedule_on(4, 32, 8, 4096, 128, 1, 256) == dash.SYMMETRIC_SHIFT
    assert dash.dash_attn_bwd_auto_schedule_on(1, 32, 32, 16384, 128, 0, 256) == dash.SHIFT
    assert dash.dash_attn_bwd_auto_schedule_on(2, 24, 24, 4096, 64, 0, 256) == dash.SHIFT
    assert dash.dash_attn_bwd_auto_schedule_on(0, 28, 4, 4096, 128, 1, 256) == dash.NAIVE  # empty
    with pytest.raises(dash.DashError) as e:
        dash.dash_attn_bwd_auto_schedule_on(1, 28, 4, 4096, 128, 1, 0)
    assert e.value.status == dash.DASH_ERR_SHAPE
