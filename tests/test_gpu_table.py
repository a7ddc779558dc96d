"""GPU tests of schedules given as task tables (dash_attn_bwd_table).

* The closed forms written as tables run bit for bit like the closed-form
  schedules (dq always; dk/dv where the closed form does not split heads).
* Searched tables with more key/value chains than workgroups (a capped grid:
  N > P, where the closed-form shift cannot run) against the float64 oracle,
  element by element, to the parity bar of tests/gpu_util.py, with every turn
  counter ending at its contributor count.
* 20 perturbed runs of a searched table are bitwise identical.
* Packed tables in the per-head form (each run one query head's key/value
  tile, dK/dV summed over fp32 per-head partials) against the float64
  oracle, with counters, a bitwise rerun, and a whole-tile table run next on
  the same workspace (the per-head mark does not outlive its run).
* 12 seeded random tables (shuffled walks, run order and item cuts, whole-tile
  and per-head runs, full and capped grids) that pass the host check match
  the oracle, end their counters right and rerun bit for bit.
* The 128-key kernel refuses a header forged to claim the per-head form.
* The kernel refuses a table made for another kernel, and a launch narrower
  than the table's widest dispatch block: nothing is written and
  dash_attn_bwd_check reports DASH_ERR_TABLE (the kernels return before any
  work, so no wait is ever started).
"""

import random
import sys

import numpy as np
import pytest
import torch

import scheduling_persistent_attn_amd as dash
from oracle import attention as oa

sys.path.insert(0, __file__.rsplit("/", 1)[0])
import gpu_util as gu  # noqa: E402

pytestmark = pytest.mark.gpu


def _tiles(S, D):
    T = dash.dash_attn_tile_size(S, D)
    return T, (S + T - 1) // T


def _same(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


CLOSED = [
    # B, S, Hq, Hkv, D, causal -- one case per kernel tile and both masks
    (1, 256, 2, 1, 64, True),     # T = 64
    (2, 1024, 4, 2, 64, False),   # D = 64, T = 256
    (1, 512, 4, 2, 128, True),    # D = 128, T = 128
    (1, 2048, 2, 2, 128, False),  # T = 256
    (1, 2048, 4, 1, 128, True),   # T = 256, G = 4 (closed forms split the heads)
]


@pytest.mark.parametrize("case", CLOSED, ids=lambda c: "B%dS%dH%d-%dD%d%s" % (
    c[0], c[1], c[2], c[3], c[4], "c" if c[5] else "f"))
def test_closed_forms_as_tables_bitwise(case):
    B, S, Hq, Hkv, D, causal = case
    T, N = _tiles(S, D)
    G = Hq // Hkv
    x = gu.gpu_inputs(B, S, Hq, Hkv, D, seed=5000)
    o, lse = gu.run_forward(x, causal)
    scheds = [dash.NAIVE, dash.DESCENDING_Q, dash.SHIFT]
    if causal and N % 2 == 0:
        scheds.append(dash.SYMMETRIC_SHIFT)
    for s in scheds:
        print("closed form as table", case, "schedule", s, flush=True)
        ref = gu.run_backward(x, o, lse, causal, s)
        offs, tasks = dash.dash_schedule_table_closed_form(int(causal), s, N, G)
        table, items = dash.upload_table(x["q"], x["k"], causal, offs, tasks)
        ws = dash.new_workspace(x["q"], x["k"], int(causal), dash.TABLE)
        got = dash.backward_table(x["q"], x["k"], x["v"], o, x["do"], lse, causal, table, items,
                                  workspace=ws)
        assert _same(got[0], ref[0]), s
        if dash.dash_attn_bwd_head_parts(B, Hq, Hkv, S, D, int(causal), s) == 1:
            assert _same(got[1], ref[1]) and _same(got[2], ref[2]), s
        cnt = gu.read_counters(ws, B, Hq, S, D)
        assert np.array_equal(cnt, gu.expected_counters(B, Hq, S, D, causal))


SEARCHED = [
    # B, S, Hq, Hkv, D, causal, grid
    (1, 2048, 2, 1, 128, False, 3),   # T = 256, N = 8 chains on 3 workgroups
    (1, 2048, 4, 2, 128, True, 2),    # T = 256, N = 8, two groups of G = 2
    (1, 4096, 2, 2, 64, False, 4),    # D = 64, T = 256, N = 16
    (1, 1900, 2, 1, 64, True, 5),     # D = 64, ragged last tile, N = 8
    (2, 512, 4, 2, 128, True, 2),     # D = 128, T = 128, N = 4
]


def _searched(case):
    B, S, Hq, Hkv, D, causal, grid = case
    T, N = _tiles(S, D)
    G = Hq // Hkv
    res = dash.dash_schedule_search(S, D, int(causal), G, B * Hkv, grid, 1.0, 1.0, 0.1)
    return res, N, G


@pytest.mark.parametrize("case", SEARCHED, ids=lambda c: "B%dS%dH%d-%dD%d%s-P%d" % (
    c[0], c[1], c[2], c[3], c[4], "c" if c[5] else "f", c[6]))
def test_searched_table_parity(case):
    B, S, Hq, Hkv, D, causal, grid = case
    res, N, G = _searched(case)
    print("searched table", case, "family", res["family"], "makespan",
          res["report"]["makespan"], flush=True)
    # the closed-form shift needs all N chains at once: not on this grid
    offs, tasks = dash.dash_schedule_table_closed_form(int(causal), dash.SHIFT, N, G)
    if not causal:
        assert dash.dash_schedule_table_check(S, D, int(causal), G, grid, offs, tasks) == \
            dash.DASH_ERR_TABLE
    x = gu.gpu_inputs(B, S, Hq, Hkv, D, seed=5100)
    h = {k: gu.host64(v) for k, v in x.items()}
    dq_ref, dk_ref, dv_ref = oa.attention_backward(h["q"], h["k"], h["v"], h["do"], causal)
    o, lse = gu.run_forward(x, causal)
    table, items = dash.upload_table(x["q"], x["k"], causal, res["item_offsets"], res["tasks"])
    ws = dash.new_workspace(x["q"], x["k"], int(causal), dash.TABLE)
    out = dash.backward_table(x["q"], x["k"], x["v"], o, x["do"], lse, causal, table, items,
                              grid=grid, workspace=ws)
    for name, got, ref in zip(("dq", "dk", "dv"), out, (dq_ref, dk_ref, dv_ref)):
        e = gu.errors(gu.host64(got), ref)
        print("  %s rel-l2 %.3e max-abs(excess) %.3e max-abs %.3e" % ((name,) + e))
        assert gu.within(e), (name, e)
    cnt = gu.read_counters(ws, B, Hq, S, D)
    assert np.array_equal(cnt, gu.expected_counters(B, Hq, S, D, causal))
    again = dash.backward_table(x["q"], x["k"], x["v"], o, x["do"], lse, causal, table, items,
                                grid=grid, workspace=ws)
    for a, b in zip(out, again):
        assert _same(a, b)


def test_searched_table_bit_identical_over_runs():
    case = (2, 4096, 8, 2, 128, False, 64)   # 16 chains per group on 64 workgroups
    B, S, Hq, Hkv, D, causal, grid = case
    res, N, G = _searched(case)
    print("determinism of a searched table", case, "family", res["family"], flush=True)
    x = gu.gpu_inputs(B, S, Hq, Hkv, D, seed=5200)
    o, lse = gu.run_forward(x, causal)
    table, items = dash.upload_table(x["q"], x["k"], causal, res["item_offsets"], res["tasks"])
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(3)]
    rng = random.Random(77)
    scratch = torch.ones(1 << 22, device="cuda")
    first = None
    for n in range(20):
        s = streams[n % 3]
        with torch.cuda.stream(s):
            for _ in range(rng.randint(0, 6)):
                scratch.mul_(1.0001)
            ws = dash.new_workspace(x["q"], x["k"], int(causal), dash.TABLE)
            out = dash.backward_table(x["q"], x["k"], x["v"], o, x["do"], lse, causal, table,
                                      items, grid=grid, workspace=ws, stream=s)
        s.synchronize()
        cur = [t.view(torch.int16).cpu().numpy().copy() for t in out]
        if first is None:
            first = cur
        for a, b in zip(first, cur):
            assert np.array_equal(a, b), n


PACKED = [
    # B, S, Hq, Hkv, D, causal, grid
    (1, 2048, 8, 2, 128, True, 16),   # T = 256, N = 8, G = 4: 32 walks per group into 8 items
    (2, 1900, 6, 2, 64, True, 12),    # D = 64, ragged last tile, G = 3
    (1, 2048, 4, 1, 128, False, 6),   # full mask, G = 4 on 6 workgroups
    (1, 3000, 7, 1, 128, True, 20),   # seven heads per group, ragged, N = 12
    (1, 2048, 16, 2, 128, True, 32),  # eight heads per group: eight partial slots
    (3, 1536, 6, 2, 64, False, 24),   # three batches, D = 64, full mask
]


@pytest.mark.parametrize("case", PACKED, ids=lambda c: "B%dS%dH%d-%dD%d%s-P%d" % (
    c[0], c[1], c[2], c[3], c[4], "c" if c[5] else "f", c[6]))
def test_packed_per_head_table_parity(case):
    from oracle import search as se
    B, S, Hq, Hkv, D, causal, grid = case
    T, N = _tiles(S, D)
    assert T == 256
    G = Hq // Hkv
    bins = se.packed_bins(N, G, B * Hkv, grid)
    offs, tasks = dash.dash_schedule_table_family(int(causal), N, G, dash.FAMILY_PACKED, 0, bins)
    tl = [tuple(int(v) for v in t) for t in np.asarray(tasks).tolist()]
    assert se.table_form([int(v) for v in offs], tl) == "head"
    assert dash.dash_schedule_table_check(S, D, int(causal), G, grid, offs, tasks) == dash.DASH_OK
    print("packed per-head table", case, "items", len(offs) - 1, flush=True)
    x = gu.gpu_inputs(B, S, Hq, Hkv, D, seed=5500)
    h = {k: gu.host64(v) for k, v in x.items()}
    dq_ref, dk_ref, dv_ref = oa.attention_backward(h["q"], h["k"], h["v"], h["do"], causal)
    o, lse = gu.run_forward(x, causal)
    table, items = dash.upload_table(x["q"], x["k"], causal, offs, tasks)
    ws = dash.new_workspace(x["q"], x["k"], int(causal), dash.TABLE)
    out = dash.backward_table(x["q"], x["k"], x["v"], o, x["do"], lse, causal, table, items,
                              grid=grid, workspace=ws)
    for name, got, ref in zip(("dq", "dk", "dv"), out, (dq_ref, dk_ref, dv_ref)):
        e = gu.errors(gu.host64(got), ref)
        print("  %s rel-l2 %.3e max-abs(excess) %.3e max-abs %.3e" % ((name,) + e))
        assert gu.within(e), (name, e)
    cnt = gu.read_counters(ws, B, Hq, S, D)
    assert np.array_equal(cnt, gu.expected_counters(B, Hq, S, D, causal))
    again = dash.backward_table(x["q"], x["k"], x["v"], o, x["do"], lse, causal, table, items,
                                grid=grid, workspace=ws)
    for a, b in zip(out, again):
        assert _same(a, b)
    # a whole-tile table next on the same workspace, on other inputs: its
    # kernel writes dK/dV itself, and the partial sum of the stale per-head
    # partials must not overwrite them (a fresh workspace gives the reference)
    print("  whole-tile table after it", flush=True)
    x2 = gu.gpu_inputs(B, S, Hq, Hkv, D, seed=5501)
    o2, lse2 = gu.run_forward(x2, causal)
    offs2, tasks2 = dash.dash_schedule_table_closed_form(int(causal), dash.NAIVE, N, G)
    table2, items2 = dash.upload_table(x2["q"], x2["k"], causal, offs2, tasks2)
    got2 = dash.backward_table(x2["q"], x2["k"], x2["v"], o2, x2["do"], lse2, causal, table2,
                               items2, workspace=ws)
    ref2 = dash.backward_table(x2["q"], x2["k"], x2["v"], o2, x2["do"], lse2, causal, table2,
                               items2)
    for a, b in zip(got2, ref2):
        assert _same(a, b)


def test_table_run_phase():
    # dash_attn_bwd_prepare (TABLE) then dash_attn_bwd_table_run gives the
    # one-call result bit for bit; a second run without a prepare computes
    # nothing, leaves the outputs untouched (no per-head sum either) and is
    # reported as not prepared
    from oracle import search as se
    B, S, Hq, Hkv, D, causal, grid = 1, 2048, 8, 2, 128, True, 16
    T, N = _tiles(S, D)
    G = Hq // Hkv
    offs, tasks = dash.dash_schedule_table_family(1, N, G, dash.FAMILY_PACKED, 0,
                                                  se.packed_bins(N, G, B * Hkv, grid))
    print("table run phase", (B, S, Hq, Hkv, D, causal, grid), flush=True)
    x = gu.gpu_inputs(B, S, Hq, Hkv, D, seed=5600)
    o, lse = gu.run_forward(x, causal)
    table, items = dash.upload_table(x["q"], x["k"], causal, offs, tasks)
    ws = dash.new_workspace(x["q"], x["k"], 1, dash.TABLE)
    ref = [t.clone() for t in dash.backward_table(x["q"], x["k"], x["v"], o, x["do"], lse, causal,
                                                  table, items, grid=grid, workspace=ws)]
    dq, dk, dv = _sentinel_outputs(x)
    dash.dash_attn_bwd_prepare(o, x["do"], lse, tuple(x["q"].shape), Hkv, 1, dash.TABLE, ws)
    dash.dash_attn_bwd_table_run(x["q"], x["k"], x["v"], x["do"], dq, dk, dv, 1, table, items,
                                 grid, ws)
    dash.dash_attn_bwd_check(ws)
    for a, b in zip(ref, (dq, dk, dv)):
        assert _same(a, b)
    dq, dk, dv = _sentinel_outputs(x)
    dash.dash_attn_bwd_table_run(x["q"], x["k"], x["v"], x["do"], dq, dk, dv, 1, table, items,
                                 grid, ws)
    with pytest.raises(dash.DashError) as e:
        dash.dash_attn_bwd_check(ws)
    assert e.value.status == dash.DASH_ERR_NOT_PREPARED
    for t in (dq, dk, dv):
        assert torch.all(t == 7.0)


def _sentinel_outputs(x):
    return (torch.full_like(x["q"], 7.0), torch.full_like(x["k"], 7.0), torch.full_like(x["v"], 7.0))


def test_kernel_refuses_a_table_for_another_kernel():
    # same N and G, packed for D = 64 (4 passes per task), launched at D = 128
    # (8 passes): the sizes agree, the header does not
    B, S, Hq, Hkv, D, causal = 1, 4096, 2, 1, 128, False
    T, N = _tiles(S, D)
    assert _tiles(S, 64)[1] == N
    offs, tasks = dash.dash_schedule_table_closed_form(0, dash.NAIVE, N, 2)
    raw = dash.dash_schedule_table_pack(S, 64, 0, 2, offs, tasks)
    table = torch.frombuffer(bytearray(raw), dtype=torch.uint8).cuda()
    x = gu.gpu_inputs(B, S, Hq, Hkv, D, seed=5300)
    o, lse = gu.run_forward(x, causal)
    dq, dk, dv = _sentinel_outputs(x)
    ws = dash.new_workspace(x["q"], x["k"], 0, dash.TABLE)
    print("refused table: wrong passes per task", flush=True)
    dash.dash_attn_bwd_table(x["q"], x["k"], x["v"], o, x["do"], lse, dq, dk, dv, 0, table,
                             len(offs) - 1, 0, ws)
    with pytest.raises(dash.DashError) as e:
        dash.dash_attn_bwd_check(ws)
    assert e.value.status == dash.DASH_ERR_TABLE
    for t in (dq, dk, dv):
        assert torch.all(t == 7.0)
    # the same workspace runs a valid table next
    table, items = dash.upload_table(x["q"], x["k"], causal, offs, tasks)
    got = dash.backward_table(x["q"], x["k"], x["v"], o, x["do"], lse, causal, table, items,
                              workspace=ws)
    ref = gu.run_backward(x, o, lse, causal, dash.NAIVE)
    assert _same(got[0], ref[0])


def test_kernel_refuses_a_per_head_flag_on_small_tiles():
    # a valid whole-tile table for 128-key tiles whose header is altered to
    # claim the per-head form: that kernel has no per-head partials, so it
    # refuses the table before any work and writes nothing
    B, S, Hq, Hkv, D, causal = 1, 512, 4, 2, 128, True
    T, N = _tiles(S, D)
    assert T == 128
    offs, tasks = dash.dash_schedule_table_closed_form(1, dash.NAIVE, N, 2)
    raw = bytearray(dash.dash_schedule_table_pack(S, D, 1, 2, offs, tasks))
    raw[12:16] = (int.from_bytes(raw[12:16], "little") | 0x100).to_bytes(4, "little")
    table = torch.frombuffer(raw, dtype=torch.uint8).cuda()
    x = gu.gpu_inputs(B, S, Hq, Hkv, D, seed=5800)
    o, lse = gu.run_forward(x, causal)
    dq, dk, dv = _sentinel_outputs(x)
    ws = dash.new_workspace(x["q"], x["k"], 1, dash.TABLE)
    print("refused table: per-head flag on 128-key tiles", flush=True)
    dash.dash_attn_bwd_table(x["q"], x["k"], x["v"], o, x["do"], lse, dq, dk, dv, 1, table,
                             len(offs) - 1, 0, ws)
    with pytest.raises(dash.DashError) as e:
        dash.dash_attn_bwd_check(ws)
    assert e.value.status == dash.DASH_ERR_TABLE
    for t in (dq, dk, dv):
        assert torch.all(t == 7.0)


def test_kernel_refuses_a_grid_narrower_than_a_block():
    # the full-mask shift is one dispatch block of N = 8 chains
    B, S, Hq, Hkv, D, causal = 1, 2048, 1, 1, 128, False
    T, N = _tiles(S, D)
    offs, tasks = dash.dash_schedule_table_closed_form(0, dash.SHIFT, N, 1)
    x = gu.gpu_inputs(B, S, Hq, Hkv, D, seed=5400)
    o, lse = gu.run_forward(x, causal)
    table, items = dash.upload_table(x["q"], x["k"], causal, offs, tasks)
    dq, dk, dv = _sentinel_outputs(x)
    ws = dash.new_workspace(x["q"], x["k"], 0, dash.TABLE)
    print("refused table: grid", N - 1, "for a block of", N, flush=True)
    dash.dash_attn_bwd_table(x["q"], x["k"], x["v"], o, x["do"], lse, dq, dk, dv, 0, table, items,
                             N - 1, ws)
    with pytest.raises(dash.DashError) as e:
        dash.dash_attn_bwd_check(ws)
    assert e.value.status == dash.DASH_ERR_TABLE
    for t in (dq, dk, dv):
        assert torch.all(t == 7.0)
    with pytest.raises(dash.DashError) as e:   # wider than the device: host refusal
        dash.dash_attn_bwd_table(x["q"], x["k"], x["v"], o, x["do"], lse, dq, dk, dv, 0, table,
                                 items, 1 << 20, ws)
    assert e.value.status == dash.DASH_ERR_SHAPE


def _random_table(mask, N, G, rng, per_head):
    """Seeded random table: shuffled walks, whole-tile or per-head runs in a
    shuffled order, random item cuts, ranks in the order the walks reach each
    dQ tile (position, then item)."""
    from oracle import schedule as sch
    chains = []
    for i in range(N):
        js = [j for j in range(N) if sch.valid(mask, i, j)]
        if per_head:
            for g in range(G):
                w = list(js)
                rng.shuffle(w)
                chains.append([(g, i, j) for j in w])
        else:
            rng.shuffle(js)
            chains.append([(g, i, j) for j in js for g in range(G)])
    rng.shuffle(chains)
    items, cur = [], []
    for x, ch in enumerate(chains):
        cur.extend(ch)
        if x == len(chains) - 1 or rng.random() < 0.5:
            items.append(cur)
            cur = []
    order = {}
    for k, lst in enumerate(items):
        for pos, (g, i, j) in enumerate(lst):
            order.setdefault((g, j), []).append((pos, k, i))
    rank = {}
    for (g, j), lst in order.items():
        for r, (_, _, i) in enumerate(sorted(lst)):
            rank[(g, i, j)] = r
    offs, tasks = [0], []
    for lst in items:
        tasks.extend((g, i, j, rank[(g, i, j)]) for (g, i, j) in lst)
        offs.append(len(tasks))
    return offs, tasks


RANDOM_CASES = [
    # B, S, Hq, Hkv, D, causal, grid (0 = the device's)
    (1, 256, 2, 1, 64, True, 0),       # 64-key tiles
    (1, 300, 3, 1, 64, False, 4),      # ragged, capped grid
    (2, 512, 4, 2, 128, True, 0),      # 128-key tiles
    (1, 1024, 4, 2, 128, False, 0),    # 256-key tiles
    (1, 1300, 6, 2, 128, True, 0),     # ragged
    (1, 2048, 6, 2, 64, True, 0),
    (2, 1024, 3, 1, 64, False, 6),
    (1, 2048, 4, 2, 128, False, 8),
    (1, 1800, 3, 3, 128, True, 0),     # one head per group
    (1, 2048, 6, 2, 128, True, 5),
    (2, 1500, 4, 1, 64, True, 0),
    (1, 1024, 8, 2, 128, True, 3),
]


@pytest.mark.parametrize("k", range(len(RANDOM_CASES)))
def test_random_valid_tables_parity(k):
    # random tables that pass the host check run to the oracle's result, end
    # every turn counter at its contributor count and rerun bit for bit;
    # per-head runs wherever the 256-key kernels and G > 1 allow them
    import random
    B, S, Hq, Hkv, D, causal, grid = RANDOM_CASES[k]
    T, N = _tiles(S, D)
    G = Hq // Hkv
    mask = int(causal)
    rng = random.Random(7000 + k)
    P = grid or dash.dash_attn_bwd_grid_size(S, D, mask)
    for _ in range(50):
        per_head = T == 256 and G > 1 and rng.random() < 0.6
        offs, tasks = _random_table(mask, N, G, rng, per_head)
        if dash.dash_schedule_table_check(S, D, mask, G, P, offs, tasks) == dash.DASH_OK:
            break
    else:
        pytest.fail("no valid random table in 50 draws")
    print("random table", RANDOM_CASES[k], "per-head", per_head, "items", len(offs) - 1, flush=True)
    x = gu.gpu_inputs(B, S, Hq, Hkv, D, seed=5700 + k)
    h = {kk: gu.host64(v) for kk, v in x.items()}
    refs = oa.attention_backward(h["q"], h["k"], h["v"], h["do"], causal)
    o, lse = gu.run_forward(x, causal)
    table, items = dash.upload_table(x["q"], x["k"], causal, offs, tasks)
    ws = dash.new_workspace(x["q"], x["k"], mask, dash.TABLE)
    out = [t.clone() for t in dash.backward_table(x["q"], x["k"], x["v"], o, x["do"], lse, causal, table,
                                                  items, grid=grid, workspace=ws)]
    for name, got, ref in zip(("dq", "dk", "dv"), out, refs):
        e = gu.errors(gu.host64(got), ref)
        print("  %s rel-l2 %.3e max-abs(excess) %.3e max-abs %.3e" % ((name,) + e))
        assert gu.within(e), (name, e)
    cnt = gu.read_counters(ws, B, Hq, S, D)
    assert np.array_equal(cnt, gu.expected_counters(B, Hq, S, D, causal))
    again = dash.backward_table(x["q"], x["k"], x["v"], o, x["do"], lse, causal, table, items, grid=grid,
                                workspace=ws)
    for a, b in zip(out, again):
        assert _same(a, b)
