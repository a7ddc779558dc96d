"""GPU checks of the AUTO schedule: it resolves, per shape and device, to one
of the deterministic schedules or the searched task table, chosen by the
critical-path simulator, and a backward with AUTO is bitwise the backward of
the schedule it resolves to."""

import sys

import pytest
import torch

import scheduling_persistent_attn_amd as dash

sys.path.insert(0, __file__.rsplit("/", 1)[0])
import gpu_util as gu  # noqa: E402

pytestmark = pytest.mark.gpu

CASES = [
    # B, S, Hq, Hkv, D, causal
    (1, 1024, 8, 2, 128, True),
    (2, 1024, 4, 4, 64, False),
    (1, 300, 2, 1, 64, True),     # odd tile count: no symmetric shift
]


@pytest.mark.parametrize("case", CASES)
def test_auto_equals_resolved_schedule(case):
    B, S, Hq, Hkv, D, causal = case
    sched = dash.dash_attn_bwd_auto_schedule(B, Hq, Hkv, S, D, int(causal))
    print("auto", case, "->", sched, flush=True)
    assert sched in dash.DETERMINISTIC
    T = dash.dash_attn_tile_size(S, D)
    if sched == dash.SYMMETRIC_SHIFT:
        assert causal and ((S + T - 1) // T) % 2 == 0
    x = gu.gpu_inputs(B, S, Hq, Hkv, D, seed=2300)
    o, lse = gu.run_forward(x, causal)
    ref = gu.run_backward(x, o, lse, causal, sched)
    got = gu.run_backward(x, o, lse, causal, dash.AUTO)
    torch.cuda.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_auto_on_the_8b_layer_shape():
    # on a 256-CU device the simulator ranks the symmetric shift first for
    # the causal B=4 S=4096 Hq=32 Hkv=8 D=128 layer, as measured
    props = torch.cuda.get_device_properties(0)
    sched = dash.dash_attn_bwd_auto_schedule(4, 32, 8, 4096, 128, 1)
    print("auto 8B layer ->", sched, "on", props.multi_processor_count, "CUs", flush=True)
    if props.multi_processor_count == 256:
        assert sched == dash.SYMMETRIC_SHIFT
    # the choice is cached: the same answer every time
    assert dash.dash_attn_bwd_auto_schedule(4, 32, 8, 4096, 128, 1) == sched


TABLE_CASES = [
    # B, S, Hq, Hkv, D, causal -- on 256 compute units AUTO runs the searched
    # table here (the closed forms split the 7 heads of a group into 7 parts)
    (1, 4096, 28, 4, 128, True),
    (1, 8192, 28, 4, 64, True),
    (1, 4096, 21, 3, 64, True),    # its workspace fits the static 64 MiB
]


@pytest.mark.parametrize("case", TABLE_CASES)
def test_auto_runs_the_searched_table(case):
    # AUTO's choice equals the host-only decision for this device's grid; where
    # it is the searched table, a backward with AUTO (one call, and prepare +
    # run on a reused workspace) is bitwise the backward of that table run
    # through dash_attn_bwd_table
    B, S, Hq, Hkv, D, causal = case
    mask = int(causal)
    grid = dash.dash_attn_bwd_grid_size(S, D, mask)
    sched = dash.dash_attn_bwd_auto_schedule(B, Hq, Hkv, S, D, mask)
    print("auto", case, "->", sched, "on a grid of", grid, flush=True)
    assert sched == dash.dash_attn_bwd_auto_schedule_on(B, Hq, Hkv, S, D, mask, grid)
    if sched != dash.TABLE:
        pytest.skip("AUTO picks a closed form on this device's grid")
    G = Hq // Hkv
    res = dash.dash_schedule_search(S, D, mask, G, B * Hkv, grid, 1.0, 1.0, 0.1)
    x = gu.gpu_inputs(B, S, Hq, Hkv, D, seed=2400)
    o, lse = gu.run_forward(x, causal)
    table, items = dash.upload_table(x["q"], x["k"], causal, res["item_offsets"], res["tasks"])
    ref = dash.backward_table(x["q"], x["k"], x["v"], o, x["do"], lse, causal, table, items)
    ws = dash.new_workspace(x["q"], x["k"], mask, dash.AUTO)
    got = gu.run_backward(x, o, lse, causal, dash.AUTO, workspace=ws)
    for a, b in zip(ref, got):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    # the two phases on the same workspace, twice (each prepare copies the
    # table in again)
    for _ in range(2):
        dq, dk, dv = (torch.full_like(t, 7.0) for t in got)
        dash.dash_attn_bwd_prepare(o, x["do"], lse, tuple(x["q"].shape), Hkv, mask, dash.AUTO, ws)
        dash.dash_attn_bwd_run(x["q"], x["k"], x["v"], x["do"], dq, dk, dv, mask, dash.AUTO, ws)
        dash.dash_attn_bwd_check(ws)
        for a, b in zip(ref, (dq, dk, dv)):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    # the no-allocation entry point keeps AUTO among the closed forms: its
    # result is bitwise one of theirs
    if dash.dash_attn_bwd_workspace_size(B, Hq, Hkv, S, D, mask, dash.AUTO) <= dash.NOALLOC_WORKSPACE_BYTES:
        print("  no-allocation entry point with AUTO", flush=True)
        dq, dk, dv = (torch.empty_like(t) for t in got)
        dash.dash_attn_bwd_noalloc(x["q"], x["k"], x["v"], o, x["do"], lse, dq, dk, dv, mask, dash.AUTO)
        torch.cuda.synchronize()
        matches = []
        for s in dash.DETERMINISTIC:
            r = gu.run_backward(x, o, lse, causal, s)
            if all(torch.equal(a.view(torch.int16), b.view(torch.int16)) for a, b in zip(r, (dq, dk, dv))):
                matches.append(s)
        assert matches, "no closed form gives the no-allocation AUTO result"
