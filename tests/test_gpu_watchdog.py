"""The watchdog error path of the ordered reduction, forced from the host, and
the turn-wait counters (the schedules' measured bubbles).

With a zero wall-clock limit any turn wait longer than 64 polls gives up.  The
naive (rigid ascending) order on a causal mask with 32 tiles makes chain i
wait about i task-times for its first turn, so some wait does; the kernel then
raises the workspace flag, every later wait gives up at once, the launch
drains, and dash_attn_bwd_check reports DASH_ERR_TIMEOUT.  With the default
limit restored, the next call on the same workspace is bit-identical to a run
before the forced failure (the preprocess clears the flag).
"""

import sys

import numpy as np
import pytest
import torch

import scheduling_persistent_attn_amd as dash

sys.path.insert(0, __file__.rsplit("/", 1)[0])
import gpu_util as gu  # noqa: E402

pytestmark = pytest.mark.gpu

CASE = (1, 4096, 8, 8, 128, True)  # B, S, Hq, Hkv, D, causal: N = 32


def _bits(ts):
    return [t.view(torch.int16).cpu().numpy().copy() for t in ts]


def test_forced_timeout_is_reported_and_recovers():
    B, S, Hq, Hkv, D, causal = CASE
    print("watchdog", CASE, "naive", flush=True)
    x = gu.gpu_inputs(B, S, Hq, Hkv, D, seed=2300)
    o, lse = gu.run_forward(x, causal)
    ws = dash.new_workspace(x["q"], x["k"], int(causal), dash.NAIVE)
    good = _bits(gu.run_backward(x, o, lse, causal, dash.NAIVE, workspace=ws))
    dash.dash_attn_bwd_check(ws)
    try:
        dash.dash_attn_set_watchdog(0.0)
        gu.run_backward(x, o, lse, causal, dash.NAIVE, workspace=ws, check=False)
        with pytest.raises(dash.DashError) as e:
            dash.dash_attn_bwd_check(ws)
        assert e.value.status == dash.DASH_ERR_TIMEOUT
        ctrl = ws.view(torch.int32)[:3].cpu().numpy()
        print("flag %d, waits that timed out %d" % (ctrl[1], ctrl[2]), flush=True)
        assert ctrl[1] == 1 and ctrl[2] >= 1
    finally:
        dash.dash_attn_set_watchdog(2.0)
    again = _bits(gu.run_backward(x, o, lse, causal, dash.NAIVE, workspace=ws))
    dash.dash_attn_bwd_check(ws)
    for a, b in zip(good, again):
        assert np.array_equal(a, b)
    cnt = gu.read_counters(ws, B, Hq, S, D)
    assert np.array_equal(cnt, gu.expected_counters(B, Hq, S, D, causal))


def test_turn_wait_counters():
    # the rigid ascending order on a causal mask keeps chain i waiting for
    # chains 0..i-1 at each of its dQ tiles, so waits are certain; the atomic
    # reference makes none.  The counters are cleared by each call.
    B, S, Hq, Hkv, D, causal = CASE
    print("wait counters", CASE, flush=True)
    x = gu.gpu_inputs(B, S, Hq, Hkv, D, seed=2400)
    o, lse = gu.run_forward(x, causal)
    ws = dash.new_workspace(x["q"], x["k"], int(causal), dash.NAIVE)
    gu.run_backward(x, o, lse, causal, dash.NAIVE, workspace=ws)
    st = dash.dash_attn_bwd_wait_stats(ws)
    print("naive", st, flush=True)
    assert st["waits"] > 0 and st["wait_seconds"] > 0.0
    assert st["polls"] >= 0
    gu.run_backward(x, o, lse, causal, dash.ATOMIC, workspace=ws)
    st = dash.dash_attn_bwd_wait_stats(ws)
    assert st == {"waits": 0, "polls": 0, "wait_seconds": 0.0}


def test_shift_family_removes_the_rigid_orders_bubbles():
    # the method's claim, measured: on a causal mask the rigid ascending order
    # leaves waves waiting for earlier dQ contributions for a large share of
    # the time, and the symmetric shift removes most of that waiting
    B, S, Hq, Hkv, D, causal = CASE
    print("bubbles", CASE, flush=True)
    x = gu.gpu_inputs(B, S, Hq, Hkv, D, seed=2500)
    o, lse = gu.run_forward(x, causal)
    waited = {}
    for sched in (dash.NAIVE, dash.SYMMETRIC_SHIFT):
        ws = dash.new_workspace(x["q"], x["k"], int(causal), sched)
        gu.run_backward(x, o, lse, causal, sched, workspace=ws)  # warm-up
        gu.run_backward(x, o, lse, causal, sched, workspace=ws)
        waited[sched] = dash.dash_attn_bwd_wait_stats(ws)["wait_seconds"]
    print("wave-seconds waiting: naive %.3g, symmetric shift %.3g"
          % (waited[dash.NAIVE], waited[dash.SYMMETRIC_SHIFT]), flush=True)
    assert waited[dash.NAIVE] > 0.0
    assert waited[dash.SYMMETRIC_SHIFT] < 0.25 * waited[dash.NAIVE]


def test_run_without_prepare_is_reported():
    # a second dash_attn_bwd_run on a workspace that dash_attn_bwd_prepare has
    # not reset computes nothing, leaves the outputs untouched and is reported
    # as DASH_ERR_NOT_PREPARED; a prepared run afterwards is bit-identical
    B, S, Hq, Hkv, D, causal = CASE
    print("run without prepare", CASE, flush=True)
    x = gu.gpu_inputs(B, S, Hq, Hkv, D, seed=2700)
    o, lse = gu.run_forward(x, causal)
    for sched in (dash.SHIFT, dash.ATOMIC):
        ws = dash.new_workspace(x["q"], x["k"], int(causal), sched)
        good = [t.clone() for t in gu.run_backward(x, o, lse, causal, sched, workspace=ws)]
        dq, dk, dv = (torch.full_like(t, 7.0) for t in good)
        dash.dash_attn_bwd_run(x["q"], x["k"], x["v"], x["do"], dq, dk, dv, int(causal), sched, ws)
        with pytest.raises(dash.DashError) as e:
            dash.dash_attn_bwd_check(ws)
        assert e.value.status == dash.DASH_ERR_NOT_PREPARED
        for t in (dq, dk, dv):
            assert bool((t == 7.0).all())
        dash.dash_attn_bwd_prepare(o, x["do"], lse, tuple(x["q"].shape), Hkv, int(causal), sched, ws)
        dash.dash_attn_bwd_run(x["q"], x["k"], x["v"], x["do"], dq, dk, dv, int(causal), sched, ws)
        dash.dash_attn_bwd_check(ws)
        if sched != dash.ATOMIC:
            for a, b in zip(good, (dq, dk, dv)):
                assert torch.equal(a.view(torch.int16), b.view(torch.int16))
