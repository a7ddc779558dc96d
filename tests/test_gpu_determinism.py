"""Run-to-run bit identity of every deterministic schedule on the GPU.

20 runs per schedule rotate over three streams with a seeded, varying amount
of unrelated GPU work queued before each call, and every other run has a
kernel on a fourth stream occupying compute units while the backward starts
(it waits on nothing, so the backward's workgroups that cannot yet be resident
only wait for it to drain), so that workgroups reach the ordered reductions in
different orders and places; dq/dk/dv must not change by a bit.
The atomic reference is run the same way at a full workload size, and at
least one of its runs must differ (the positive control that shows the harness
can see non-determinism).  One case has more items than the persistent grid
has workgroups, so workgroups take further items as they finish, in an order
that varies from run to run; the full-size cases are in
test_gpu_determinism_fullsize.py.
"""

import random
import sys

import numpy as np
import pytest
import torch

import scheduling_persistent_attn_amd as dash

sys.path.insert(0, __file__.rsplit("/", 1)[0])
import gpu_util as gu  # noqa: E402

pytestmark = pytest.mark.gpu

RUNS = 20

CASES = [
    # B, S, Hq, Hkv, D, causal
    (1, 1024, 8, 2, 128, True),
    (2, 1024, 4, 4, 64, False),
    (1, 2048, 8, 8, 128, False),
    (2, 1024, 16, 4, 128, True),  # 8 groups: one item queue per XCD
    (2, 4096, 8, 8, 128, False),  # 512 chains on 256 workgroups: dynamic re-dispatch
]


def _perturb(rng, stream, scratch):
    # unrelated work of random length ahead of the call on the same stream
    with torch.cuda.stream(stream):
        for _ in range(rng.randint(0, 6)):
            scratch.mul_(1.0001)


def _runs(case, sched):
    B, S, Hq, Hkv, D, causal = case
    x = gu.gpu_inputs(B, S, Hq, Hkv, D, seed=2000)
    o, lse = gu.run_forward(x, causal)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(3)]
    busy = torch.cuda.Stream()
    rng = random.Random(1234 + sched)
    scratch = torch.ones(1 << 22, device="cuda")
    big = torch.ones(1 << 27, device="cuda")  # 512 MiB: about a millisecond per pass over it
    outs = []
    for n in range(RUNS):
        s = streams[n % 3]
        _perturb(rng, s, scratch)
        if n % 2:
            # compute units occupied by unrelated work as the backward launches
            busy.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(busy):
                for _ in range(2):
                    big.mul_(1.0001)
        ws = dash.new_workspace(x["q"], x["k"], int(causal), sched)
        with torch.cuda.stream(s):
            dq, dk, dv = gu.run_backward(x, o, lse, causal, sched, workspace=ws, stream=s)
        dash.dash_attn_bwd_check(ws, stream=s)
        torch.cuda.current_stream().wait_stream(busy)
        outs.append(tuple(t.view(torch.int16).cpu().numpy().copy() for t in (dq, dk, dv)))
        if sched != dash.ATOMIC:
            cnt = gu.read_counters(ws, B, Hq, S, D)
            assert np.array_equal(cnt, gu.expected_counters(B, Hq, S, D, causal))
    return outs


def _sched_list(case):
    B, S, Hq, Hkv, D, causal = case
    T = dash.dash_attn_tile_size(S, D)
    N = (S + T - 1) // T
    out = [dash.NAIVE, dash.DESCENDING_Q, dash.SHIFT]
    if causal and N % 2 == 0:
        out.append(dash.SYMMETRIC_SHIFT)
    return out


@pytest.mark.parametrize("case", CASES)
def test_bit_identical_over_runs(case):
    for sched in _sched_list(case):
        print("determinism", case, "schedule", sched, flush=True)
        outs = _runs(case, sched)
        for n in range(1, RUNS):
            for a, b in zip(outs[0], outs[n]):
                assert np.array_equal(a, b), (sched, n)


def test_atomic_reference_spread():
    # the causal 8B-Llama-shaped layer (B=4 S=4096 Hq=32 Hkv=8 D=128): with
    # 32768 dQ slices each summed from up to 32 unordered atomic contributions,
    # the harness must see the order change
    case = (4, 4096, 32, 8, 128, True)
    print("atomic reference", case, flush=True)
    outs = _runs(case, dash.ATOMIC)
    differing = sum(1 for n in range(1, RUNS)
                    if not np.array_equal(outs[0][0], outs[n][0]))
    print("atomic reference: %d of %d runs differ from the first in dq" % (differing, RUNS - 1))
    assert differing >= 1


@pytest.mark.parametrize("sched", [dash.SHIFT, dash.SYMMETRIC_SHIFT])
def test_two_phase_call_equals_single_call(sched):
    # dash_attn_bwd_prepare + dash_attn_bwd_run is dash_attn_bwd, bit for bit,
    # and a workspace can be reused call after call
    B, S, Hq, Hkv, D, causal = CASES[0]
    print("two-phase", CASES[0], "schedule", sched, flush=True)
    x = gu.gpu_inputs(B, S, Hq, Hkv, D, seed=2100)
    o, lse = gu.run_forward(x, causal)
    ws = dash.new_workspace(x["q"], x["k"], int(causal), sched)
    ref = gu.run_backward(x, o, lse, causal, sched, workspace=ws)
    ref = [t.clone() for t in ref]
    dq, dk, dv = (torch.empty_like(t) for t in ref)
    for _ in range(3):
        dash.dash_attn_bwd_prepare(o, x["do"], lse, tuple(x["q"].shape), Hkv, int(causal),
                                   sched, ws)
        dash.dash_attn_bwd_run(x["q"], x["k"], x["v"], x["do"], dq, dk, dv, int(causal),
                               sched, ws)
        dash.dash_attn_bwd_check(ws)
        for a, b in zip(ref, (dq, dk, dv)):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16))
