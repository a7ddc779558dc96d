"""dash_attn_bwd_noalloc: the backward on the library's static device
workspace, for callers that cannot allocate.

Called through the C ABI twice in a row, the second time on a smaller problem
(whose workspace region overlaps what the first call left behind), then once
more on the first problem; every result must equal, bit for bit, that of
dash_attn_bwd with a workspace of its own on the same inputs (the same
kernels, so the same bits; that is stricter than the oracle tolerance).  A
problem whose workspace exceeds the static array is refused with
DASH_ERR_WORKSPACE before anything is enqueued.
"""

import sys

import pytest
import torch

import scheduling_persistent_attn_amd as dash

sys.path.insert(0, __file__.rsplit("/", 1)[0])
import gpu_util as gu  # noqa: E402

pytestmark = pytest.mark.gpu

CALLS = [
    # B, S, Hq, Hkv, D, causal, schedule
    (1, 2048, 8, 2, 128, True, dash.SYMMETRIC_SHIFT),
    (1, 640, 4, 4, 64, False, dash.SHIFT),        # smaller: reuses the first call's memory
    (1, 2048, 8, 2, 128, True, dash.SYMMETRIC_SHIFT),
]


def _case(B, S, Hq, Hkv, D, causal, sched, seed):
    x = gu.gpu_inputs(B, S, Hq, Hkv, D, seed=seed)
    o, lse = gu.run_forward(x, causal)
    ref = gu.run_backward(x, o, lse, causal, sched)
    dq, dk, dv = (torch.full_like(t, 3.0) for t in ref)
    dash.dash_attn_bwd_noalloc(x["q"], x["k"], x["v"], o, x["do"], lse, dq, dk, dv,
                               int(causal), sched)
    torch.cuda.synchronize()
    return ref, (dq, dk, dv)


def test_noalloc_equals_workspace_entry_point():
    for n, (B, S, Hq, Hkv, D, causal, sched) in enumerate(CALLS):
        print("noalloc call", n, (B, S, Hq, Hkv, D, causal), "schedule", sched, flush=True)
        need = dash.dash_attn_bwd_workspace_size(B, Hq, Hkv, S, D, int(causal), sched)
        assert 0 < need <= dash.NOALLOC_WORKSPACE_BYTES
        ref, got = _case(B, S, Hq, Hkv, D, causal, sched, seed=5000 + 10 * (n % 2))
        for name, a, b in zip(("dq", "dk", "dv"), ref, got):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), (n, name)


def test_noalloc_refuses_problems_beyond_the_static_workspace():
    B, S, Hq, Hkv, D = 1, 16384, 32, 32, 128
    assert dash.dash_attn_bwd_workspace_size(B, Hq, Hkv, S, D, 0, dash.SHIFT) > \
        dash.NOALLOC_WORKSPACE_BYTES
    x = gu.gpu_inputs(1, 64, 1, 1, 128)
    q = torch.empty((B, S, Hq, D), dtype=torch.bfloat16, device="cuda")
    k = torch.empty((B, S, Hkv, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device="cuda")
    with pytest.raises(dash.DashError) as e:
        dash.dash_attn_bwd_noalloc(q, k, k, q, q, lse, q, k, k, 0, dash.SHIFT)
    assert e.value.status == dash.DASH_ERR_WORKSPACE
    del x
