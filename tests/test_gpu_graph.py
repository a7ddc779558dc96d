"""GPU checks of the backward under HIP graph capture.

The library enqueues only kernels and, when AUTO resolves to the searched
table, one asynchronous host-to-device copy of that table from pinned host
memory; it records no memset and allocates nothing while enqueueing (the
first AUTO call for a shape, which searches and allocates the pinned copy,
is made before the capture).  Each case captures one backward into a graph,
replays it three times with unrelated eager work and synchronisations
between the replays, and compares every replay bit for bit with the eager
result of the same call.
"""

import sys

import pytest
import torch

import scheduling_persistent_attn_amd as dash

sys.path.insert(0, __file__.rsplit("/", 1)[0])
import gpu_util as gu  # noqa: E402

pytestmark = pytest.mark.gpu

CASES = [
    # B, S, Hq, Hkv, D, causal, schedule, entry point
    (1, 4096, 21, 3, 64, True, dash.AUTO, "workspace"),    # AUTO: the searched table on 256 CUs
    (1, 2048, 8, 2, 128, True, dash.SYMMETRIC_SHIFT, "workspace"),
    (1, 2048, 4, 4, 128, False, dash.SHIFT, "noalloc"),
    (1, 4096, 21, 3, 64, True, dash.AUTO, "noalloc"),     # AUTO among the closed forms
]


def _bits(ts):
    return [t.view(torch.int16).clone() for t in ts]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%dS%dH%d-%dD%d%s-s%d-%s" % (
    c[0], c[1], c[2], c[3], c[4], "c" if c[5] else "f", c[6], c[7]))
def test_backward_replays_bitwise(case):
    B, S, Hq, Hkv, D, causal, sched, entry = case
    mask = int(causal)
    print("graph capture", case, flush=True)
    x = gu.gpu_inputs(B, S, Hq, Hkv, D, seed=2600)
    o, lse = gu.run_forward(x, causal)
    dq, dk, dv = torch.empty_like(x["q"]), torch.empty_like(x["k"]), torch.empty_like(x["v"])
    ws = None
    if entry == "workspace":
        ws = dash.new_workspace(x["q"], x["k"], mask, sched)

    def call():
        if entry == "workspace":
            dash.dash_attn_bwd(x["q"], x["k"], x["v"], o, x["do"], lse, dq, dk, dv, mask, sched, ws)
        else:
            dash.dash_attn_bwd_noalloc(x["q"], x["k"], x["v"], o, x["do"], lse, dq, dk, dv, mask, sched)

    # eager, twice (the first call resolves AUTO and fills its cache)
    call()
    call()
    torch.cuda.synchronize()
    if ws is not None:
        dash.dash_attn_bwd_check(ws)
    ref = _bits((dq, dk, dv))

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    scratch = torch.ones(1 << 22, device="cuda")
    for r in range(3):
        for t in (dq, dk, dv):
            t.fill_(7.0)
        for _ in range(r + 1):
            scratch.mul_(1.0001)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        if ws is not None:
            dash.dash_attn_bwd_check(ws)
        for a, b in zip(ref, _bits((dq, dk, dv))):
            assert torch.equal(a, b), ("replay", r)
        # eager work between the replays: the same call outside the graph
        call()
        torch.cuda.synchronize()
        for a, b in zip(ref, _bits((dq, dk, dv))):
            assert torch.equal(a, b), ("eager after replay", r)
