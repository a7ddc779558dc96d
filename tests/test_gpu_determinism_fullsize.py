"""Run-to-run bit identity at the full workload sizes, 20 runs per schedule.

Every deterministic schedule (and AUTO where it resolves to the searched
task table) of the four large workloads (an 8B-Llama-shaped
causal layer, a diffusion/vision full-mask block, a 16k full-mask layer and a
7B-Qwen-shaped 16k causal layer) runs 20 times on the whole problem in the
launch configuration the benchmark times.  The runs rotate over three streams
behind a seeded random amount of unrelated work, and every other run starts
while a kernel on a fourth stream occupies compute units, so workgroups take
items and reach the ordered reductions in different orders and places.  dq,
dk and dv must not change by a bit (bitwise reproducibility is the point of
the method: DASH technical summary, section 1).  The check stops at the first
differing run.  This also guards the counted memory waits that order each
hand-off: a miscounted wait would show up as a rare differing run here.
"""

import random
import sys

import pytest
import torch

import scheduling_persistent_attn_amd as dash

sys.path.insert(0, __file__.rsplit("/", 1)[0])
import gpu_util as gu  # noqa: E402

pytestmark = pytest.mark.gpu

RUNS = 20

WORKLOADS = {
    # name: (B, S, Hq, Hkv, D, causal)
    "llama8b_causal": (4, 4096, 32, 8, 128, True),
    "dit_full": (2, 4096, 24, 24, 64, False),
    "long_full": (1, 16384, 32, 32, 128, False),
    "qwen7b_causal": (1, 16384, 28, 4, 128, True),
}


def _schedules(causal, N, shape):
    out = [dash.NAIVE, dash.DESCENDING_Q, dash.SHIFT]
    if causal and N % 2 == 0:
        out.append(dash.SYMMETRIC_SHIFT)
    # AUTO where it runs the searched task table
    B, Hq, Hkv, S, D = shape
    if dash.dash_attn_bwd_auto_schedule(B, Hq, Hkv, S, D, int(causal)) == dash.TABLE:
        out.append(dash.AUTO)
    return out


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_fullsize_bit_identical_over_20_runs(name):
    B, S, Hq, Hkv, D, causal = WORKLOADS[name]
    T = dash.dash_attn_tile_size(S, D)
    N = (S + T - 1) // T
    print("fullsize determinism", name, flush=True)
    x = gu.gpu_inputs(B, S, Hq, Hkv, D, seed=3000)
    o, lse = gu.run_forward(x, causal)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(3)]
    busy = torch.cuda.Stream()
    filler = torch.ones(1 << 22, device="cuda")
    big = torch.ones(1 << 27, device="cuda")  # 512 MiB: about a millisecond per pass
    dq = torch.empty_like(x["q"])
    dk = torch.empty_like(x["k"])
    dv = torch.empty_like(x["v"])
    for sched in _schedules(causal, N, (B, Hq, Hkv, S, D)):
        print("  schedule", sched, flush=True)
        rng = random.Random(4321 + sched)
        ws = dash.new_workspace(x["q"], x["k"], int(causal), sched)
        ref = None
        for n in range(RUNS):
            s = streams[n % 3]
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                for _ in range(rng.randint(0, 6)):
                    filler.mul_(1.0001)
            if n % 2:
                busy.wait_stream(torch.cuda.current_stream())
                with torch.cuda.stream(busy):
                    for _ in range(2):
                        big.mul_(1.0001)
            dash.dash_attn_bwd(x["q"], x["k"], x["v"], o, x["do"], lse, dq, dk, dv, int(causal),
                               sched, ws, stream=s)
            dash.dash_attn_bwd_check(ws, stream=s)
            torch.cuda.current_stream().wait_stream(s)
            torch.cuda.current_stream().wait_stream(busy)
            bits = [t.view(torch.int16) for t in (dq, dk, dv)]
            if ref is None:
                ref = [b.clone() for b in bits]
                continue
            same = all(torch.equal(a, b) for a, b in zip(ref, bits))
            assert same, "%s schedule %d: run %d differs from run 0" % (name, sched, n)
        print("    %d runs bit-identical" % RUNS, flush=True)
        del ws
