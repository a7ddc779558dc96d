"""Helpers shared by the GPU tests (not collected: no test_ prefix)."""

import numpy as np
import torch

import scheduling_persistent_attn_amd as dash
from scheduling_persistent_attn_amd.inputs import as_float64, make_inputs

# Tolerance of the backward against the float64 oracle (bf16 inputs, fp32
# accumulation, bf16 outputs): rel-L2 <= 1e-2 and an absolute error of at most
# 2e-2 beyond the rounding of the output to bf16 itself.  Round-to-nearest to
# bf16 (8 significant bits) moves a value x by at most 2^-8 |x|, which alone
# exceeds 2e-2 once |x| > 5.12, so the absolute bar is applied to
# |got - ref| - 2^-8 |ref|.
REL_L2 = 1e-2
MAX_ABS = 2e-2
BF16_HALF_ULP_REL = 2.0 ** -8


def rel_l2(a, b):
    den = np.linalg.norm(b.ravel())
    return np.linalg.norm((a - b).ravel()) / (den if den > 0 else 1.0)


def errors(got, ref):
    """(rel-L2, max-abs beyond bf16 output rounding, plain max-abs)."""
    if not ref.size:
        return 0.0, 0.0, 0.0
    d = np.abs(got - ref)
    return (rel_l2(got, ref), float(np.max(d - BF16_HALF_ULP_REL * np.abs(ref))),
            float(np.max(d)))


def within(e):
    return e[0] <= REL_L2 and e[1] <= MAX_ABS


def run_forward(x, causal):
    o, lse = dash.forward(x["q"], x["k"], x["v"], causal)
    return o, lse


def run_backward(x, o, lse, causal, schedule, workspace=None, stream=None, check=True):
    return dash.backward(x["q"], x["k"], x["v"], o, x["do"], lse, causal, schedule, check=check,
                         workspace=workspace, stream=stream)


def gpu_inputs(B, S, Hq, Hkv, D, seed=1000):
    return make_inputs(B, S, Hq, Hkv, D, seed=seed, device="cuda")


def host64(t):
    return as_float64(t)


def contributors(causal, N, j):
    return j + 1 if causal else N


def slices_per_tile(T, D):
    """Turn counters per dQ tile: one per slice a wave reduces per pass (32 x
    32 for tiles of 64 and 128 rows, 32 x 16 for 256)."""
    return T * D // 512 if T == 256 else T * D // 1024


def expected_counters(B, Hq, S, D, causal):
    T = dash.dash_attn_tile_size(S, D)
    N = (S + T - 1) // T
    NW = slices_per_tile(T, D)
    want = np.zeros((B, Hq, N, NW), dtype=np.int64)
    for j in range(N):
        want[:, :, j, :] = contributors(causal, N, j)
    return want


def read_counters(workspace, B, Hq, S, D):
    T = dash.dash_attn_tile_size(S, D)
    N = (S + T - 1) // T
    NW = slices_per_tile(T, D)
    n = B * Hq * N * NW
    # after the 64 control words and the 4096 x 4 uint64 wait counters
    off = (256 + 4096 * 32) // 4
    ws = workspace.view(torch.int32)
    return ws[off:off + n].cpu().numpy().reshape(B, Hq, N, NW)
