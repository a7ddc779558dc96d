"""Seeded synthetic inputs (shared by tests, the smoke check and the bench).

Holds none of the attention arithmetic: it only draws N(0, 1) float32
samples from fixed seeds and rounds them to bfloat16 (round to nearest even).
Seeds: Q = seed, K = seed + 1, V = seed + 2, dO = seed + 3.
Layouts: q, do [B, S, Hq, D]; k, v [B, S, Hkv, D]; contiguous.
"""

import torch


def _randn(shape, seed):
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float32).to(torch.bfloat16)


def make_inputs(B, S, Hq, Hkv, D, seed=1000, device="cpu"):
    """Return dict q, k, v, do of bfloat16 tensors on ``device``."""
    out = {
        "q": _randn((B, S, Hq, D), seed),
        "k": _randn((B, S, Hkv, D), seed + 1),
        "v": _randn((B, S, Hkv, D), seed + 2),
        "do": _randn((B, S, Hq, D), seed + 3),
    }
    if device != "cpu":
        out = {k: t.to(device) for k, t in out.items()}
    return out


def as_float64(t):
    """Exact float64 numpy copy of a (bfloat16) tensor."""
    return t.detach().to("cpu", torch.float32).double().numpy()
