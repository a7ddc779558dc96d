"""Pins of the float64 attention oracle against things other than itself.

* central finite differences of L = sum(dO * O) on tiny shapes;
* PyTorch float64 autograd of plain softmax attention on the CPU (a library
  routine for the same mathematical object);
* identities of the softmax gradient; closed forms of degenerate inputs;
* planted mistakes in the oracle must make a pin fail.
"""

import numpy as np
import pytest

from oracle import attention as oa


def _rand(shape, rng):
    return rng.standard_normal(shape)


def _loss(q, k, v, do, causal, scale=None):
    o, _ = oa.attention_forward(q, k, v, causal, scale)
    return float(np.sum(o * do))


def _fd_grad(f, x, h=1e-6):
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        idx = it.multi_index
        old = x[idx]
        x[idx] = old + h
        fp = f()
        x[idx] = old - h
        fm = f()
        x[idx] = old
        g[idx] = (fp - fm) / (2 * h)
    return g


SHAPES = [
    # B, S, Hq, Hkv, D
    (1, 1, 1, 1, 1),
    (1, 2, 1, 1, 2),
    (1, 3, 2, 1, 2),
    (1, 5, 2, 2, 4),
    (2, 8, 2, 1, 4),
    (1, 5, 4, 2, 1),
]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("causal", [False, True])
def test_finite_differences(shape, causal):
    B, S, Hq, Hkv, D = shape
    rng = np.random.default_rng(abs(hash((shape, causal))) % 2**32)
    q = _rand((B, S, Hq, D), rng)
    k = _rand((B, S, Hkv, D), rng)
    v = _rand((B, S, Hkv, D), rng)
    do = _rand((B, S, Hq, D), rng)
    dq, dk, dv = oa.attention_backward(q, k, v, do, causal)
    for x, g in ((q, dq), (k, dk), (v, dv)):
        fd = _fd_grad(lambda: _loss(q, k, v, do, causal), x)
        err = np.max(np.abs(fd - g))
        ref = max(1.0, np.max(np.abs(g)))
        assert err <= 1e-6 * ref, (err, ref)


def _torch_reference(q, k, v, do, causal, scale):
    torch = pytest.importorskip("torch")
    tq = torch.tensor(q, dtype=torch.float64, requires_grad=True)
    tk = torch.tensor(k, dtype=torch.float64, requires_grad=True)
    tv = torch.tensor(v, dtype=torch.float64, requires_grad=True)
    G = q.shape[2] // k.shape[2]
    # [B,S,H,D] -> [B,H,S,D]; expand kv heads to query heads
    qh = tq.permute(0, 2, 1, 3)
    kh = tk.permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    vh = tv.permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    sc = scale * torch.matmul(qh, kh.transpose(-1, -2).contiguous())
    if causal:
        S = q.shape[1]
        m = torch.triu(torch.ones(S, S, dtype=torch.bool), diagonal=1)
        sc = sc.masked_fill(m, float("-inf"))
    p = torch.softmax(sc, dim=-1)
    o = torch.matmul(p, vh).permute(0, 2, 1, 3)
    lse = torch.logsumexp(sc, dim=-1)
    o.backward(torch.tensor(do, dtype=torch.float64))
    return (o.detach().numpy(), lse.detach().numpy(), tq.grad.numpy(),
            tk.grad.numpy(), tv.grad.numpy())


@pytest.mark.parametrize("shape", [(1, 64, 2, 2, 16), (2, 37, 4, 2, 8),
                                   (1, 130, 6, 2, 32), (1, 1, 2, 1, 8)])
@pytest.mark.parametrize("causal", [False, True])
def test_against_torch_float64_autograd(shape, causal):
    B, S, Hq, Hkv, D = shape
    rng = np.random.default_rng(7)
    q = _rand((B, S, Hq, D), rng)
    k = _rand((B, S, Hkv, D), rng)
    v = _rand((B, S, Hkv, D), rng)
    do = _rand((B, S, Hq, D), rng)
    scale = 1.0 / np.sqrt(D)
    o_t, lse_t, dq_t, dk_t, dv_t = _torch_reference(q, k, v, do, causal, scale)
    o, lse = oa.attention_forward(q, k, v, causal)
    dq, dk, dv = oa.attention_backward(q, k, v, do, causal)
    for a, b in ((o, o_t), (lse, lse_t), (dq, dq_t), (dk, dk_t), (dv, dv_t)):
        assert np.max(np.abs(a - b)) <= 1e-12 * max(1.0, np.max(np.abs(b)))


def test_row_blocking_is_exact(monkeypatch):
    rng = np.random.default_rng(3)
    B, S, Hq, Hkv, D = 1, 50, 2, 1, 8
    q = _rand((B, S, Hq, D), rng)
    k = _rand((B, S, Hkv, D), rng)
    v = _rand((B, S, Hkv, D), rng)
    do = _rand((B, S, Hq, D), rng)
    ref = oa.attention_backward(q, k, v, do, True)
    monkeypatch.setattr(oa, "ROW_BLOCK", 7)
    got = oa.attention_backward(q, k, v, do, True)
    for a, b in zip(ref, got):
        assert np.max(np.abs(a - b)) <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_identities(causal):
    rng = np.random.default_rng(11)
    B, S, Hq, Hkv, D = 2, 24, 4, 2, 8
    G = Hq // Hkv
    q = _rand((B, S, Hq, D), rng)
    k = _rand((B, S, Hkv, D), rng)
    v = _rand((B, S, Hkv, D), rng)
    do = _rand((B, S, Hq, D), rng)
    dq, dk, dv, inter = oa.attention_backward(q, k, v, do, causal,
                                              return_intermediates=True)
    for (b, h), t in inter["per_head"].items():
        P, dP, dS = t["P"], t["dP"], t["dS"]
        assert np.allclose(P.sum(axis=1), 1.0, atol=1e-12)
        assert np.allclose(dS.sum(axis=1), 0.0, atol=1e-12)
        # Dl = rowsum(dO * O) = rowsum(P * dP)
        assert np.allclose((P * dP).sum(axis=1), inter["Dl"][b, h], atol=1e-12)
        if causal:
            assert np.all(P[np.triu_indices(S, 1)] == 0.0)
    for b in range(B):
        for kv in range(Hkv):
            hs = slice(kv * G, (kv + 1) * G)
            # sum over keys of dV = sum over queries of dO (group summed)
            assert np.allclose(dv[b, :, kv].sum(axis=0),
                               do[b, :, hs].sum(axis=(0, 1)), atol=1e-11)
            # key-translation invariance: sum over keys of dK = 0
            assert np.allclose(dk[b, :, kv].sum(axis=0), 0.0, atol=1e-11)


def test_closed_form_single_token():
    rng = np.random.default_rng(5)
    q = _rand((2, 1, 4, 8), rng)
    k = _rand((2, 1, 2, 8), rng)
    v = _rand((2, 1, 2, 8), rng)
    do = _rand((2, 1, 4, 8), rng)
    for causal in (False, True):
        o, lse = oa.attention_forward(q, k, v, causal)
        assert np.allclose(o, np.repeat(v, 2, axis=2), atol=1e-15)
        dq, dk, dv = oa.attention_backward(q, k, v, do, causal)
        assert np.all(np.abs(dq) < 1e-15) and np.all(np.abs(dk) < 1e-15)
        assert np.allclose(dv[:, :, 0], do[:, :, 0] + do[:, :, 1], atol=1e-15)
        assert np.allclose(dv[:, :, 1], do[:, :, 2] + do[:, :, 3], atol=1e-15)


def test_closed_form_causal_first_row_and_zero_q_k():
    rng = np.random.default_rng(9)
    B, S, Hq, Hkv, D = 1, 16, 2, 1, 8
    q = _rand((B, S, Hq, D), rng)
    k = _rand((B, S, Hkv, D), rng)
    v = _rand((B, S, Hkv, D), rng)
    do = _rand((B, S, Hq, D), rng)
    dq, dk, dv = oa.attention_backward(q, k, v, do, True)
    assert np.all(np.abs(dq[:, 0]) < 1e-15)
    # Q = 0: uniform attention over the visible keys; dK = 0
    zq = np.zeros_like(q)
    o, lse = oa.attention_forward(zq, k, v, True)
    for i in range(S):
        assert np.allclose(o[0, i, 0], v[0, :i + 1, 0].mean(axis=0), atol=1e-13)
        assert abs(lse[0, 0, i] - np.log(i + 1)) < 1e-13
    _, dk0, _ = oa.attention_backward(zq, k, v, do, True)
    assert np.max(np.abs(dk0)) < 1e-13
    # K = 0: scores are constant, dQ = 0
    zk = np.zeros_like(k)
    dq0, _, _ = oa.attention_backward(q, zk, v, do, False)
    assert np.max(np.abs(dq0)) < 1e-13


def test_empty_sequence():
    q = np.zeros((1, 0, 2, 8))
    k = np.zeros((1, 0, 1, 8))
    o, lse = oa.attention_forward(q, k, k, True)
    assert o.shape == (1, 0, 2, 8) and lse.shape == (1, 2, 0)
    dq, dk, dv = oa.attention_backward(q, k, k, q, True)
    assert dq.shape == q.shape and dk.shape == k.shape


# --- planted mistakes: each must be caught by one of the pins above ---------

def _fd_fails(monkeypatch_target=None):
    rng = np.random.default_rng(1)
    B, S, Hq, Hkv, D = 1, 4, 2, 1, 3
    q = _rand((B, S, Hq, D), rng)
    k = _rand((B, S, Hkv, D), rng)
    v = _rand((B, S, Hkv, D), rng)
    do = _rand((B, S, Hq, D), rng)
    dq, dk, dv = oa.attention_backward(q, k, v, do, True)
    worst = 0.0
    for x, g in ((q, dq), (k, dk), (v, dv)):
        fd = _fd_grad(lambda: _loss(q, k, v, do, True), x)
        worst = max(worst, np.max(np.abs(fd - g)))
    return worst > 1e-6


def test_planted_dropped_delta_is_caught(monkeypatch):
    orig = oa.delta
    monkeypatch.setattr(oa, "delta", lambda o, do: 0.0 * orig(o, do))
    assert _fd_fails()


def test_planted_wrong_mask_direction_is_caught(monkeypatch):
    def bad_scores(qb, kh, row0, scale, causal):
        sc = scale * (qb @ kh.T)
        if causal:
            rows = np.arange(row0, row0 + qb.shape[0])[:, None]
            cols = np.arange(kh.shape[0])[None, :]
            sc = np.where(cols < rows, -np.inf, sc)
        return sc
    assert not _fd_fails()
    rng = np.random.default_rng(2)
    q = _rand((1, 6, 1, 4), rng)
    k = _rand((1, 6, 1, 4), rng)
    v = _rand((1, 6, 1, 4), rng)
    do = _rand((1, 6, 1, 4), rng)
    good = oa.attention_backward(q, k, v, do, True)
    monkeypatch.setattr(oa, "_scores", bad_scores)
    bad = oa.attention_backward(q, k, v, do, True)
    # the closed form "dQ of causal row 0 is zero" no longer holds
    assert np.max(np.abs(bad[0][:, 0])) > 1e-6 or np.max(np.abs(bad[1] - good[1])) > 1e-6


# --- the sampled form used by the full-size GPU tests ------------------------
#
# attention_backward_sampled(kv_heads=[kv]) must equal, element by element, the
# slices of the whole-problem attention_backward that belong to key/value head
# kv: dq of query heads kv*G .. kv*G+G-1, dk and dv of head kv, for every batch
# entry.  attention_backward itself is pinned above (finite differences,
# torch autograd), so this pins the sampled form to them.

def _sampled_mismatch(sampled_fn, causal, rows=None):
    rng = np.random.default_rng(11)
    B, S, Hq, Hkv, D = 2, 9, 6, 2, 4
    G = Hq // Hkv
    q = _rand((B, S, Hq, D), rng)
    k = _rand((B, S, Hkv, D), rng)
    v = _rand((B, S, Hkv, D), rng)
    do = _rand((B, S, Hq, D), rng)
    dq, dk, dv = oa.attention_backward(q, k, v, do, causal)
    got = sampled_fn(q, k, v, do, causal, list(range(Hkv)), q_rows=rows)
    worst = 0.0
    for kv in range(Hkv):
        sdq, sdk, sdv = got[kv]
        want_dq = dq[:, :, kv * G:(kv + 1) * G]
        if rows is not None:
            want_dq = want_dq[:, rows]
        if sdq.shape != want_dq.shape or sdk.shape != dk[:, :, kv].shape:
            return float("inf")
        worst = max(worst, np.max(np.abs(sdq - want_dq)), np.max(np.abs(sdk - dk[:, :, kv])),
                    np.max(np.abs(sdv - dv[:, :, kv])))
    return worst


@pytest.mark.parametrize("causal", [False, True])
def test_sampled_equals_whole_problem(causal):
    assert _sampled_mismatch(oa.attention_backward_sampled, causal) < 1e-12
    assert _sampled_mismatch(oa.attention_backward_sampled, causal, rows=[0, 4, 8]) < 1e-12


def test_planted_sampled_head_mistakes_are_caught():
    # every key/value head served by head 0's data
    def kv0(q, k, v, do, causal, kv_heads, q_rows=None):
        r = oa.attention_backward_sampled(q, k, v, do, causal, [0], q_rows=q_rows)
        return {kv: r[0] for kv in kv_heads}

    # the query heads of key/value head kv taken as kv .. kv+G-1
    def shifted_heads(q, k, v, do, causal, kv_heads, q_rows=None):
        G = q.shape[2] // k.shape[2]
        out = {}
        for kv in kv_heads:
            hs = list(range(kv, kv + G))
            r = oa.attention_backward_sampled(q[:, :, hs], k[:, :, kv:kv + 1], v[:, :, kv:kv + 1],
                                              do[:, :, hs], causal, [0], q_rows=q_rows)
            out[kv] = r[0]
        return out

    for fn in (kv0, shifted_heads):
        assert _sampled_mismatch(fn, True) > 1e-6
