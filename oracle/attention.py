"""Float64 softmax attention forward and backward (oracle; test infrastructure only).

Definition followed (textbook scaled-dot-product attention; the DASH pages fix
only that the dQ accumulation order must be fixed -- DASH technical summary,
section 1 "Problem statement" -- and leave the equations to the standard
FlashAttention backward):

    Sc  = s * Q K^T                      (s = 1/sqrt(D) unless given)
    Sc[i, j] = -inf  where causal and key j > query i
    LSE_i = log sum_j exp(Sc_ij)         (natural log)
    P   = exp(Sc - LSE)
    O   = P V
    dV  = P^T dO
    dP  = dO V^T
    Dl_i = sum_d dO_id O_id
    dS  = P * (dP - Dl)
    dQ  = s * dS K
    dK  = s * dS^T Q

Layouts: q, o, do are [B, S, Hq, D]; k, v are [B, S, Hkv, D]; lse is
[B, Hq, S].  Query head h reads key/value head h // (Hq // Hkv); dK and dV of
a key/value head are the sums over the Hq // Hkv query heads that read it.

All arithmetic is float64.  Rows are independent, so the row blocking below
(to bound memory at long sequence lengths) does not change the definition;
dK and dV are float64 sums over the row blocks.
"""

import numpy as np

ROW_BLOCK = 1024


def _check(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, S, H, D]")
    B, S, Hq, D = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[1] != S or k.shape[3] != D:
        raise ValueError("k, v must be [B, S, Hkv, D] matching q")
    Hkv = k.shape[2]
    if Hkv == 0 or Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    return B, S, Hq, Hkv, D


def _scores(qb, kh, row0, scale, causal):
    """Scaled scores of query rows row0.. against all keys, masked."""
    sc = scale * (qb @ kh.T)
    if causal:
        rows = np.arange(row0, row0 + qb.shape[0])[:, None]
        cols = np.arange(kh.shape[0])[None, :]
        sc = np.where(cols > rows, -np.inf, sc)
    return sc


def attention_forward(q, k, v, causal, scale=None):
    """Return (o, lse) in float64; o is [B,S,Hq,D], lse is [B,Hq,S]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, S, Hq, Hkv, D = _check(q, k, v)
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D) if D > 0 else 1.0
    o = np.zeros((B, S, Hq, D))
    lse = np.zeros((B, Hq, S))
    for b in range(B):
        for h in range(Hq):
            kh = k[b, :, h // G, :]
            vh = v[b, :, h // G, :]
            for r0 in range(0, S, ROW_BLOCK):
                qb = q[b, r0:r0 + ROW_BLOCK, h, :]
                sc = _scores(qb, kh, r0, scale, causal)
                m = sc.max(axis=1, keepdims=True)
                e = np.exp(sc - m)
                l = e.sum(axis=1, keepdims=True)
                lse[b, h, r0:r0 + qb.shape[0]] = (m + np.log(l))[:, 0]
                o[b, r0:r0 + qb.shape[0], h, :] = (e / l) @ vh
    return o, lse


def delta(o, do):
    """Dl[b, h, i] = sum_d dO[b,i,h,d] * O[b,i,h,d]  -> [B, Hq, S]."""
    o = np.asarray(o, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    return np.einsum("bshd,bshd->bhs", do, o)


def attention_backward(q, k, v, do, causal, scale=None, o=None, lse=None,
                       return_intermediates=False):
    """Return (dq, dk, dv) in float64 with the layouts of q, k, v.

    If ``o``/``lse`` are not given they are computed here in float64.  With
    ``return_intermediates`` (small shapes only) also returns a dict with the
    full P, dP, dS per (b, h) and the row vector Dl.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, S, Hq, Hkv, D = _check(q, k, v)
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D) if D > 0 else 1.0
    if o is None or lse is None:
        o, lse = attention_forward(q, k, v, causal, scale)
    o = np.asarray(o, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    dl = delta(o, do)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    inter = {}
    for b in range(B):
        for h in range(Hq):
            kv = h // G
            kh = k[b, :, kv, :]
            vh = v[b, :, kv, :]
            for r0 in range(0, S, ROW_BLOCK):
                r1 = min(S, r0 + ROW_BLOCK)
                qb = q[b, r0:r1, h, :]
                dob = do[b, r0:r1, h, :]
                sc = _scores(qb, kh, r0, scale, causal)
                p = np.exp(sc - lse[b, h, r0:r1][:, None])
                dv[b, :, kv, :] += p.T @ dob
                dp = dob @ vh.T
                ds = p * (dp - dl[b, h, r0:r1][:, None])
                dq[b, r0:r1, h, :] = scale * (ds @ kh)
                dk[b, :, kv, :] += scale * (ds.T @ qb)
                if return_intermediates:
                    inter.setdefault((b, h), []).append((p, dp, ds))
    if return_intermediates:
        full = {}
        for key, parts in inter.items():
            full[key] = {
                "P": np.concatenate([x[0] for x in parts], axis=0),
                "dP": np.concatenate([x[1] for x in parts], axis=0),
                "dS": np.concatenate([x[2] for x in parts], axis=0),
            }
        return dq, dk, dv, {"per_head": full, "Dl": dl, "o": o, "lse": lse}
    return dq, dk, dv


def attention_backward_sampled(q, k, v, do, causal, kv_heads, q_rows=None,
                               scale=None):
    """Oracle gradients restricted to the query heads of the given kv heads.

    Returns dict kv_head -> (dq_rows [len(rows) or S, G, D], dk [S, D],
    dv [S, D]) for batch entries stacked on axis 0 of each array: the arrays
    are [B, ...].  Everything is computed from the definition above for the
    G query heads that read each listed kv head, so dk/dv are complete for
    those kv heads.  ``q_rows`` (optional) limits the returned dq rows.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, S, Hq, Hkv, D = _check(q, k, v)
    G = Hq // Hkv
    out = {}
    for kv in kv_heads:
        hs = list(range(kv * G, (kv + 1) * G))
        qs = q[:, :, hs, :]
        dos = do[:, :, hs, :]
        ks = k[:, :, kv:kv + 1, :]
        vs = v[:, :, kv:kv + 1, :]
        dq, dk, dv = attention_backward(qs, ks, vs, dos, causal, scale)
        if q_rows is not None:
            dq = dq[:, q_rows]
        out[kv] = (dq, dk[:, :, 0, :], dv[:, :, 0, :])
    return out
