"""fp64 oracle: packed variable-length causal / sliding-window GQA attention forward.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Definition followed, for every document d spanning tokens [s_d, e_d) of the
packed stream (cu_seqlens holds the padded document boundaries, as
``_build_magi_plan`` describes them on the muse_spark magi_cp page), every
token i in it and every query head h:

1. GQA: query head h reads KV head g = h // G with G = Hq // Hkv — the
   ``num_key_value_groups`` / ``repeat_kv`` mapping of MuseGlimmerAttention on
   the muse_glimmer model page (contiguous groups).
2. Mask: key j is allowed iff s_d <= j <= i and (window == 0 or i - j < window).
   Causal within the document (``SequenceLayout.allowed`` on the mistral_large4
   attention page); the window counts the current token and 0 means full
   causal (``FlintMagiPlan.attention``, window parameter, on the flint magi
   page).
3. S_j = scale * <q[i, h], k[j, g]>.
4. Z = sum_j exp(S_j) + exp(sink_h)  (the sink term only when sinks are given:
   a learned fp32 logit per query head, ``FlintMagiPlan.attention`` sink
   parameter; it joins the softmax normaliser, is not multiplied by scale and
   carries no value vector).
5. out[i, h] = sum_j exp(S_j) v[j, g] / Z ;  lse[i, h] = ln Z.

The shift by the row maximum below only avoids overflow; it cancels exactly.
Tokens outside every document (a padded tail, or before cu_seqlens[0]) get
out = 0 and lse = -inf.
"""
from __future__ import annotations

import numpy as np


def _check(q, k, v, cu_seqlens, window):
    T, Hq, D = q.shape
    assert k.shape[0] == T and v.shape[0] == T and k.shape[1] == v.shape[1]
    assert k.shape[2] == D and v.shape[2] == D
    Hkv = k.shape[1]
    assert Hkv > 0 and Hq % Hkv == 0, "query heads must be a multiple of KV heads"
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    assert cu.ndim == 1 and cu.size >= 1
    assert np.all(np.diff(cu) >= 0) and cu[0] >= 0 and cu[-1] <= T
    assert window >= 0
    return T, Hq, Hkv, D, cu


def kv_head_of(h: int, Hq: int, Hkv: int) -> int:
    """KV head serving query head h: contiguous groups of Hq // Hkv query heads."""
    return h // (Hq // Hkv)


def key_range(i0: int, i1: int, s: int, window: int):
    """Keys any query in [i0, i1) of a document starting at s may see: [lo, i1)."""
    lo = s if window == 0 else max(s, i0 - window + 1)
    return lo, i1


def allowed_block(i0: int, i1: int, lo: int, hi: int, s: int, window: int) -> np.ndarray:
    """Boolean [i1-i0, hi-lo] mask: s <= j <= i and (window == 0 or i - j < window)."""
    i = np.arange(i0, i1)[:, None]
    j = np.arange(lo, hi)[None, :]
    ok = (j >= s) & (j <= i)
    if window > 0:
        ok &= (i - j) < window
    return ok


def varlen_attn_ref(q, k, v, cu_seqlens, window: int, scale: float, sinks=None, block: int = 256):
    """fp64 out [T, Hq, D] and lse [T, Hq] of packed varlen GQA attention.

    q: [T, Hq, D]; k, v: [T, Hkv, D] (any real dtype, widened to float64);
    cu_seqlens: [n_docs + 1] non-decreasing token offsets; window: 0 = full
    causal, else keys with i - j < window; scale: score multiplier; sinks:
    optional [Hq] learned logits.
    """
    T, Hq, Hkv, D, cu = _check(q, k, v, cu_seqlens, window)
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    sk = None if sinks is None else np.asarray(sinks, dtype=np.float64)
    out = np.zeros((T, Hq, D), dtype=np.float64)
    lse = np.full((T, Hq), -np.inf, dtype=np.float64)
    for d in range(cu.size - 1):
        s, e = int(cu[d]), int(cu[d + 1])
        for i0 in range(s, e, block):
            i1 = min(i0 + block, e)
            lo, hi = key_range(i0, i1, s, window)
            ok = allowed_block(i0, i1, lo, hi, s, window)
            for h in range(Hq):
                g = kv_head_of(h, Hq, Hkv)
                S = scale * (q[i0:i1, h, :] @ k[lo:hi, g, :].T)
                S = np.where(ok, S, -np.inf)
                m = S.max(axis=1)
                if sk is not None:
                    m = np.maximum(m, sk[h])
                E = np.exp(S - m[:, None])
                Z = E.sum(axis=1)
                if sk is not None:
                    Z = Z + np.exp(sk[h] - m)
                out[i0:i1, h, :] = (E @ v[lo:hi, g, :]) / Z[:, None]
                lse[i0:i1, h] = m + np.log(Z)
    return out, lse


def varlen_attn_ref_rows(q, k, v, cu_seqlens, window: int, scale: float, sinks, tokens, heads):
    """The same definition for chosen (token, head) pairs: out [n, D], lse [n] in fp64."""
    T, Hq, Hkv, D, cu = _check(q, k, v, cu_seqlens, window)
    tokens = np.asarray(tokens, dtype=np.int64)
    heads = np.asarray(heads, dtype=np.int64)
    out = np.zeros((tokens.size, D), dtype=np.float64)
    lse = np.full(tokens.size, -np.inf, dtype=np.float64)
    for n, (i, h) in enumerate(zip(tokens.tolist(), heads.tolist())):
        d = int(np.searchsorted(cu, i, side="right")) - 1
        if d < 0 or d >= cu.size - 1 or not (cu[d] <= i < cu[d + 1]):
            continue  # padding token
        s = int(cu[d])
        lo = s if window == 0 else max(s, i - window + 1)
        g = kv_head_of(h, Hq, Hkv)
        kk = np.asarray(k[lo:i + 1, g, :], dtype=np.float64)
        vv = np.asarray(v[lo:i + 1, g, :], dtype=np.float64)
        S = scale * (kk @ np.asarray(q[i, h, :], dtype=np.float64))
        m = S.max()
        if sinks is not None:
            m = max(m, float(sinks[h]))
        E = np.exp(S - m)
        Z = E.sum()
        if sinks is not None:
            Z += np.exp(float(sinks[h]) - m)
        out[n] = (E @ vv) / Z
        lse[n] = m + np.log(Z)
    return out, lse
