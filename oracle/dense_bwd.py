"""fp64 oracle: backward of packed varlen causal / sliding-window GQA attention.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages print no backward formulas.  ``MuseMagiPlan.attention`` on the
muse_spark magi_cp page returns only the attention output (no log-sum-exp);
``sparse_mla`` on the mistral_large4 attention page calls its value weight
differentiable, and ``MistralLarge4Attention.forward`` keeps a shared KV that is
never detached, so gradients flow through attention.  The gradient of a loss L that depends on ``out`` is the unique
derivative of the forward definition (``dense.varlen_attn_ref``), so this
module writes it out by the chain rule.  For every document [s, e), query token
i in it, query head h with KV head g = h // G, and allowed keys j
(s <= j <= i, and i - j < window when window > 0):

    S_ij   = scale * <q[i, h], k[j, g]>
    Z_i    = sum_j exp(S_ij) + exp(sink_h)           (sink term only with sinks)
    P_ij   = exp(S_ij) / Z_i ;  p_sink_i = exp(sink_h) / Z_i
    out_i  = sum_j P_ij v[j, g]

    dP_ij  = <dout[i, h], v[j, g]>
    delta_i = sum_j P_ij dP_ij  (= <dout[i, h], out[i, h]>)
    dS_ij  = P_ij (dP_ij - delta_i)
    dq[i, h]  = scale * sum_j dS_ij k[j, g]
    dk[j, g] += scale * sum_{i, h in group g} dS_ij q[i, h]
    dv[j, g] += sum_{i, h in group g} P_ij dout[i, h]
    dsink[h]  = - sum_i p_sink_i delta_i

(The sink joins Z but carries no value, so d out_i / d sink_h = -p_sink_i out_i.)
Tokens outside every document neither receive nor pass gradient.  Only the
gradient through ``out`` is taken; ``lse`` is treated as an auxiliary output.
"""
from __future__ import annotations

import numpy as np

from .dense import _check, allowed_block, key_range, kv_head_of


def varlen_attn_bwd_ref(q, k, v, dout, cu_seqlens, window: int, scale: float, sinks=None, block: int = 256):
    """fp64 (dq [T, Hq, D], dk [T, Hkv, D], dv [T, Hkv, D], dsink [Hq] or None, delta [T, Hq]).

    Arguments as ``varlen_attn_ref`` plus dout [T, Hq, D] = dL/dout.  delta is
    the per-row <dout, out> of the definition (0 on padding tokens).
    """
    T, Hq, Hkv, D, cu = _check(q, k, v, cu_seqlens, window)
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(dout, dtype=np.float64)
    assert do.shape == q.shape
    sk = None if sinks is None else np.asarray(sinks, dtype=np.float64)
    dq = np.zeros((T, Hq, D))
    dk = np.zeros((T, Hkv, D))
    dv = np.zeros((T, Hkv, D))
    dsink = None if sk is None else np.zeros(Hq)
    delta = np.zeros((T, Hq))
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
                P = E / Z[:, None]
                dP = do[i0:i1, h, :] @ v[lo:hi, g, :].T
                dl = (P * dP).sum(axis=1)
                dS = P * (dP - dl[:, None])
                dq[i0:i1, h, :] = scale * (dS @ k[lo:hi, g, :])
                dk[lo:hi, g, :] += scale * (dS.T @ q[i0:i1, h, :])
                dv[lo:hi, g, :] += P.T @ do[i0:i1, h, :]
                delta[i0:i1, h] = dl
                if sk is not None:
                    dsink[h] -= (np.exp(sk[h] - m) / Z * dl).sum()
    return dq, dk, dv, dsink, delta
