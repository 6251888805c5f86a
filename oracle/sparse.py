"""fp64 oracle: sparse MLA forward over gathered top-k latent rows — TEST INFRASTRUCTURE ONLY.

Definition followed (``sparse_mla`` and ``MistralLarge4Attention._sparse_forward``
on the mistral_large4 attention page): each query token t has H heads of
dimension d_l + d_r (latent part first, rotary part last), every key is one
shared row: latent[idx] (d_l) with rotary k_pe[idx] (d_r), and the value is
the latent row itself (the KV-B value up-projection is not applied here).

For token t and head h, over the slots r of indices[t]:

1. Slot r is valid iff idx = indices[t, r] is in [0, T), idx <= t and
   doc_ids[idx] == doc_ids[t] (and t itself belongs to a document,
   doc_ids[t] >= 0).  -1 marks an empty slot.  The page leaves the
   document/causal boundary to the caller; checking it here too makes both
   sides agree on inputs that break that contract.
2. S_r = scale * (<q[t,h,:d_l], latent[idx]> + <q[t,h,d_l:], k_pe[idx]>).
3. out[t,h] = sum_r softmax(S)_r latent[idx_r];  lse[t,h] = ln sum_r exp(S_r).
4. No valid slot: out = 0, lse = -inf (empty query rows are zero).

Slots count one by one: an index repeated in a row contributes twice.
"""
from __future__ import annotations

import numpy as np


def slot_validity(indices, doc_ids, t: int) -> np.ndarray:
    """bool mask over the slots of row t (rule 1 above)."""
    T = doc_ids.shape[0]
    idx = np.asarray(indices[t], dtype=np.int64)
    if doc_ids[t] < 0:
        return np.zeros(idx.shape, dtype=bool)
    ok = (idx >= 0) & (idx < T) & (idx <= t)
    safe = np.where(ok, idx, 0)
    ok &= np.asarray(doc_ids)[safe] == doc_ids[t]
    return ok


def _one_token(q, latent, k_pe, indices, doc_ids, scale, t, d_l):
    ok = slot_validity(indices, doc_ids, t)
    sel = np.asarray(indices[t], dtype=np.int64)[ok]
    H = q.shape[1]
    if sel.size == 0:
        return np.zeros((H, d_l)), np.full(H, -np.inf)
    qt = np.asarray(q[t], dtype=np.float64)
    lat = np.asarray(latent[sel], dtype=np.float64)           # [n, d_l]
    rope = np.asarray(k_pe[sel], dtype=np.float64)            # [n, d_r]
    S = scale * (qt[:, :d_l] @ lat.T + qt[:, d_l:] @ rope.T)   # [H, n]
    m = S.max(axis=1, keepdims=True)
    E = np.exp(S - m)
    Z = E.sum(axis=1)
    return (E @ lat) / Z[:, None], m[:, 0] + np.log(Z)


def sparse_mla_ref(q, latent, k_pe, indices, doc_ids, scale: float):
    """fp64 out [T, H, d_l] and lse [T, H]."""
    T, H, dqk = q.shape
    d_l = latent.shape[1]
    assert k_pe.shape[0] == T and latent.shape[0] == T and dqk == d_l + k_pe.shape[1]
    out = np.zeros((T, H, d_l))
    lse = np.full((T, H), -np.inf)
    doc_ids = np.asarray(doc_ids)
    for t in range(T):
        out[t], lse[t] = _one_token(q, latent, k_pe, indices, doc_ids, scale, t, d_l)
    return out, lse


def sparse_mla_ref_rows(q, latent, k_pe, indices, doc_ids, scale: float, tokens):
    """The same definition for chosen tokens only: out [n, H, d_l], lse [n, H]."""
    d_l = latent.shape[1]
    doc_ids = np.asarray(doc_ids)
    outs, lses = [], []
    for t in np.asarray(tokens, dtype=np.int64).tolist():
        o, l = _one_token(q, latent, k_pe, indices, doc_ids, scale, t, d_l)
        outs.append(o)
        lses.append(l)
    return np.stack(outs), np.stack(lses)


def mla_value_proj_ref(o_latent, value_weight):
    """fp64 out_v [T, H, d_v] with out_v[t, h] = value_weight[h] @ o_latent[t, h].

    The KV-B value up-projection that ``sparse_mla`` on the mistral_large4
    attention page applies to the attention output over latent rows: its
    value_weight is [heads, value_dim, 512] and it returns [tokens, heads,
    value_dim].  Empty query rows (o_latent = 0) stay zero.
    """
    o = np.asarray(o_latent, dtype=np.float64)
    w = np.asarray(value_weight, dtype=np.float64)
    T, H, d_l = o.shape
    assert w.shape[0] == H and w.shape[2] == d_l
    out = np.empty((T, H, w.shape[1]))
    for h in range(H):
        out[:, h, :] = o[:, h, :] @ w[h].T
    return out


def sparse_mla_value_ref(q, latent, k_pe, indices, doc_ids, value_weight, scale: float):
    """``sparse_mla`` as the page states it: attention over gathered latent rows, then the
    value up-projection.  Returns out_v [T, H, d_v] and lse [T, H]."""
    o, lse = sparse_mla_ref(q, latent, k_pe, indices, doc_ids, scale)
    return mla_value_proj_ref(o, value_weight), lse
