"""Brute-force second path for the dense oracle — TEST INFRASTRUCTURE ONLY.

Builds the whole [T, T] mask from per-token metadata, the way
``SequenceLayout.allowed`` on the mistral_large4 attention page describes a
causal document mask (document ids and positions per token), with the sliding
window of ``FlintMagiPlan.attention`` (flint magi page) counted inclusive of
the current token.  The softmax is then taken over a row of T scores plus one
extra "sink" column whose value vector is zero, instead of adding a term to
the normaliser.  Tiny inputs only (T up to a few hundred).
"""
from __future__ import annotations

import numpy as np


def doc_ids_and_positions(cu_seqlens, T: int):
    """Per-token document id (-1 outside every document) and position in it."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    doc = np.full(T, -1, dtype=np.int64)
    pos = np.zeros(T, dtype=np.int64)
    for d in range(cu.size - 1):
        for t in range(int(cu[d]), int(cu[d + 1])):
            doc[t] = d
            pos[t] = t - int(cu[d])
    return doc, pos


def allowed_matrix(cu_seqlens, T: int, window: int) -> np.ndarray:
    """bool [T, T]: row i may attend column j."""
    doc, pos = doc_ids_and_positions(cu_seqlens, T)
    A = np.zeros((T, T), dtype=bool)
    for i in range(T):
        for j in range(T):
            if doc[i] < 0 or doc[i] != doc[j]:
                continue
            if pos[j] > pos[i]:
                continue
            if window and pos[i] - pos[j] >= window:
                continue
            A[i, j] = True
    return A


def varlen_attn_bruteforce(q, k, v, cu_seqlens, window: int, scale: float, sinks=None):
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    rep = Hq // Hkv
    A = allowed_matrix(cu_seqlens, T, window)
    doc, _ = doc_ids_and_positions(cu_seqlens, T)
    out = np.zeros((T, Hq, D))
    lse = np.full((T, Hq), -np.inf)
    for h in range(Hq):
        kh = np.repeat(k, rep, axis=1)[:, h, :]   # repeat_kv, then pick head h
        vh = np.repeat(v, rep, axis=1)[:, h, :]
        scores = scale * q[:, h, :] @ kh.T       # [T, T]
        sink_col = np.full((T, 1), -np.inf if sinks is None else float(sinks[h]))
        logits = np.concatenate([np.where(A, scores, -np.inf), sink_col], axis=1)
        vals = np.concatenate([vh, np.zeros((1, D))], axis=0)
        for i in range(T):
            if doc[i] < 0:
                continue  # padding token: not a query (out 0, lse -inf)
            row = logits[i]
            if not np.isfinite(row).any():
                continue
            mx = row[np.isfinite(row)].max()
            w = np.exp(row - mx)
            out[i, h] = (w @ vals) / w.sum()
            lse[i, h] = mx + np.log(w.sum())
    return out, lse
