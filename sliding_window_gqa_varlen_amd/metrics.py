"""Algorithmic work and byte counts used to price a launch against the roofline.

These are counts of what the method must do, not of what a kernel happens to
touch: masked-out (query, key) pairs and invalid sparse slots are not counted,
and every tensor is read or written exactly once.

Dense (packed varlen GQA forward):
    flops = 4 * D * Hq * |allowed pairs|      (2*D for q.k, 2*D for p*v)
    bytes = q + k + v + out (+ lse + sinks + cu_seqlens)
Sparse MLA forward (latent d_l + rotary d_r keys, value = latent):
    flops = 2 * H * (d_l + d_r + d_l) * |valid slots|
    bytes = (d_l + d_r) * 2 * |valid slots| + q + indices + doc_ids + out + lse
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

# MI355X (gfx950) published peaks used as roofline denominators.
MI355X_BF16_DENSE_TFLOPS = 2500.0
MI355X_FP32_MFMA_TFLOPS = 157.3
MI355X_HBM_GBPS = 8000.0


def dense_allowed_pairs(lengths: Sequence[int], window: int) -> int:
    """(query, key) pairs a causal (window == 0) or sliding-window document mask allows.

    A token at position p of its document sees min(p + 1, window) keys, or
    p + 1 keys when window == 0.
    """
    total = 0
    for L in lengths:
        L = int(L)
        if window <= 0 or window >= L:
            total += L * (L + 1) // 2
        else:
            total += window * (window + 1) // 2 + (L - window) * window
    return total


def dense_flops(lengths: Sequence[int], window: int, Hq: int, D: int) -> int:
    return 4 * D * Hq * dense_allowed_pairs(lengths, window)


def dense_bwd_flops(lengths: Sequence[int], window: int, Hq: int, D: int) -> int:
    """Backward work per allowed pair and head: recompute q.k, then dout.v, dv, dq, dk (2 D each)."""
    return 10 * D * Hq * dense_allowed_pairs(lengths, window)


def dense_min_bytes(T: int, Hq: int, Hkv: int, D: int, elem_bytes: int, n_docs: int,
                    with_lse: bool = True, with_sinks: bool = False) -> int:
    b = elem_bytes * D * T * (2 * Hq + 2 * Hkv)
    if with_lse:
        b += 4 * T * Hq
    if with_sinks:
        b += 4 * Hq
    b += 4 * (n_docs + 1)
    return b


def dense_bwd_min_bytes(T: int, Hq: int, Hkv: int, D: int, n_docs: int, with_sinks: bool = False) -> int:
    """Backward HBM minimum (bf16): q, out, dout [T, Hq, D], k, v [T, Hkv, D] and the fp32 lse
    [T, Hq] read once; dq, dk, dv written once; cu_seqlens read, sinks read and dsinks written."""
    b = 2 * D * T * (3 * Hq + 2 * Hkv) + 4 * T * Hq
    b += 2 * D * T * (Hq + 2 * Hkv)
    b += 4 * (n_docs + 1)
    if with_sinks:
        b += 2 * 4 * Hq
    return b


def sparse_valid_slots(indices: np.ndarray, doc_ids: np.ndarray) -> int:
    """Slots that name an in-range, causal, same-document key (duplicates count per slot)."""
    T = indices.shape[0]
    t = np.arange(T, dtype=np.int64)[:, None]
    idx = indices.astype(np.int64)
    ok = (idx >= 0) & (idx < T) & (idx <= t)
    safe = np.where(ok, idx, 0)
    ok &= doc_ids[safe] == doc_ids[:, None]
    ok &= (doc_ids >= 0)[:, None]
    return int(ok.sum())


def sparse_generated_slots(lengths: Sequence[int], topk: int) -> int:
    """Valid slots of the seeded generator: min(p + 1, topk) per token."""
    total = 0
    for L in lengths:
        L = int(L)
        if L <= topk:
            total += L * (L + 1) // 2
        else:
            total += topk * (topk + 1) // 2 + (L - topk) * topk
    return total


def sparse_flops(valid_slots: int, H: int, d_latent: int, d_rope: int) -> int:
    return 2 * H * (d_latent + d_rope + d_latent) * valid_slots


def sparse_bytes(valid_slots: int, T: int, H: int, d_latent: int, d_rope: int, topk: int,
                 with_lse: bool = True) -> int:
    gather = 2 * (d_latent + d_rope) * valid_slots
    q = 2 * T * H * (d_latent + d_rope)
    out = 2 * T * H * d_latent
    idx = 4 * T * topk
    ids = 4 * T
    lse = 4 * T * H if with_lse else 0
    return gather + q + out + idx + ids + lse


def value_proj_bytes(T: int, H: int, d_latent: int, d_value: int) -> int:
    """Read o_latent and value_weight once, write out once (bf16)."""
    return 2 * (T * H * d_latent + H * d_value * d_latent + T * H * d_value)


def value_proj_flops(T: int, H: int, d_latent: int, d_value: int) -> int:
    return 2 * T * H * d_latent * d_value


def roofline(bound: str, achieved: float, peak: float, unit: str, traffic: Optional[float]) -> dict:
    return {"bound": bound, "achieved": achieved, "peak": peak, "unit": unit,
            "frac": (achieved / peak) if peak else None, "traffic": traffic}
