"""Seeded synthetic inputs for packed varlen attention (dense GQA and sparse MLA).

This module only draws random numbers and lays them out; it holds none of the
attention arithmetic.  Both the fp64 oracle (through the tests and the bench's
CPU leg) and the HIP path consume exactly the arrays produced here, so the two
sides see identical input values.

Recipe (fixed so runs reproduce):

* ``rng = numpy.random.default_rng(seed)`` draws the document lengths first:
  lengths are drawn until they cover ``T`` tokens and the last one is
  truncated.  "uniform" lengths use ``rng.integers(a, b, endpoint=True)``;
  "loguniform" lengths use ``round(exp(rng.uniform(ln a, ln b)))`` clipped to
  ``[a, b]``.  Packed document lengths per pack follow the
  ``prepare_magi_inputs`` batch description on the muse_spark magi_cp page.
* Every tensor then comes from its own stream ``default_rng([seed, stream])``
  (q=1, k=2, v=3, sinks=4, indices=5, latent=6, k_pe=7, value_weight=8, dout=9), so a
  tensor can be regenerated without drawing the others.  Values are standard
  normal float32; the sparse value weight is scaled by 1/sqrt(d_latent) (the
  usual fan-in initialisation) so its outputs stay of unit order.
* Configuration "sliding window, RMS-normalised q/k" applies the parameter-free
  RMS normalisation (MuseGlimmerScalelessRMSNorm on the muse_glimmer model
  page, eps 1e-5) over head_dim to q and k before rounding.
* bf16 workloads round every floating input to bfloat16 with round-to-nearest-
  even and hand them out as float32 arrays holding bf16-exact values (so the
  widening to fp64 in the oracle and to torch.bfloat16 on the GPU is exact).
* Sparse indices: for a token at position p of its document, all p+1 causal
  same-document keys are taken when p+1 <= topk; otherwise ``topk`` distinct
  keys are drawn with ``rng.choice(p + 1, topk, replace=False)``.  The document
  start is added, each row is sorted ascending (the ascending-key tie-breaking
  of MistralLarge4Indexer.forward on the mistral_large4 attention page) and
  padded with -1 at the tail.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np

STREAM_Q, STREAM_K, STREAM_V, STREAM_SINK, STREAM_IDX, STREAM_LATENT, STREAM_KPE, STREAM_VW, STREAM_DOUT = \
    1, 2, 3, 4, 5, 6, 7, 8, 9


# ---------------------------------------------------------------------------
# workload descriptions
# ---------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class DenseWorkload:
    """One packed varlen GQA problem (the forward, or with ``backward`` its gradients)."""

    name: str
    dtype: str  # "f32" or "bf16"
    T: int
    Hq: int
    Hkv: int
    D: int
    window: int
    scale: float
    seed: int
    doc_lengths: Optional[tuple] = None  # fixed lengths (sum <= T); else drawn
    doc_dist: Optional[tuple] = None  # ("uniform"|"loguniform", a, b)
    rms_norm_qk: bool = False
    sinks: bool = False
    backward: bool = False  # measure varlen_attn_bwd (dout from stream 9) instead of the forward

    def with_tokens(self, T: int, name: Optional[str] = None) -> "DenseWorkload":
        """Same recipe at another token count (document lengths capped at T)."""
        dist = self.doc_dist
        if dist is not None:
            kind, a, b = dist
            b = min(b, T)
            a = min(a, b)
            dist = (kind, a, b)
        return dataclasses.replace(self, T=T, doc_dist=dist, name=name or f"{self.name}@T{T}")


@dataclasses.dataclass(frozen=True)
class SparseWorkload:
    """One sparse MLA forward problem (latent 512 + rotary 64 keys, top-k gather)."""

    name: str
    T: int
    H: int
    d_latent: int
    d_rope: int
    topk: int
    scale: float
    seed: int
    doc_dist: tuple = ("uniform", 1024, 8192)
    doc_lengths: Optional[tuple] = None

    @property
    def d_qk(self) -> int:
        return self.d_latent + self.d_rope

    def with_tokens(self, T: int, topk: Optional[int] = None, name: Optional[str] = None) -> "SparseWorkload":
        kind, a, b = self.doc_dist
        b = min(b, T)
        a = min(a, b)
        return dataclasses.replace(self, T=T, topk=topk or self.topk, doc_dist=(kind, a, b),
                                   name=name or f"{self.name}@T{T}")


# The five workloads the method is measured on.  Seeds equal the list index.
WORKLOADS = (
    DenseWorkload("tiny_causal_gqa_f32", "f32", T=64, Hq=4, Hkv=2, D=64, window=0, scale=1.0 / 8.0,
                  seed=0, doc_lengths=(5, 17, 42)),
    DenseWorkload("causal_gqa_bf16_t8192", "bf16", T=8192, Hq=32, Hkv=8, D=128, window=0,
                  scale=1.0 / math.sqrt(128.0), seed=1, doc_dist=("uniform", 128, 2048)),
    DenseWorkload("swa1024_gqa_bf16_t32768", "bf16", T=32768, Hq=32, Hkv=4, D=128, window=1024,
                  scale=1.0 / math.sqrt(128.0), seed=2, doc_dist=("uniform", 512, 8192), rms_norm_qk=True),
    DenseWorkload("swa128_sink_gqa_bf16_t65536", "bf16", T=65536, Hq=64, Hkv=8, D=64, window=128,
                  scale=1.0 / 8.0, seed=3, doc_dist=("loguniform", 64, 16384), sinks=True),
    SparseWorkload("sparse_mla_bf16_t16384", T=16384, H=128, d_latent=512, d_rope=64, topk=2048,
                   scale=1.0 / math.sqrt(576.0), seed=4, doc_dist=("uniform", 1024, 8192)),
)



@dataclasses.dataclass(frozen=True)
class ValueProjWorkload:
    """The sparse MLA value up-projection on its own: o_latent [T, H, d_latent] -> [T, H, d_value]."""
    name: str
    T: int
    H: int
    d_latent: int
    d_value: int
    seed: int


# Variants measured beside the five: the backward of the three bf16 workloads (same
# inputs, dout from its own stream), dense full-causal GQA with head_dim 256 (the packed
# documents of the 8192-token workload, half its heads), the sparse workload without the
# rotary part (NoPE, same documents and index rows), and the value projection at the sparse
# workload's shape (its attention output feeds that step).
EXTRA_WORKLOADS = (
    DenseWorkload("causal_gqa_bwd_bf16_t8192", "bf16", T=8192, Hq=32, Hkv=8, D=128, window=0,
                  scale=1.0 / math.sqrt(128.0), seed=1, doc_dist=("uniform", 128, 2048), backward=True),
    DenseWorkload("swa1024_gqa_bwd_bf16_t32768", "bf16", T=32768, Hq=32, Hkv=4, D=128, window=1024,
                  scale=1.0 / math.sqrt(128.0), seed=2, doc_dist=("uniform", 512, 8192), rms_norm_qk=True,
                  backward=True),
    DenseWorkload("swa128_sink_gqa_bwd_bf16_t65536", "bf16", T=65536, Hq=64, Hkv=8, D=64, window=128,
                  scale=1.0 / 8.0, seed=3, doc_dist=("loguniform", 64, 16384), sinks=True, backward=True),
    DenseWorkload("causal_gqa_d256_bf16_t8192", "bf16", T=8192, Hq=16, Hkv=4, D=256, window=0,
                  scale=1.0 / 16.0, seed=1, doc_dist=("uniform", 128, 2048)),
    SparseWorkload("sparse_mla_nope_bf16_t16384", T=16384, H=128, d_latent=512, d_rope=0, topk=2048,
                   scale=1.0 / math.sqrt(512.0), seed=4, doc_dist=("uniform", 1024, 8192)),
    ValueProjWorkload("mla_value_proj_bf16_t16384", T=16384, H=128, d_latent=512, d_value=128, seed=4),
)


# ---------------------------------------------------------------------------
# primitives
# ---------------------------------------------------------------------------
def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), returned as float32.

    Works in place on chunks to bound temporary memory; inputs must be finite.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    flat = x.reshape(-1)
    u = flat.view(np.uint32)
    step = 1 << 24
    for s in range(0, u.size, step):
        c = u[s:s + step]
        bias = ((c >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
        c += bias
        c &= np.uint32(0xFFFF0000)
    return x


def draw_doc_lengths(seed: int, T: int, dist: tuple) -> list:
    """Document lengths drawn until they cover T tokens; the last one is truncated."""
    kind, a, b = dist
    rng = np.random.default_rng(seed)
    out, total = [], 0
    while total < T:
        if kind == "uniform":
            L = int(rng.integers(a, b, endpoint=True))
        elif kind == "loguniform":
            L = int(round(math.exp(rng.uniform(math.log(a), math.log(b)))))
            L = min(max(L, a), b)
        else:
            raise ValueError(f"unknown length distribution {kind!r}")
        L = min(L, T - total)
        out.append(L)
        total += L
    return out


def cu_seqlens_from_lengths(lengths: Sequence[int]) -> np.ndarray:
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    if len(lengths):
        cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64)).astype(np.int32)
    return cu


def stream(seed: int, which: int) -> np.random.Generator:
    return np.random.default_rng([seed, which])


def normal(seed: int, which: int, shape) -> np.ndarray:
    """Standard-normal float32 tensor drawn row-chunk by row-chunk from one stream."""
    rng = stream(seed, which)
    out = np.empty(shape, dtype=np.float32)
    rows = out.reshape(shape[0], -1)
    per_row = rows.shape[1]
    chunk = max(1, (1 << 24) // max(per_row, 1))
    for r in range(0, shape[0], chunk):
        rows[r:r + chunk] = rng.standard_normal((min(chunk, shape[0] - r), per_row), dtype=np.float32)
    return out


def scaleless_rms_norm(x: np.ndarray, eps: float = 1e-5) -> np.ndarray:
    """x / sqrt(mean(x^2 over the last axis) + eps), computed in fp64, returned float32.

    Input preparation only (MuseGlimmerScalelessRMSNorm on the muse_glimmer
    model page, used for Q/K normalisation); the attention kernel never sees it.
    """
    out = np.empty_like(x, dtype=np.float32)
    flat_in = x.reshape(-1, x.shape[-1])
    flat_out = out.reshape(-1, x.shape[-1])
    step = 1 << 18
    for s in range(0, flat_in.shape[0], step):
        c = flat_in[s:s + step].astype(np.float64)
        flat_out[s:s + step] = (c / np.sqrt(np.mean(c * c, axis=-1, keepdims=True) + eps)).astype(np.float32)
    return out


# ---------------------------------------------------------------------------
# dense workloads
# ---------------------------------------------------------------------------
def dense_doc_lengths(w: DenseWorkload) -> list:
    if w.doc_lengths is not None:
        return list(w.doc_lengths)
    return draw_doc_lengths(w.seed, w.T, w.doc_dist)


def make_dense(w: DenseWorkload, lengths: Optional[Sequence[int]] = None) -> dict:
    """Inputs for one dense problem.

    Returns a dict with q [T,Hq,D], k [T,Hkv,D], v [T,Hkv,D] (float32 arrays,
    bf16-exact for bf16 workloads), cu_seqlens int32 [n_docs+1], n_docs,
    window, scale, sinks (float32 [Hq] or None) and the workload itself.
    ``lengths`` overrides the drawn document lengths (their sum may be < T,
    leaving a padded tail).
    """
    if lengths is None:
        lengths = dense_doc_lengths(w)
    lengths = [int(x) for x in lengths]
    assert sum(lengths) <= w.T
    q = normal(w.seed, STREAM_Q, (w.T, w.Hq, w.D))
    k = normal(w.seed, STREAM_K, (w.T, w.Hkv, w.D))
    v = normal(w.seed, STREAM_V, (w.T, w.Hkv, w.D))
    if w.rms_norm_qk:
        q = scaleless_rms_norm(q)
        k = scaleless_rms_norm(k)
    if w.dtype == "bf16":
        q, k, v = round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)
    elif w.dtype != "f32":
        raise ValueError(w.dtype)
    sinks = None
    if w.sinks:
        sinks = stream(w.seed, STREAM_SINK).standard_normal(w.Hq, dtype=np.float32)
    return dict(q=q, k=k, v=v, cu_seqlens=cu_seqlens_from_lengths(lengths), n_docs=len(lengths),
                window=w.window, scale=w.scale, sinks=sinks, workload=w, lengths=lengths)


# ---------------------------------------------------------------------------
# sparse workloads
# ---------------------------------------------------------------------------
def sparse_doc_lengths(w: SparseWorkload) -> list:
    if w.doc_lengths is not None:
        return list(w.doc_lengths)
    return draw_doc_lengths(w.seed, w.T, w.doc_dist)


def doc_ids_from_lengths(T: int, lengths: Sequence[int]) -> np.ndarray:
    """Per-token document id; tokens past the last document get -1."""
    ids = np.full(T, -1, dtype=np.int32)
    s = 0
    for d, L in enumerate(lengths):
        ids[s:s + L] = d
        s += L
    return ids


def make_sparse_indices(seed: int, lengths: Sequence[int], T: int, topk: int) -> np.ndarray:
    """int32 [T, topk] causal same-document key indices, ascending, -1 padded."""
    rng = stream(seed, STREAM_IDX)
    idx = np.full((T, topk), -1, dtype=np.int32)
    s = 0
    for L in lengths:
        for p in range(L):
            t = s + p
            if p + 1 <= topk:
                idx[t, :p + 1] = np.arange(s, t + 1, dtype=np.int32)
            else:
                sel = rng.choice(p + 1, topk, replace=False)
                sel.sort()
                idx[t] = (sel + s).astype(np.int32)
        s += L
    return idx


def make_sparse(w: SparseWorkload, lengths: Optional[Sequence[int]] = None) -> dict:
    """Inputs for one sparse MLA problem (bf16-exact float32 arrays).

    q [T,H,d_latent+d_rope], latent [T,d_latent], k_pe [T,d_rope],
    indices int32 [T,topk] (-1 padded), doc_ids int32 [T].
    """
    if lengths is None:
        lengths = sparse_doc_lengths(w)
    lengths = [int(x) for x in lengths]
    q = round_to_bf16(normal(w.seed, STREAM_Q, (w.T, w.H, w.d_qk)))
    latent = round_to_bf16(normal(w.seed, STREAM_LATENT, (w.T, w.d_latent)))
    k_pe = round_to_bf16(normal(w.seed, STREAM_KPE, (w.T, w.d_rope))) if w.d_rope > 0 else \
        np.zeros((w.T, 0), dtype=np.float32)
    indices = make_sparse_indices(w.seed, lengths, w.T, w.topk)
    return dict(q=q, latent=latent, k_pe=k_pe, indices=indices,
                doc_ids=doc_ids_from_lengths(w.T, lengths), scale=w.scale, workload=w, lengths=lengths)


def make_value_weight(seed: int, H: int, d_value: int, d_latent: int = 512) -> np.ndarray:
    """value_weight [H, d_value, d_latent] (bf16-exact float32): standard normal / sqrt(d_latent)."""
    w = normal(seed, STREAM_VW, (H, d_value, d_latent)) * np.float32(1.0 / math.sqrt(d_latent))
    return round_to_bf16(w)


def make_value_proj(w: ValueProjWorkload) -> dict:
    """o_latent [T, H, d_latent] standard normal and value_weight [H, d_value, d_latent] (bf16-exact float32)."""
    o = round_to_bf16(normal(w.seed, STREAM_LATENT, (w.T, w.H, w.d_latent)))
    return dict(o_latent=o, value_weight=make_value_weight(w.seed, w.H, w.d_value, w.d_latent), workload=w)


def make_dout(seed: int, shape) -> np.ndarray:
    """Upstream gradient dL/dout for the backward (bf16-exact float32, standard normal)."""
    return round_to_bf16(normal(seed, STREAM_DOUT, tuple(shape)))
