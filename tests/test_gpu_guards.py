"""Every output element written, nothing outside written: sparse_mla_fwd, mla_value_proj and
varlen_attn_bwd (the dense forward has its own in test_gpu_dense.py).

Each output is a strided view into a larger buffer filled with NaN, with guard regions before
and after it.  After the call the view holds finite values (zeros / -inf exactly where the
contract says so) and every byte outside the view - the guards and the gaps between strided
rows - is still NaN.  Inputs include padding tokens and empty sparse rows.
"""
import math

import numpy as np
import pytest
import torch

from sliding_window_gqa_varlen_amd import binding, workloads as W
from tests.gpu_util import dev

pytestmark = pytest.mark.gpu

GUARD = 4096


def guarded(shape, pad_last=0, dtype=torch.bfloat16, pad_mid=0):
    """A NaN buffer with GUARD elements on both sides holding a view of `shape`; the view's
    rows are padded by pad_mid heads / pad_last elements (a strided view when non-zero)."""
    T, H, D = shape
    full = (T, H + pad_mid, D + pad_last)
    n = int(np.prod(full))
    buf = torch.full((2 * GUARD + n,), float("nan"), device="cuda", dtype=dtype)
    inner = buf[GUARD:GUARD + n].view(full)
    # the view starts 8 elements into each row when padded (16-byte aligned) and skips one head
    h0 = 1 if pad_mid else 0
    d0 = 8 if pad_last else 0
    view = inner[:, h0:h0 + H, d0:d0 + D]
    mask = torch.zeros(full, dtype=torch.bool, device="cuda")
    mask[:, h0:h0 + H, d0:d0 + D] = True
    return buf, inner, view, mask


def guarded_vec(n, dtype=torch.float32):
    buf = torch.full((2 * GUARD + n,), float("nan"), device="cuda", dtype=dtype)
    return buf, buf[GUARD:GUARD + n]


def untouched(buf, inner=None, mask=None):
    assert torch.isnan(buf[:GUARD].float()).all() and torch.isnan(buf[-GUARD:].float()).all(), "guard written"
    if inner is not None:
        assert torch.isnan(inner[~mask].float()).all(), "a gap between strided rows was written"


def test_sparse_mla_outputs(gpu):
    """Padding tokens (doc id -1), an all -1 index row, duplicate and out-of-document slots."""
    T, H, topk = 300, 32, 64
    w = W.SparseWorkload("guard", T=T, H=H, d_latent=512, d_rope=64, topk=topk, scale=1.0 / math.sqrt(576.0),
                         seed=11, doc_lengths=(120, 1, 150))
    inp = W.make_sparse(w)
    idx = inp["indices"].copy()
    idx[5] = -1                      # an empty row inside a document
    idx[40, :8] = idx[40, 0]         # duplicates
    idx[200, 3] = 10                 # a key of another document (masked)
    ids = inp["doc_ids"].copy()      # tokens 271.. lie past the last document: padding (-1)
    assert (ids[271:] == -1).all() and (ids[:271] >= 0).all()
    obuf, oin, out, omask = guarded((T, H, 512), pad_mid=2)
    lbuf, lse = guarded_vec(T * H)
    binding.sparse_mla_fwd(dev(inp["q"], torch.bfloat16), dev(inp["latent"], torch.bfloat16),
                           dev(inp["k_pe"], torch.bfloat16), torch.from_numpy(idx).cuda(),
                           torch.from_numpy(ids).cuda(), w.scale, out=out, lse=lse.view(T, H))
    torch.cuda.synchronize()
    untouched(obuf, oin, omask)
    untouched(lbuf)
    assert torch.isfinite(out.float()).all()
    l = lse.view(T, H)
    assert not torch.isnan(l).any()
    for t in [5] + list(range(271, T)):  # empty rows: zeros and -inf
        assert (out[t] == 0).all() and torch.isneginf(l[t]).all(), t
    assert torch.isfinite(l[:5]).all() and torch.isfinite(l[6:271]).all()


@pytest.mark.parametrize("Dv", [64, 128])
def test_value_projection_output(gpu, Dv):
    T, H = 97, 8
    rng = np.random.default_rng(Dv)
    o = W.round_to_bf16(rng.standard_normal((T, H, 512)).astype(np.float32))
    o[10] = 0.0
    wv = W.make_value_weight(3, H, Dv)
    obuf, oin, out, omask = guarded((T, H, Dv), pad_last=24)
    binding.mla_value_proj(dev(o, torch.bfloat16), dev(wv, torch.bfloat16), out=out)
    torch.cuda.synchronize()
    untouched(obuf, oin, omask)
    assert torch.isfinite(out.float()).all()
    assert (out[10] == 0).all()


@pytest.mark.parametrize("D,sinks", [(128, True), (64, False)])
def test_backward_outputs(gpu, D, sinks):
    """Gradients as strided views (dq skips one head per token, dk/dv rows padded), a padding
    tail, a guarded delta workspace and dsinks."""
    lengths = [100, 1, 70]
    T, Hq, Hkv = 190, 8, 2
    w = W.DenseWorkload("guard", "bf16", T=T, Hq=Hq, Hkv=Hkv, D=D, window=33 if sinks else 0,
                        scale=1.0 / math.sqrt(D), seed=D, doc_lengths=tuple(lengths), sinks=sinks)
    inp = W.make_dense(w)
    q, k, v = (dev(inp[n], torch.bfloat16) for n in ("q", "k", "v"))
    cu = torch.from_numpy(inp["cu_seqlens"]).cuda()
    s = torch.from_numpy(np.asarray(inp["sinks"], np.float32)).cuda() if sinks else None
    out, lse = binding.varlen_attn_fwd(q, k, v, cu, inp["n_docs"], w.window, w.scale, s)
    dout = dev(W.make_dout(D, inp["q"].shape), torch.bfloat16)
    qb, qin, dq, qmask = guarded((T, Hq, D), pad_mid=2)
    kb, kin, dk, kmask = guarded((T, Hkv, D), pad_last=16)
    vb, vin, dv, vmask = guarded((T, Hkv, D), pad_last=8)
    db, delta = guarded_vec(T * Hq)
    sb, dsinks = guarded_vec(Hq)
    binding.varlen_attn_bwd(q, k, v, out, dout, lse, cu, inp["n_docs"], w.window, w.scale, s, dq=dq, dk=dk, dv=dv,
                            dsinks=dsinks if sinks else None, delta=delta.view(T, Hq))
    torch.cuda.synchronize()
    for b, i, m in ((qb, qin, qmask), (kb, kin, kmask), (vb, vin, vmask)):
        untouched(b, i, m)
    untouched(db)
    untouched(sb)
    for g in (dq, dk, dv):
        assert torch.isfinite(g.float()).all()
        assert (g[sum(lengths):] == 0).all()  # the padding tail receives no gradient
    if sinks:
        assert torch.isfinite(dsinks).all()
    else:
        assert torch.isnan(dsinks).all()  # not given to the call, so never written
