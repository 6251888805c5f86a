"""Stream and graph behaviour of the entry points (GPU).

Every entry point enqueues its kernels on the stream it is given and touches nothing else (no
allocation, no memset, no host synchronisation), so it may be called on any stream and captured
into a HIP graph.  These tests check both: a call on a side stream equals the same call on the
default stream bitwise, and a captured call replayed several times, with the inputs rewritten in
place by ordinary eager work between replays, reproduces an eager call on the same inputs
bitwise on every replay.  The eager results are checked against the oracle once, so equality
with them is equality with a correct result.
"""
import math

import numpy as np
import pytest
import torch

from oracle import varlen_attn_ref
from sliding_window_gqa_varlen_amd import (mla_value_proj, sparse_mla_fwd, varlen_attn_bwd, varlen_attn_fwd,
                                           workloads as W)
from tests.gpu_util import BF16_MAX_ABS, assert_dense_parity, dev

pytestmark = pytest.mark.gpu

REPLAYS = 3


def dense_inputs(seed, window, sinks, D=128):
    w = W.DenseWorkload("graph", "bf16", T=700, Hq=8, Hkv=2, D=D, window=window, scale=1.0 / math.sqrt(D),
                        seed=seed, doc_lengths=(5, 130, 0, 301, 200), sinks=sinks)
    return W.make_dense(w)


def to_gpu(inp):
    q, k, v = (dev(inp[n], torch.bfloat16) for n in ("q", "k", "v"))
    s = None if inp["sinks"] is None else torch.from_numpy(np.asarray(inp["sinks"], np.float32)).cuda()
    return q, k, v, torch.from_numpy(inp["cu_seqlens"]).cuda(), s


def capture(fn):
    """Warm up on a side stream, then capture fn() into a graph (torch's capture protocol)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("window,sinks", [(0, False), (64, True)])
def test_forward_on_a_side_stream_and_in_a_graph(gpu, window, sinks):
    inp = dense_inputs(1, window, sinks)
    q, k, v, cu, s = to_gpu(inp)
    n_docs, scale = inp["n_docs"], inp["scale"]
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], device=gpu, dtype=torch.float32)

    ref_o, ref_l = varlen_attn_fwd(q, k, v, cu, n_docs, window, scale, s)
    torch.cuda.synchronize()
    want_o, want_l = varlen_attn_ref(inp["q"], inp["k"], inp["v"], inp["cu_seqlens"], window, scale, inp["sinks"])
    assert_dense_parity("bf16", ref_o.float().cpu().numpy().astype(np.float64),
                        ref_l.cpu().numpy().astype(np.float64), want_o, want_l)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        so, sl = varlen_attn_fwd(q, k, v, cu, n_docs, window, scale, s, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert torch.equal(so, ref_o) and torch.equal(sl, ref_l)

    g = capture(lambda: varlen_attn_fwd(q, k, v, cu, n_docs, window, scale, s, out=out, lse=lse))
    for r in range(REPLAYS):
        nxt = dense_inputs(10 + r, window, sinks)
        for t, name in ((q, "q"), (k, "k"), (v, "v")):  # eager in-place rewrite of the captured inputs
            t.copy_(dev(nxt[name], torch.bfloat16))
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        eo, el = varlen_attn_fwd(q, k, v, cu, n_docs, window, scale, s)
        torch.cuda.synchronize()
        assert torch.equal(out, eo), f"replay {r}: out differs from the eager call"
        assert torch.equal(lse, el), f"replay {r}: lse differs from the eager call"


def test_backward_on_a_side_stream_and_in_a_graph(gpu):
    window = 48
    inp = dense_inputs(2, window, True)
    q, k, v, cu, s = to_gpu(inp)
    n_docs, scale = inp["n_docs"], inp["scale"]
    o, lse = varlen_attn_fwd(q, k, v, cu, n_docs, window, scale, s)
    do = dev(W.make_dout(3, inp["q"].shape), torch.bfloat16)
    bufs = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v),
            torch.empty(q.shape[1], device=gpu, dtype=torch.float32),
            torch.empty(q.shape[:2], device=gpu, dtype=torch.float32))

    def eager():
        r = varlen_attn_bwd(q, k, v, o, do, lse, cu, n_docs, window, scale, s)
        torch.cuda.synchronize()
        return r

    ref = eager()
    assert all(torch.isfinite(x.float()).all() for x in ref)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        got = varlen_attn_bwd(q, k, v, o, do, lse, cu, n_docs, window, scale, s, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for a, b in zip(got, ref):
        assert torch.equal(a, b)

    g = capture(lambda: varlen_attn_bwd(q, k, v, o, do, lse, cu, n_docs, window, scale, s, dq=bufs[0], dk=bufs[1],
                                        dv=bufs[2], dsinks=bufs[3], delta=bufs[4]))
    for r in range(REPLAYS):
        do.copy_(dev(W.make_dout(20 + r, inp["q"].shape), torch.bfloat16))
        for b in bufs[:4]:
            b.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want = eager()
        for name, a, b in zip(("dq", "dk", "dv", "dsinks"), bufs[:4], want):
            assert torch.equal(a, b), f"replay {r}: {name} differs from the eager call"


def test_sparse_and_value_projection_in_a_graph(gpu):
    w = W.SparseWorkload("graph", T=300, H=64, d_latent=512, d_rope=64, topk=96, scale=1.0 / 24.0, seed=5,
                         doc_dist=("uniform", 40, 200), doc_lengths=None)
    inp = W.make_sparse(w)
    q = dev(inp["q"], torch.bfloat16)
    lat = dev(inp["latent"], torch.bfloat16)
    kpe = dev(inp["k_pe"], torch.bfloat16)
    idx = torch.from_numpy(inp["indices"]).cuda()
    ids = torch.from_numpy(inp["doc_ids"]).cuda()
    gen = torch.Generator().manual_seed(6)
    wv = (torch.randn(64, 128, 512, generator=gen) * 0.05).to(torch.bfloat16).cuda()
    o_lat = torch.empty(300, 64, 512, device=gpu, dtype=torch.bfloat16)
    lse = torch.empty(300, 64, device=gpu, dtype=torch.float32)
    out_v = torch.empty(300, 64, 128, device=gpu, dtype=torch.bfloat16)

    def step():
        sparse_mla_fwd(q, lat, kpe, idx, ids, inp["scale"], out=o_lat, lse=lse)
        mla_value_proj(o_lat, wv, out=out_v)

    g = capture(step)
    rng = np.random.default_rng(7)
    for r in range(REPLAYS):
        lat.copy_(dev(rng.standard_normal((300, 512)).astype(np.float32), torch.bfloat16))
        for t in (o_lat, out_v, lse):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        eo, el = sparse_mla_fwd(q, lat, kpe, idx, ids, inp["scale"])
        ev = mla_value_proj(eo, wv)
        torch.cuda.synchronize()
        assert torch.equal(o_lat, eo) and torch.equal(lse, el), f"replay {r}: sparse output differs"
        assert torch.equal(out_v, ev), f"replay {r}: projected output differs"
        assert torch.isfinite(out_v.float()).all() and float(out_v.float().abs().max()) > BF16_MAX_ABS
