"""GPU parity of varlen_attn_bwd (through the C ABI) against the fp64 backward oracle.

The HIP path receives a forward output `out` (the oracle's, rounded to bf16, or the GPU
forward's), the matching log-sum-exp and the same seeded dout; its dq, dk, dv, dsinks are
compared element by element with the exact (fp64) gradients.

Tolerance, per element, from the arithmetic of the kernel:
  |got - ref| <= (2^-8 + 1e-4) max(|ref|, |got|) + 6 * 2^-9 * rss + |e_delta| + 1e-6
* 2^-8 max(|ref|, |got|): the one bf16 rounding of the result (round to nearest even, 8
  significant bits: relative error at most 2^-8 of the value rounded, which is the exact
  gradient shifted by e_delta).  1e-4 covers fp32 effects (exp2, accumulation order, the
  fp32 lse).
* 6 * 2^-9 * rss: rss is the root sum of squares of the terms the element sums (dv[j]:
  P_ij dout[i]; dk[j]: scale dS_ij q[i]; dq[i]: scale dS_ij k[j]), with the dS the kernel
  forms from its delta (below).  The kernel rounds P and
  dS to bf16 as matrix operands; a rounding to 8 significant bits has a relative standard
  deviation of about 2^-9, independently per term, so the sum's error has a standard deviation
  of about 2^-9 rss; six of them bound it.  This matters where the terms cancel to a small
  result.
* e_delta: the kernel computes delta_i = <dout_i, out_i> from the `out` it is given, which
  differs from the exact output (bf16 rounding, or the GPU forward's own error).  The
  gradient error this induces is linear and computed exactly by the test:
  dq_i: -scale (delta_used - delta)_i sum_j P_ij k_j ; dk_j: -scale sum_i P_ij (delta_used -
  delta)_i q_i ; dv is unaffected.  It also carries an fp32 bound: dP_ij and delta_i are fp32
  sums of D products (error <= D 2^-24 of the sum of their magnitudes each) that cancel in
  dS_ij = P_ij (dP_ij - delta_i) (exactly, on rows with one key), and P carries ~1e-6 of fp32
  exp2 / lse error: |e| += scale sum_j (2 D 2^-24 + 1e-5) P_ij (|dout_i|.|v_j| + |dout_i|.|out_i|)
  |k_j| for dq (likewise for dk), and 1e-5 sum_i P_ij |dout_i| for dv.

dsinks_h = -sum_i p_sink_i delta_i is a sum whose terms cancel (delta_i = <dout_i, out_i> has
either sign), so a relative bar does not apply.  Its error is set by the bf16 out the kernel
receives: rounding element e of out moves the sum by p_sink_i dout_ie out_ie times a relative
error of standard deviation about 2^-9, independently per element, so the error has a standard
deviation below sigma_h = 2^-9 sqrt(sum_{i,e} (p_sink_i dout_ie out_ie)^2).  The bar is
6 sigma_h + 1e-3 * max(1, |ref|).  A second check recomputes the sum in fp64 from the very
bf16 out the kernel was given and holds the kernel to 1e-4 of sum_i p_sink_i |delta_i| (fp32
summation).
"""
import math

import numpy as np
import pytest
import torch

from oracle import varlen_attn_bwd_ref, varlen_attn_ref
from sliding_window_gqa_varlen_amd import varlen_attn_bwd, varlen_attn_fwd, workloads as W
from tests.gpu_util import dev

pytestmark = pytest.mark.gpu

ROUND = 2.0 ** -8 + 1e-4  # one bf16 rounding of the result, plus fp32 effects


def custom(lengths, T, Hq, Hkv, window, sinks=False, seed=0, D=128):
    w = W.DenseWorkload("custom", "bf16", T=T, Hq=Hq, Hkv=Hkv, D=D, window=window, scale=1.0 / math.sqrt(D),
                        seed=seed, doc_lengths=tuple(lengths), sinks=sinks)
    return W.make_dense(w)


def dout_for(inp, seed):
    return W.make_dout(seed, inp["q"].shape)


def gpu_forward(inp):
    q, k, v = (dev(inp[n], torch.bfloat16) for n in ("q", "k", "v"))
    cu = torch.from_numpy(inp["cu_seqlens"]).cuda()
    s = None if inp["sinks"] is None else torch.from_numpy(np.asarray(inp["sinks"], np.float32)).cuda()
    return varlen_attn_fwd(q, k, v, cu, inp["n_docs"], inp["window"], inp["scale"], s)


def run_bwd(inp, do, window=None, out=None, lse=None):
    """HIP backward on the oracle's forward output (or the given out / lse tensors)."""
    win = inp["window"] if window is None else window
    if out is None:
        ref_o, ref_l = varlen_attn_ref(inp["q"], inp["k"], inp["v"], inp["cu_seqlens"], win, inp["scale"],
                                       inp["sinks"])
        out = dev(ref_o, torch.bfloat16)
        lse = torch.from_numpy(ref_l.astype(np.float32)).cuda()
    q, k, v = (dev(inp[n], torch.bfloat16) for n in ("q", "k", "v"))
    cu = torch.from_numpy(inp["cu_seqlens"]).cuda()
    s = None if inp["sinks"] is None else torch.from_numpy(np.asarray(inp["sinks"], np.float32)).cuda()
    dq, dk, dv, ds = varlen_attn_bwd(q, k, v, out, dev(do, torch.bfloat16), lse, cu, inp["n_docs"], win,
                                     inp["scale"], s)
    torch.cuda.synchronize()
    f = lambda x: None if x is None else x.float().cpu().numpy().astype(np.float64)  # noqa: E731
    return f(dq), f(dk), f(dv), f(ds), f(out)


def oracle_bwd(inp, do, window=None):
    win = inp["window"] if window is None else window
    return varlen_attn_bwd_ref(inp["q"], inp["k"], inp["v"], do, inp["cu_seqlens"], win, inp["scale"],
                               inp["sinks"])[:4]


def term_rss(q, k, v, do, cu, window, scale, sinks, out_used=None):
    """Root sum of squares of the terms each dq, dk, dv element sums, and the exact gradient
    error that delta computed from `out_used` instead of the exact output induces in dq and dk
    (tolerance only)."""
    q, k, v, do = (np.asarray(x, np.float64) for x in (q, k, v, do))
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    rq, rk, rv = np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape)
    eq, ek = np.zeros(q.shape), np.zeros(k.shape)
    fq, fk, fv = np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape)
    for d in range(len(cu) - 1):
        s, e = int(cu[d]), int(cu[d + 1])
        for i0 in range(s, e, 256):  # query blocks; keys limited to the block's causal / window range
            i1 = min(i0 + 256, e)
            lo = max(s, i0 - window + 1) if window > 0 else s
            i, j = np.arange(i0, i1)[:, None], np.arange(lo, i1)[None, :]
            ok = (j <= i) & ((window == 0) | (i - j < window))
            for h in range(Hq):
                g = h // G
                S = np.where(ok, scale * q[i0:i1, h] @ k[lo:i1, g].T, -np.inf)
                m = S.max(axis=1)
                if sinks is not None:
                    m = np.maximum(m, sinks[h])
                E = np.exp(S - m[:, None])
                Z = E.sum(axis=1) + (0.0 if sinks is None else np.exp(sinks[h] - m))
                P = E / Z[:, None]
                dP = do[i0:i1, h] @ v[lo:i1, g].T
                dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
                # fp32 bound on the kernel's dS_ij = P_ij (dP_ij - delta_i): both dots are fp32
                # sums of D products (relative error <= D 2^-24 of the sum of their magnitudes),
                # and P carries ~1e-6 of fp32 exp2 / lse error
                o_abs = np.abs(P @ v[lo:i1, g]) if out_used is None else np.abs(np.asarray(out_used[i0:i1, h], np.float64))
                mag = np.abs(do[i0:i1, h]) @ np.abs(v[lo:i1, g]).T + (np.abs(do[i0:i1, h]) * o_abs).sum(axis=1)[:, None]
                g32 = (2 * D * 2.0 ** -24 + 1e-5) * P * mag
                fq[i0:i1, h] = scale * g32 @ np.abs(k[lo:i1, g])
                fk[lo:i1, g] += scale * g32.T @ np.abs(q[i0:i1, h])
                fv[lo:i1, g] += 1e-5 * P.T @ np.abs(do[i0:i1, h])
                if out_used is not None:
                    o_exact = P @ v[lo:i1, g]
                    ddelta = (do[i0:i1, h] * (np.asarray(out_used[i0:i1, h], np.float64) - o_exact)).sum(axis=1)
                    eq[i0:i1, h] = -scale * ddelta[:, None] * (P @ k[lo:i1, g])
                    ek[lo:i1, g] += -scale * (P.T @ (ddelta[:, None] * q[i0:i1, h]))
                    dS = dS - P * ddelta[:, None]  # the dS the kernel forms (and rounds) from that delta
                rv[lo:i1, g] += (P ** 2).T @ do[i0:i1, h] ** 2
                rk[lo:i1, g] += scale ** 2 * (dS ** 2).T @ q[i0:i1, h] ** 2
                rq[i0:i1, h] = scale ** 2 * (dS ** 2) @ k[lo:i1, g] ** 2
    return (np.sqrt(rq), np.sqrt(rk), np.sqrt(rv)), (np.abs(eq) + fq, np.abs(ek) + fk, fv)


def check(got, ref, what, rss, e_delta=0.0):
    assert got.shape == ref.shape, what
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    bar = ROUND * np.maximum(np.abs(ref), np.abs(got)) + 6 * 2.0 ** -9 * rss + e_delta + 1e-6
    err = np.abs(got - ref) / bar
    i = np.unravel_index(np.argmax(err), err.shape)
    assert err.max() <= 1.0, f"{what}: error {err.max():.2f} x its bar at {i} (got {got[i]:.5f}, ref {ref[i]:.5f})"
    return float(err.max())


def sink_probabilities(inp, window=None):
    win = inp["window"] if window is None else window
    o, l = varlen_attn_ref(inp["q"], inp["k"], inp["v"], inp["cu_seqlens"], win, inp["scale"], inp["sinks"])
    with np.errstate(over="ignore"):
        p = np.where(np.isneginf(l), 0.0, np.exp(np.asarray(inp["sinks"], np.float64)[None, :] - l))
    return o, p


def check_all(got, ref, inp=None, do=None, window=None, out_given=None, lse_given=None):
    """got = (dq, dk, dv, dsinks, out the kernel received)."""
    win = inp["window"] if window is None else window
    rss, ed = term_rss(inp["q"], inp["k"], inp["v"], do, inp["cu_seqlens"], win, inp["scale"], inp["sinks"],
                       out_used=got[4])
    for name, g, r, x, e in zip(("dq", "dk", "dv"), got, ref, rss, ed):
        check(g, r, name, x, e)
    if ref[3] is None:
        assert got[3] is None
        return
    check_dsinks(got[3], ref[3], inp, do, window, out_given, lse_given)


def check_dsinks(g, r, inp, do, window=None, out_given=None, lse_given=None):
    o, p = sink_probabilities(inp, window)
    d = np.asarray(do, np.float64)
    sigma = 2.0 ** -9 * np.sqrt(((p[:, :, None] * d * o) ** 2).sum(axis=(0, 2)))
    err = np.abs(g - r)
    bar = 6 * sigma + 1e-3 * np.maximum(1.0, np.abs(r))
    assert np.all(err <= bar), f"dsinks: error {err.max():.3e} beyond its rounding bar {bar[np.argmax(err - bar)]:.3e}"
    ob = W.round_to_bf16(o.astype(np.float32)).astype(np.float64) if out_given is None else out_given
    if lse_given is not None:
        with np.errstate(over="ignore"):
            p = np.where(np.isneginf(lse_given), 0.0,
                         np.exp(np.asarray(inp["sinks"], np.float64)[None, :] - lse_given))
    delta_b = (d * ob).sum(axis=2)
    same_input = -(p * delta_b).sum(axis=0)
    assert np.all(np.abs(g - same_input) <= 1e-4 * np.maximum(1.0, (p * np.abs(delta_b)).sum(axis=0)))


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("sinks", [False, True])
def test_ragged_documents_and_padding_tail(gpu, sinks, D):
    lengths = [1, 31, 33, 63, 65, 127, 129, 2, 200]
    inp = custom(lengths, T=sum(lengths) + 37, Hq=8, Hkv=2, window=0, sinks=sinks, seed=1 + sinks, D=D)
    do = dout_for(inp, 3)
    got = run_bwd(inp, do)
    check_all(got, oracle_bwd(inp, do), inp, do)
    T0 = sum(lengths)
    assert np.all(got[0][T0:] == 0) and np.all(got[1][T0:] == 0) and np.all(got[2][T0:] == 0)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("window", [1, 17, 64, 65, 100, 128, 200])
def test_windows_with_sinks(gpu, window, D):
    lengths = [300, 5, 129, 64]
    inp = custom(lengths, T=sum(lengths), Hq=16, Hkv=2, window=window, sinks=True, seed=window, D=D)
    do = dout_for(inp, window)
    check_all(run_bwd(inp, do), oracle_bwd(inp, do), inp, do)


@pytest.mark.parametrize("Hq,Hkv,D", [(4, 4, 128), (6, 1, 128), (12, 2, 128), (40, 8, 128), (64, 1, 128),
                                     (6, 1, 64), (64, 8, 64)])
def test_gqa_group_shapes(gpu, Hq, Hkv, D):
    lengths = [100, 37, 150]
    inp = custom(lengths, T=287, Hq=Hq, Hkv=Hkv, window=50, sinks=True, seed=Hq + Hkv, D=D)
    do = dout_for(inp, 7)
    check_all(run_bwd(inp, do), oracle_bwd(inp, do), inp, do)


def test_zero_length_documents_head_and_tail_padding(gpu):
    lengths = [0, 40, 0, 0, 70, 1, 0]
    inp = custom(lengths, T=130, Hq=8, Hkv=2, window=0, sinks=True, seed=5)
    inp["cu_seqlens"] = inp["cu_seqlens"] + 9  # tokens 0..8 sit before the first document
    do = dout_for(inp, 5)
    got = run_bwd(inp, do)
    check_all(got, oracle_bwd(inp, do), inp, do)
    for g in got[:3]:
        assert np.all(g[:9] == 0) and np.all(g[120:] == 0)


@pytest.mark.parametrize("n_docs,window", [(61, 0), (62, 0), (63, 0), (90, 0), (90, 29)])
def test_many_documents(gpu, n_docs, window):
    """Segment decodes on both sides of 61 documents (dq), heaviest-first dk/dv key tiles up to
    62 documents and document order beyond (causal), with empty documents and padding."""
    rng = np.random.default_rng(n_docs + window)
    lengths = [int(x) for x in rng.integers(0, 40, n_docs)]
    lengths[5] = 0
    inp = custom(lengths, T=sum(lengths) + 11, Hq=8, Hkv=2, window=window, sinks=window > 0, seed=n_docs, D=128)
    do = dout_for(inp, n_docs)
    got = run_bwd(inp, do)
    check_all(got, oracle_bwd(inp, do), inp, do)
    T0 = sum(lengths)
    for g in got[:3]:
        assert np.all(g[T0:] == 0)


@pytest.mark.parametrize("D", [64, 128])
def test_scores_growing_along_the_keys(gpu, D):
    """Scores that grow by 0.08 to 0.11 per key span more than 60 natural units along a
    document: P = exp(S scale - lse) then ranges over many orders of magnitude per row."""
    lengths = [700, 333]
    inp = custom(lengths, T=1033, Hq=8, Hkv=2, window=0, sinks=True, seed=D + 3, D=D)
    T = 1033
    pos = np.concatenate([np.arange(700), np.arange(333)]).astype(np.float32)
    u = np.ones(D, np.float32)
    inp["q"] = W.round_to_bf16(np.ascontiguousarray(np.broadcast_to(u, (T, 8, D)) + 0.05 * inp["q"], np.float32))
    inp["k"] = W.round_to_bf16(np.ascontiguousarray(
        (0.01 * pos)[:, None, None] * np.broadcast_to(u, (T, 2, D)) + 0.05 * inp["k"], np.float32))
    do = dout_for(inp, D)
    check_all(run_bwd(inp, do), oracle_bwd(inp, do), inp, do)


def test_packed_documents_elementwise(gpu):
    """2048 tokens in documents of 128..512 tokens, 16 query / 4 KV heads, full causal."""
    w = W.DenseWorkload("bwd", "bf16", T=2048, Hq=16, Hkv=4, D=128, window=0, scale=1.0 / math.sqrt(128.0),
                        seed=8, doc_dist=("uniform", 128, 512))
    inp = W.make_dense(w)
    do = dout_for(inp, 8)
    check_all(run_bwd(inp, do), oracle_bwd(inp, do), inp, do)


@pytest.mark.parametrize("idx", [1, 2, 3])
def test_full_size_workloads_on_chosen_documents(gpu, idx):
    """The full-size workloads in the bench's launch configuration (out and lse from the GPU
    forward); the oracle recomputes whole documents (documents are independent), the smallest
    ones plus one of ~1100 tokens."""
    inp = W.make_dense(W.WORKLOADS[idx])
    do = dout_for(inp, 10 + idx)
    out, lse = gpu_forward(inp)
    got = run_bwd(inp, do, out=out, lse=lse)
    cu = inp["cu_seqlens"]
    lens = np.diff(cu)
    order = list(np.argsort(lens)[:2]) + [int(np.argmin(np.abs(lens - 1100)))]
    for d in sorted(set(order)):
        s, e = int(cu[d]), int(cu[d + 1])
        sl = slice(s, e)
        args = (inp["q"][sl], inp["k"][sl], inp["v"][sl], do[sl], [0, e - s], inp["window"], inp["scale"],
                inp["sinks"])
        ref = varlen_attn_bwd_ref(*args)
        rss, ed = term_rss(*args, out_used=got[4][sl])
        for name, g, r, x, err in zip(("dq", "dk", "dv"), got[:3], ref[:3], rss, ed):
            check(g[sl], r, f"{name} of document {d} ({e - s} tokens)", x, err)


@pytest.mark.parametrize("idx,groups", [(2, (1,)), (3, (0, 7))])
def test_full_size_windowed_every_element_of_chosen_kv_groups(gpu, idx, groups):
    """The full-size windowed backwards as bench times them (out and lse from the GPU forward),
    every token: each element of dq for the query heads of the chosen KV groups, of dk and dv
    for those KV heads, and of dsinks for those heads (the window-128 workload has sinks).
    Groups are independent (query head h reads KV head h // G only), so the oracle runs on
    the chosen groups alone."""
    wl = W.WORKLOADS[idx]
    inp = W.make_dense(wl)
    do = dout_for(inp, 20 + idx)
    out, lse = gpu_forward(inp)
    got = run_bwd(inp, do, out=out, lse=lse)
    G = wl.Hq // wl.Hkv
    heads = [h for g in groups for h in range(g * G, (g + 1) * G)]
    sel = dict(inp)
    sel["q"] = inp["q"][:, heads]
    sel["k"] = inp["k"][:, list(groups)]
    sel["v"] = inp["v"][:, list(groups)]
    sel["sinks"] = None if inp["sinks"] is None else np.asarray(inp["sinks"])[heads]
    do_sel = do[:, heads]
    ref = oracle_bwd(sel, do_sel)
    out_sel = got[4][:, heads]
    rss, ed = term_rss(sel["q"], sel["k"], sel["v"], do_sel, inp["cu_seqlens"], wl.window, wl.scale, sel["sinks"],
                       out_used=out_sel)
    sub = (got[0][:, heads], got[1][:, list(groups)], got[2][:, list(groups)])
    for name, g, r, x, e in zip(("dq", "dk", "dv"), sub, ref[:3], rss, ed):
        check(g, r, f"{name} of KV groups {groups}", x, e)
    if wl.sinks:
        check_dsinks(got[3][heads], ref[3], sel, do_sel, out_given=out_sel,
                     lse_given=lse.cpu().numpy().astype(np.float64)[:, heads])


def test_causal_workload_every_element(gpu):
    """The 8192-token causal backward as bench times it (out and lse from the GPU forward): every
    element of dq, dk and dv against the fp64 oracle over all documents (about 30 s of host time)."""
    inp = W.make_dense(W.WORKLOADS[1])
    do = dout_for(inp, 11)
    out, lse = gpu_forward(inp)
    got = run_bwd(inp, do, out=out, lse=lse)
    args = (inp["q"], inp["k"], inp["v"], do, inp["cu_seqlens"], inp["window"], inp["scale"], inp["sinks"])
    ref = varlen_attn_bwd_ref(*args)
    rss, ed = term_rss(*args, out_used=got[4])
    for name, g, r, x, e in zip(("dq", "dk", "dv"), got[:3], ref[:3], rss, ed):
        check(g, r, name, x, e)


def test_with_the_gpu_forward_outputs(gpu):
    """out and lse straight from varlen_attn_fwd (bf16 out, fp32 lse) feed the backward."""
    lengths = [120, 300, 80]
    inp = custom(lengths, T=500, Hq=8, Hkv=2, window=90, sinks=True, seed=31)
    out, lse = gpu_forward(inp)
    do = dout_for(inp, 31)
    ob = out.float().cpu().numpy().astype(np.float64)
    lb = lse.cpu().numpy().astype(np.float64)
    check_all(run_bwd(inp, do, out=out, lse=lse), oracle_bwd(inp, do), inp, do, out_given=ob, lse_given=lb)


def test_window_at_least_document_length_is_bitwise_full_causal(gpu):
    lengths = [250, 40, 123]
    inp = custom(lengths, T=413, Hq=8, Hkv=4, window=0, seed=4)
    do = dout_for(inp, 4)
    a = run_bwd(inp, do)
    b = run_bwd(inp, do, window=250)
    for x, y in zip(a[:3], b[:3]):
        np.testing.assert_array_equal(x, y)


def test_strided_views_of_fused_buffers(gpu):
    """q, k, v as views of one [T, Hq + 2 Hkv, D] buffer; dq, dk, dv as views of another."""
    lengths = [77, 130]
    inp = custom(lengths, T=207, Hq=8, Hkv=2, window=0, sinks=False, seed=6)
    do = dout_for(inp, 6)
    ref_o, ref_l = varlen_attn_ref(inp["q"], inp["k"], inp["v"], inp["cu_seqlens"], 0, inp["scale"], None)
    qkv = torch.cat([dev(inp[n], torch.bfloat16) for n in ("q", "k", "v")], dim=1)
    q, k, v = qkv[:, :8], qkv[:, 8:10], qkv[:, 10:12]
    grads = torch.full((207, 12, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    dq, dk, dv = grads[:, :8], grads[:, 8:10], grads[:, 10:12]
    cu = torch.from_numpy(inp["cu_seqlens"]).cuda()
    lse = torch.from_numpy(ref_l.astype(np.float32)).cuda()
    varlen_attn_bwd(q, k, v, dev(ref_o, torch.bfloat16), dev(do, torch.bfloat16), lse, cu, 2, 0, inp["scale"],
                    None, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    ref = oracle_bwd(inp, do)
    rss, ed = term_rss(inp["q"], inp["k"], inp["v"], do, inp["cu_seqlens"], 0, inp["scale"], None,
                       out_used=W.round_to_bf16(ref_o.astype(np.float32)))
    for name, g, r, x, e in zip(("dq", "dk", "dv"), (dq, dk, dv), ref[:3], rss, ed):
        check(g.float().cpu().numpy().astype(np.float64), r, name, x, e)


def test_repeat_runs_are_bitwise_identical(gpu):
    lengths = [300, 211]
    inp = custom(lengths, T=511, Hq=16, Hkv=4, window=0, sinks=True, seed=12)
    do = dout_for(inp, 12)
    a, b = run_bwd(inp, do), run_bwd(inp, do)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
