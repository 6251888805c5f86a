"""GPU parity of varlen_attn_fwd (through the C ABI) against the fp64 oracle.

Small problems are compared element by element with the whole oracle output;
the full-size workloads are run in the launch configuration the bench times
and compared on sampled (token, head) rows the oracle computes one by one.
"""
import math

import numpy as np
import pytest
import torch

from oracle import varlen_attn_ref, varlen_attn_ref_rows
from sliding_window_gqa_varlen_amd import varlen_attn_fwd, workloads as W
from tests.golden_util import load
from tests.gpu_util import BF16_MAX_ABS, assert_dense_parity, dev, run_dense

pytestmark = pytest.mark.gpu


def oracle_full(inp):
    return varlen_attn_ref(inp["q"], inp["k"], inp["v"], inp["cu_seqlens"], inp["window"], inp["scale"],
                           inp["sinks"])


def custom(lengths, T, Hq, Hkv, D, window, dtype, sinks=False, seed=0, scale=None):
    w = W.DenseWorkload("custom", dtype, T=T, Hq=Hq, Hkv=Hkv, D=D, window=window,
                        scale=scale or 1.0 / math.sqrt(D), seed=seed, doc_lengths=tuple(lengths), sinks=sinks)
    return W.make_dense(w)


# ------------------------------------------------------------------ hand cases on the GPU
@pytest.mark.parametrize("case", load("dense_hand_cases.json"), ids=lambda c: c["name"])
def test_hand_cases_f32(gpu, case):
    """Hand-derived closed forms, embedded in D=64 by zero padding (dot products unchanged)."""
    q = np.zeros((len(case["q"]), case["Hq"], 64), np.float32)
    k = np.zeros((len(case["k"]), case["Hkv"], 64), np.float32)
    v = np.zeros_like(k)
    q[..., :1] = case["q"]
    k[..., :1] = case["k"]
    v[..., :1] = case["v"]
    cu = np.array(case["cu_seqlens"], np.int32)
    inp = dict(q=q, k=k, v=v, cu_seqlens=cu, n_docs=len(cu) - 1, window=case["window"], scale=case["scale"],
               sinks=None if case["sinks"] is None else np.array(case["sinks"], np.float32))
    out, lse = run_dense(inp, "f32")
    np.testing.assert_allclose(out[..., 0], case["out_expected"], rtol=2e-6, atol=2e-6)
    assert np.all(out[..., 1:] == 0)
    exp_lse = case["lse_expected"]
    assert np.array_equal(np.isneginf(lse), np.isneginf(exp_lse))
    fin = np.isfinite(exp_lse)
    np.testing.assert_allclose(lse[fin], exp_lse[fin], rtol=2e-6, atol=2e-6)


# ------------------------------------------------------------------ the five workloads
def test_tiny_causal_gqa_f32_workload(gpu):
    inp = W.make_dense(W.WORKLOADS[0])
    ref_o, ref_l = oracle_full(inp)
    out, lse = run_dense(inp, "f32")
    assert_dense_parity("f32", out, lse, ref_o, ref_l)


@pytest.mark.parametrize("idx,T", [(1, 2048), (2, 4096), (3, 4096)])
def test_bf16_workloads_scaled_down_elementwise(gpu, idx, T):
    """Same recipe (head counts, D, window, sinks, RMS norm) at a T the oracle finishes quickly."""
    inp = W.make_dense(W.WORKLOADS[idx].with_tokens(T))
    ref_o, ref_l = oracle_full(inp)
    out, lse = run_dense(inp, "bf16")
    assert_dense_parity("bf16", out, lse, ref_o, ref_l)


def sample_rows(inp, n_random, seed):
    rng = np.random.default_rng(seed)
    T, Hq = inp["q"].shape[:2]
    cu = inp["cu_seqlens"]
    toks = [int(x) for x in rng.integers(0, T, n_random)]
    for d in range(len(cu) - 1):  # document edges: first, second, last tokens, window edge
        s, e = int(cu[d]), int(cu[d + 1])
        toks += [t for t in (s, s + 1, e - 1, e - 2, s + inp["window"] - 1, s + inp["window"]) if s <= t < e]
    toks = np.array(toks)
    heads = rng.integers(0, Hq, toks.size)
    return toks, heads


@pytest.mark.parametrize("idx", [1, 2, 3])
def test_bf16_workloads_full_size_sampled(gpu, idx):
    inp = W.make_dense(W.WORKLOADS[idx])
    out, lse = run_dense(inp, "bf16")
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    toks, heads = sample_rows(inp, 300, idx)
    ref_o, ref_l = varlen_attn_ref_rows(inp["q"], inp["k"], inp["v"], inp["cu_seqlens"], inp["window"],
                                        inp["scale"], inp["sinks"], toks, heads)
    err_o = np.abs(out[toks, heads] - ref_o).max()
    err_l = np.abs(lse[toks, heads] - ref_l).max()
    assert err_o <= BF16_MAX_ABS, err_o
    assert err_l <= BF16_MAX_ABS, err_l


@pytest.mark.parametrize("idx", [1, 2, 3])
def test_bf16_workloads_full_size_every_row(gpu, idx):
    """The full-size workloads exactly as bench times them, every (token, head) row of out and
    lse against the full fp64 oracle (about 5, 15 and 30 s of host time)."""
    inp = W.make_dense(W.WORKLOADS[idx])
    out, lse = run_dense(inp, "bf16")
    ref_o, ref_l = oracle_full(inp)
    assert_dense_parity("bf16", out, lse, ref_o, ref_l)


# ------------------------------------------------------------------ edge cases
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
def test_ragged_documents_and_tails(gpu, dtype, D):
    lengths = [1, 31, 33, 63, 65, 127, 129, 2, 200]
    inp = custom(lengths, T=sum(lengths) + 37, Hq=8, Hkv=2, D=D, window=0, dtype=dtype, seed=D)
    ref_o, ref_l = oracle_full(inp)
    out, lse = run_dense(inp, dtype)
    assert_dense_parity(dtype, out, lse, ref_o, ref_l)


@pytest.mark.parametrize("window", [1, 2, 17, 64, 65, 100])
def test_windows(gpu, window):
    lengths = [300, 5, 129, 64]
    inp = custom(lengths, T=sum(lengths), Hq=16, Hkv=2, D=64, window=window, dtype="bf16", sinks=True,
                 seed=window)
    ref_o, ref_l = oracle_full(inp)
    out, lse = run_dense(inp, "bf16")
    assert_dense_parity("bf16", out, lse, ref_o, ref_l)


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (5, 1)])
def test_fully_masked_lanes_beside_visible_ones(gpu, Hq, Hkv):
    """One query head per fold puts 32 consecutive tokens in a wave; with a short window the
    first key tile is fully masked for the wave's last tokens while visible to its first ones."""
    lengths = [40, 200, 300]
    inp = custom(lengths, T=540, Hq=Hq, Hkv=Hkv, D=128, window=9, dtype="bf16", sinks=False, seed=21)
    ref_o, ref_l = oracle_full(inp)
    out, lse = run_dense(inp, "bf16")
    assert_dense_parity("bf16", out, lse, ref_o, ref_l)


def test_window_one_returns_v(gpu):
    inp = custom([70, 3, 90], T=163, Hq=4, Hkv=1, D=128, window=1, dtype="f32", seed=3)
    out, _ = run_dense(inp, "f32")
    np.testing.assert_allclose(out, np.repeat(inp["v"], 4, axis=1), rtol=1e-6, atol=1e-6)


def test_window_at_least_document_length_is_bitwise_full_causal(gpu):
    inp = custom([250, 40, 123], T=413, Hq=8, Hkv=4, D=128, window=0, dtype="bf16", seed=4)
    o0, l0 = run_dense(inp, "bf16")
    o1, l1 = run_dense(inp, "bf16", window=250)
    o2, l2 = run_dense(inp, "bf16", window=100000)
    np.testing.assert_array_equal(o0, o1)
    np.testing.assert_array_equal(o0, o2)
    np.testing.assert_array_equal(l0, l1)


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (6, 1), (12, 2), (16, 1), (64, 1), (40, 8)])
def test_gqa_group_shapes(gpu, Hq, Hkv):
    lengths = [100, 37, 150]
    inp = custom(lengths, T=287, Hq=Hq, Hkv=Hkv, D=64, window=50, dtype="bf16", sinks=True, seed=Hq + Hkv)
    ref_o, ref_l = oracle_full(inp)
    out, lse = run_dense(inp, "bf16")
    assert_dense_parity("bf16", out, lse, ref_o, ref_l)


def test_zero_length_documents_head_and_tail_padding(gpu):
    q_lengths = [0, 40, 0, 0, 70, 1, 0]
    base = custom(q_lengths, T=130, Hq=8, Hkv=2, D=64, window=0, dtype="f32", sinks=True, seed=5)
    # shift every boundary by 9 tokens: tokens 0..8 sit before the first document
    base["cu_seqlens"] = base["cu_seqlens"] + 9
    ref_o, ref_l = oracle_full(base)
    out, lse = run_dense(base, "f32")
    assert np.all(out[:9] == 0) and np.all(np.isneginf(lse[:9]))
    assert np.all(out[9 + 111:] == 0) and np.all(np.isneginf(lse[9 + 111:]))
    assert_dense_parity("f32", out, lse, ref_o, ref_l)


def test_no_documents_means_all_padding(gpu):
    from sliding_window_gqa_varlen_amd import varlen_attn_fwd
    q = torch.randn(77, 4, 64, device=gpu, dtype=torch.bfloat16)
    k = torch.randn(77, 2, 64, device=gpu, dtype=torch.bfloat16)
    out = torch.full((77, 4, 64), float("nan"), device=gpu, dtype=torch.bfloat16)
    lse = torch.full((77, 4), 0.0, device=gpu)
    varlen_attn_fwd(q, k, k, None, 0, 0, 0.1, out=out, lse=lse)
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))


@pytest.mark.parametrize("n_docs", [61, 62, 90])
@pytest.mark.parametrize("D,window", [(128, 0), (64, 37)])
def test_many_documents_both_segment_decodes(gpu, n_docs, D, window):
    """Up to 61 documents the tile decode counts boundaries with one ballot, beyond that it
    binary-searches cu_seqlens; both, with empty documents and head and tail padding."""
    rng = np.random.default_rng(n_docs + D)
    lengths = [int(x) for x in rng.integers(0, 48, n_docs)]
    lengths[3] = lengths[n_docs // 2] = 0
    inp = custom(lengths, T=sum(lengths) + 20, Hq=8, Hkv=2, D=D, window=window, dtype="bf16",
                 sinks=window > 0, seed=n_docs)
    inp["cu_seqlens"] = inp["cu_seqlens"] + 7  # tokens 0..6 sit before the first document
    ref_o, ref_l = oracle_full(inp)
    out, lse = run_dense(inp, "bf16")
    assert_dense_parity("bf16", out, lse, ref_o, ref_l)
    assert np.all(out[:7] == 0) and np.all(np.isneginf(lse[:7]))


@pytest.mark.parametrize("lengths", [[4096, 1, 0, 2500, 517], [4097, 300, 64]])
def test_heaviest_first_tile_order_and_its_document_order_fallback(gpu, lengths):
    """With fewer head chunks than XCDs under a full causal mask the query tiles run heaviest
    first over all documents when every document has at most 64 key tiles (4096 tokens: 64
    weight levels, the first case, with an empty and a one-token document and head and tail
    padding), else in document order (the second case)."""
    inp = custom(lengths, T=sum(lengths) + 16, Hq=4, Hkv=2, D=64, window=0, dtype="bf16", seed=len(lengths))
    inp["cu_seqlens"] = inp["cu_seqlens"] + 5  # tokens 0..4 sit before the first document
    ref_o, ref_l = oracle_full(inp)
    out, lse = run_dense(inp, "bf16")
    assert_dense_parity("bf16", out, lse, ref_o, ref_l)
    end = 5 + sum(lengths)
    assert np.all(out[:5] == 0) and np.all(out[end:] == 0)
    assert np.all(np.isneginf(lse[:5])) and np.all(np.isneginf(lse[end:]))


@pytest.mark.parametrize("D,window,sinks", [(128, 0, False), (64, 0, True), (128, 300, True), (256, 0, False)])
def test_scores_growing_along_the_keys(gpu, D, window, sinks):
    """Every query's scores grow by 0.08 to 0.11 per key (5 to 7 per 64-key tile), so the
    running maximum keeps moving: the lazy reference is exceeded by more than 2^8 every few
    tiles and the O rescale runs inside the loop, not only on the first tile."""
    inp = custom([700, 333], T=1033, Hq=8, Hkv=2, D=D, window=window, dtype="bf16", sinks=sinks, seed=D + window)
    T = 1033
    pos = np.concatenate([np.arange(700), np.arange(333)]).astype(np.float32)
    u = np.ones(D, np.float32)
    # q . k = D * 0.01 * pos (+ noise); times scale = D^-1/2 the score grows by 0.01 sqrt(D) per key
    q = np.broadcast_to(u, (T, 8, D)) + 0.05 * inp["q"]
    k = (0.01 * pos)[:, None, None] * np.broadcast_to(u, (T, 2, D)) + 0.05 * inp["k"]
    inp["q"] = W.round_to_bf16(np.ascontiguousarray(q, np.float32))
    inp["k"] = W.round_to_bf16(np.ascontiguousarray(k, np.float32))
    ref_o, ref_l = oracle_full(inp)
    out, lse = run_dense(inp, "bf16")
    assert_dense_parity("bf16", out, lse, ref_o, ref_l)


@pytest.mark.parametrize("D,Hq,Hkv,size,where", [(64, 8, 2, 20, "end"), (128, 8, 2, 20, "end"), (128, 4, 4, 20, "end"),
                                                  (256, 8, 2, 20, "end"), (64, 8, 2, 200, "end"),
                                                  (128, 8, 2, 200, "end"), (128, 8, 2, 200, "middle"),
                                                  (64, 8, 2, 200, "middle")])
def test_score_jump_in_the_last_key_tile(gpu, D, Hq, Hkv, size, where):
    """Scores are flat except for 40 keys of each document, which score `size` above the rest.
    At the end of a document, the query tiles there meet them only in their last key tile, so the
    lazy reference moves after the pipelined loop (the last tile's exact path); in the middle
    (keys 100-139), inside the loop.  A jump of 200 (288 in log2 units) overflows the fast path's
    probabilities to inf, which must send the tile to the exact path, not into the output."""
    lengths = [300, 200, 170]
    T = sum(lengths)
    inp = custom(lengths, T=T, Hq=Hq, Hkv=Hkv, D=D, window=0, dtype="bf16", seed=D + Hq)
    sel = (lambda n: np.arange(n) >= n - 40) if where == "end" else (lambda n: (np.arange(n) >= 100) & (np.arange(n) < 140))
    jump = np.concatenate([sel(n) for n in lengths]).astype(np.float32) * (size / math.sqrt(D))
    u = np.ones(D, np.float32)
    q = np.broadcast_to(u, (T, Hq, D)) + 0.05 * inp["q"]
    k = jump[:, None, None] * np.broadcast_to(u, (T, Hkv, D)) + 0.05 * inp["k"]
    inp["q"] = W.round_to_bf16(np.ascontiguousarray(q, np.float32))
    inp["k"] = W.round_to_bf16(np.ascontiguousarray(k, np.float32))
    ref_o, ref_l = oracle_full(inp)
    out, lse = run_dense(inp, "bf16")
    assert_dense_parity("bf16", out, lse, ref_o, ref_l)


def test_single_token_documents(gpu):
    inp = custom([1] * 300, T=300, Hq=8, Hkv=8, D=128, window=0, dtype="f32", seed=6)
    out, lse = run_dense(inp, "f32")
    np.testing.assert_allclose(out, inp["v"].astype(np.float64), rtol=1e-6, atol=1e-6)
    qk = np.einsum("thd,thd->th", inp["q"].astype(np.float64), inp["k"].astype(np.float64))
    np.testing.assert_allclose(lse, qk * inp["scale"], rtol=1e-5, atol=1e-5)


def test_sink_of_minus_infinity_is_bitwise_no_sink(gpu):
    inp = custom([90, 200], T=290, Hq=8, Hkv=2, D=64, window=33, dtype="bf16", seed=7)
    o0, l0 = run_dense(inp, "bf16", sinks=None)
    o1, l1 = run_dense(inp, "bf16", sinks=np.full(8, -np.inf, np.float32))
    np.testing.assert_array_equal(o0, o1)
    np.testing.assert_array_equal(l0, l1)


def test_strided_views_of_a_fused_qkv_buffer(gpu):
    T, Hq, Hkv, D = 333, 8, 2, 128
    inp = custom([120, 213], T=T, Hq=Hq, Hkv=Hkv, D=D, window=64, dtype="bf16", sinks=True, seed=8)
    fused = torch.zeros(T, Hq + 2 * Hkv, D, device=gpu, dtype=torch.bfloat16)
    fused[:, :Hq] = dev(inp["q"], torch.bfloat16)
    fused[:, Hq:Hq + Hkv] = dev(inp["k"], torch.bfloat16)
    fused[:, Hq + Hkv:] = dev(inp["v"], torch.bfloat16)
    q, k, v = fused[:, :Hq], fused[:, Hq:Hq + Hkv], fused[:, Hq + Hkv:]
    big = torch.full((T, Hq + 3, D), 7.0, device=gpu, dtype=torch.bfloat16)
    out = big[:, 1:Hq + 1]
    cu = torch.from_numpy(inp["cu_seqlens"]).to(gpu)
    varlen_attn_fwd(q, k, v, cu, 2, 64, inp["scale"], torch.from_numpy(inp["sinks"]).to(gpu), out=out,
                    return_lse=False)
    torch.cuda.synchronize()
    assert torch.all(big[:, 0] == 7) and torch.all(big[:, Hq + 1:] == 7)  # neighbours untouched
    ref_o, _ = oracle_full(inp)
    err = np.abs(out.float().cpu().numpy() - ref_o).max()
    assert err <= BF16_MAX_ABS, err


def test_every_output_written_and_nothing_else(gpu):
    """NaN-filled outputs must come back finite; guard regions around them stay untouched."""
    inp = custom([500, 3, 90], T=600, Hq=8, Hkv=4, D=64, window=0, dtype="bf16", sinks=True, seed=9)
    T, Hq, D = 600, 8, 64
    guard = 4096
    obuf = torch.full((2 * guard + T * Hq * D,), float("nan"), device=gpu, dtype=torch.bfloat16)
    lbuf = torch.full((2 * guard + T * Hq,), float("nan"), device=gpu)
    out = obuf[guard:guard + T * Hq * D].view(T, Hq, D)
    lse = lbuf[guard:guard + T * Hq].view(T, Hq)
    q, k, v = (dev(inp[n], torch.bfloat16) for n in ("q", "k", "v"))
    cu = torch.from_numpy(inp["cu_seqlens"]).to(gpu)
    varlen_attn_fwd(q, k, v, cu, 3, 0, inp["scale"], torch.from_numpy(inp["sinks"]).to(gpu), out=out, lse=lse)
    torch.cuda.synchronize()
    assert torch.isnan(obuf[:guard]).all() and torch.isnan(obuf[-guard:]).all()
    assert torch.isnan(lbuf[:guard]).all() and torch.isnan(lbuf[-guard:]).all()
    assert not torch.isnan(out).any() and not torch.isnan(lse[:593]).any()
    assert torch.isneginf(lse[593:]).all() and (out[593:] == 0).all()


def test_repeat_runs_are_bitwise_identical(gpu):
    inp = W.make_dense(W.WORKLOADS[1].with_tokens(4096))
    o0, l0 = run_dense(inp, "bf16")
    o1, l1 = run_dense(inp, "bf16")
    np.testing.assert_array_equal(o0, o1)
    np.testing.assert_array_equal(l0, l1)


# ------------------------------------------------------------------ head_dim 256 (bf16)
def test_head_dim_256_ragged_causal(gpu):
    lengths = [1, 31, 33, 63, 65, 127, 129, 2, 200]
    inp = custom(lengths, T=sum(lengths) + 37, Hq=8, Hkv=2, D=256, window=0, dtype="bf16", seed=256)
    ref_o, ref_l = oracle_full(inp)
    out, lse = run_dense(inp, "bf16")
    assert_dense_parity("bf16", out, lse, ref_o, ref_l)


@pytest.mark.parametrize("window,sinks", [(65, True), (1, False), (300, True)])
def test_head_dim_256_windows_sinks_gqa(gpu, window, sinks):
    lengths = [300, 5, 129, 64]
    inp = custom(lengths, T=sum(lengths), Hq=16, Hkv=2, D=256, window=window, dtype="bf16", sinks=sinks,
                 seed=window + 1)
    ref_o, ref_l = oracle_full(inp)
    out, lse = run_dense(inp, "bf16")
    assert_dense_parity("bf16", out, lse, ref_o, ref_l)


def test_head_dim_256_packed_documents_elementwise(gpu):
    """2048 tokens in eight documents of 128..512 tokens, 16 query / 4 KV heads, full causal."""
    w = W.DenseWorkload("d256", "bf16", T=2048, Hq=16, Hkv=4, D=256, window=0, scale=1.0 / 16.0, seed=7,
                        doc_dist=("uniform", 128, 512))
    inp = W.make_dense(w)
    ref_o, ref_l = oracle_full(inp)
    out, lse = run_dense(inp, "bf16")
    assert_dense_parity("bf16", out, lse, ref_o, ref_l)


def test_head_dim_256_workload_full_size_every_row(gpu):
    """The 8192-token head_dim-256 causal workload exactly as bench times it, every row."""
    inp = W.make_dense([w for w in W.EXTRA_WORKLOADS if w.name == "causal_gqa_d256_bf16_t8192"][0])
    out, lse = run_dense(inp, "bf16")
    ref_o, ref_l = oracle_full(inp)
    assert_dense_parity("bf16", out, lse, ref_o, ref_l)
