"""GPU parity of sparse_mla_fwd (through the C ABI) against the fp64 oracle."""
import math

import numpy as np
import pytest
import torch

from oracle import sparse_mla_ref, sparse_mla_ref_rows, varlen_attn_ref
from sliding_window_gqa_varlen_amd import metrics, sparse_mla_fwd, workloads as W
from tests.golden_util import load
from tests.gpu_util import BF16_MAX_ABS, assert_lse_match, dev

pytestmark = pytest.mark.gpu


def run_sparse(inp, device="cuda:0", with_lse=True, indices=None, doc_ids=None, scale=None):
    q = dev(inp["q"], torch.bfloat16, device)
    lat = dev(inp["latent"], torch.bfloat16, device)
    kpe = dev(inp["k_pe"], torch.bfloat16, device)
    idx = torch.from_numpy(np.ascontiguousarray(inp["indices"] if indices is None else indices)).to(device)
    ids = torch.from_numpy(np.ascontiguousarray(inp["doc_ids"] if doc_ids is None else doc_ids)).to(device)
    out, lse = sparse_mla_fwd(q, lat, kpe, idx, ids, inp["scale"] if scale is None else scale, return_lse=with_lse)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), (None if lse is None else lse.cpu().numpy().astype(np.float64))


def check(out, lse, ref_o, ref_l):
    assert np.all(np.isfinite(out))
    err = np.abs(out - ref_o).max()
    assert err <= BF16_MAX_ABS, f"out max abs error {err:.3e}"
    if lse is not None:
        assert_lse_match(lse, ref_l, BF16_MAX_ABS)


def oracle(inp, indices=None, doc_ids=None):
    return sparse_mla_ref(inp["q"], inp["latent"], inp["k_pe"], inp["indices"] if indices is None else indices,
                          inp["doc_ids"] if doc_ids is None else doc_ids, inp["scale"])


def small(T, topk, seed=4, H=128, lengths=None, dist=("uniform", 64, 600), d_rope=64):
    w = W.SparseWorkload("sparse_small", T=T, H=H, d_latent=512, d_rope=d_rope, topk=topk, scale=1.0 / 24.0,
                         seed=seed, doc_dist=dist, doc_lengths=None if lengths is None else tuple(lengths))
    return W.make_sparse(w)


def test_hand_case_embedded(gpu):
    """The hand-derived sparse case (d_latent = d_rope = 1), embedded by zero padding."""
    for case in load("sparse_hand_cases.json"):
        T, H = case["T"], case["H"]
        Hp = 16
        q = np.zeros((T, Hp, 576), np.float32)
        lat = np.zeros((T, 512), np.float32)
        kpe = np.zeros((T, 64), np.float32)
        qc = np.array(case["q"], np.float32)
        q[:, :H, 0] = qc[..., 0]
        q[:, :H, 512] = qc[..., 1]
        lat[:, 0] = np.array(case["latent"])[:, 0]
        kpe[:, 0] = np.array(case["k_pe"])[:, 0]
        inp = dict(q=q, latent=lat, k_pe=kpe, indices=np.array(case["indices"], np.int32),
                   doc_ids=np.array(case["doc_ids"], np.int32), scale=case["scale"])
        out, lse = run_sparse(inp)
        exp_o = case["out_expected"][..., 0]
        np.testing.assert_allclose(out[:, :H, 0], exp_o, rtol=1e-2, atol=1e-2)
        assert np.all(out[:, :H, 1:] == 0)
        exp_l = case["lse_expected"]
        assert np.array_equal(np.isneginf(lse[:, :H]), np.isneginf(exp_l))
        fin = np.isfinite(exp_l)
        np.testing.assert_allclose(lse[:, :H][fin], exp_l[fin], rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("T,topk", [(300, 64), (700, 128), (1200, 256)])
def test_small_workloads_elementwise(gpu, T, topk):
    inp = small(T, topk, seed=T)
    ref_o, ref_l = oracle(inp)
    out, lse = run_sparse(inp)
    check(out, lse, ref_o, ref_l)


def test_full_size_workload_sampled(gpu):
    """The full-size workload as bench times it: 1000 random tokens plus document edges, every
    head of each (about 10 s of host time)."""
    inp = W.make_sparse(W.WORKLOADS[4])
    out, lse = run_sparse(inp)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    rng = np.random.default_rng(0)
    T = inp["q"].shape[0]
    cu = np.concatenate([[0], np.cumsum(inp["lengths"])])
    toks = list(rng.integers(0, T, 1000))
    for d in range(len(cu) - 1):
        s, e = int(cu[d]), int(cu[d + 1])
        toks += [s, s + 1, s + 31, s + 32, s + 2047, s + 2048, e - 1]
    toks = np.array(sorted(set(t for t in toks if 0 <= t < T)))
    ref_o, ref_l = sparse_mla_ref_rows(inp["q"], inp["latent"], inp["k_pe"], inp["indices"], inp["doc_ids"],
                                       inp["scale"], toks)
    check(out[toks], lse[toks], ref_o, ref_l)


def test_all_causal_keys_match_dense_attention(gpu):
    """Selecting every causal same-document key reproduces dense causal MQA (d_qk 576, d_v 512)."""
    lengths = [100, 37, 200]
    inp = small(337, 256, seed=11, lengths=lengths)
    k = np.concatenate([inp["latent"], inp["k_pe"]], axis=1)[:, None, :]
    v = np.concatenate([inp["latent"], np.zeros_like(inp["k_pe"])], axis=1)[:, None, :]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    ref_o, ref_l = varlen_attn_ref(inp["q"], k, v, cu, 0, inp["scale"])
    out, lse = run_sparse(inp)
    check(out, lse, ref_o[..., :512], ref_l)


def test_slot_order_padding_duplicates_and_violations(gpu):
    inp = small(500, 96, seed=12)
    base_o, base_l = run_sparse(inp)
    rng = np.random.default_rng(1)
    idx = inp["indices"]
    perm = np.stack([rng.permutation(idx.shape[1]) for _ in range(idx.shape[0])])
    shuffled = np.take_along_axis(idx, perm, axis=1)
    o1, l1 = run_sparse(inp, indices=shuffled)
    assert np.abs(o1 - base_o).max() <= BF16_MAX_ABS and np.abs(l1 - base_l)[np.isfinite(base_l)].max() <= 1e-4
    # contract violations (future keys, other documents, out of range) act like -1
    bad = idx.copy()
    T = bad.shape[0]
    for t in range(T):
        free = np.where(bad[t] < 0)[0]
        junk = [min(t + 1 + k, T + 5) for k in range(3)] + [T, -7, 10 ** 6]
        for f, j in zip(free, junk):
            bad[t, f] = j
    o2, l2 = run_sparse(inp, indices=bad)
    ref_o, ref_l = oracle(inp, indices=bad)
    check(o2, l2, ref_o, ref_l)
    # duplicated slots count once per slot
    dup = idx.copy()
    dup[:, -8:] = dup[:, :8]
    o3, l3 = run_sparse(inp, indices=dup)
    ref_o, ref_l = oracle(inp, indices=dup)
    check(o3, l3, ref_o, ref_l)


def test_empty_rows_and_padding_tokens(gpu):
    inp = small(200, 64, seed=13)
    idx = inp["indices"].copy()
    idx[50:60] = -1
    ids = inp["doc_ids"].copy()
    ids[190:] = -1
    out, lse = run_sparse(inp, indices=idx, doc_ids=ids)
    ref_o, ref_l = oracle(inp, indices=idx, doc_ids=ids)
    check(out, lse, ref_o, ref_l)
    assert np.all(out[50:60] == 0) and np.all(np.isneginf(lse[50:60]))
    assert np.all(out[190:] == 0) and np.all(np.isneginf(lse[190:]))


@pytest.mark.parametrize("H", [16, 48, 256])
def test_other_head_counts(gpu, H):
    inp = small(260, 80, seed=H, H=H)
    ref_o, ref_l = oracle(inp)
    out, lse = run_sparse(inp)
    check(out, lse, ref_o, ref_l)


def test_long_index_rows_span_segments(gpu):
    """topk above the 2048-slot compaction segment, with valid slots in every segment."""
    lengths = [3000, 1100]
    inp = small(4100, 2600, seed=14, lengths=lengths)
    toks = np.array([0, 5, 2047, 2048, 2599, 2600, 2999, 3000, 4099])
    out, lse = run_sparse(inp)
    ref_o, ref_l = sparse_mla_ref_rows(inp["q"], inp["latent"], inp["k_pe"], inp["indices"], inp["doc_ids"],
                                       inp["scale"], toks)
    check(out[toks], lse[toks], ref_o, ref_l)
    assert metrics.sparse_valid_slots(inp["indices"], inp["doc_ids"]) > 0


def test_scores_growing_along_the_slots(gpu):
    """Rotary key rows whose dot product with every query grows with the key position (the
    rotary part enters the scores but not the values, so outputs stay O(1)), and index rows in
    ascending order: the running maximum keeps moving chunk after chunk, so the lazy O rescale
    runs inside the chunk loop."""
    inp = small(T=1500, topk=512, lengths=[1500], seed=9)
    T = 1500
    pos = np.arange(T, dtype=np.float32)
    inp["k_pe"] = W.round_to_bf16((0.01 * pos)[:, None] + 0.05 * inp["k_pe"])
    q = inp["q"].copy()
    q[:, :, 512:] = 1.0
    inp["q"] = W.round_to_bf16(q)
    ref_o, ref_l = oracle(inp)
    out, lse = run_sparse(inp)
    check(out, lse, ref_o, ref_l)


@pytest.mark.parametrize("size", [20.0, 200.0])
def test_score_jump_in_the_middle_of_the_index_rows(gpu, size):
    """Rotary key rows from position 700 on raise every query's score by `size` (natural-log
    units; the rotary part enters the scores but not the values).  Ascending index rows meet the
    jump mid-row, so a chunk's probabilities against the running reference exceed the bound of
    the path that skips the chunk maximum (for 200, 288 log2 units, they overflow to inf) and
    that chunk must take the exact path with its maximum."""
    inp = small(T=1500, topk=512, lengths=[1500], seed=19)
    kpe = 0.05 * inp["k_pe"]
    kpe[700:] += size * 24.0 / 64.0  # 64 rotary coordinates, q = 1 there, scale 1/24
    inp["k_pe"] = W.round_to_bf16(np.ascontiguousarray(kpe, np.float32))
    q = inp["q"].copy()
    q[:, :, 512:] = 1.0
    inp["q"] = W.round_to_bf16(q)
    ref_o, ref_l = oracle(inp)
    assert ref_l[1000:].min() > size - 5.0  # the jump dominates the rows that reach it
    out, lse = run_sparse(inp)
    check(out, lse, ref_o, ref_l)


def test_repeat_runs_are_bitwise_identical(gpu):
    inp = small(400, 128, seed=15)
    o0, l0 = run_sparse(inp)
    o1, l1 = run_sparse(inp)
    np.testing.assert_array_equal(o0, o1)
    np.testing.assert_array_equal(l0, l1)


# ---------------------------------------------------------------- NoPE variant (no rotary part)
@pytest.mark.parametrize("T,topk,H", [(300, 64, 128), (1200, 256, 128), (700, 128, 48)])
def test_nope_small_workloads_elementwise(gpu, T, topk, H):
    inp = small(T, topk, seed=T + 1, H=H, d_rope=0)
    assert inp["q"].shape[2] == 512 and inp["k_pe"].shape == (T, 0)
    ref_o, ref_l = oracle(inp)
    out, lse = run_sparse(inp)
    check(out, lse, ref_o, ref_l)


def test_nope_all_causal_keys_match_dense_attention(gpu):
    """NoPE with every causal same-document key selected is dense causal MQA with d_qk = d_v = 512."""
    lengths = [90, 250, 17]
    inp = small(357, 256, seed=16, lengths=lengths, d_rope=0)
    k = inp["latent"][:, None, :]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    ref_o, ref_l = varlen_attn_ref(inp["q"], k, k, cu, 0, inp["scale"])
    out, lse = run_sparse(inp)
    check(out, lse, ref_o, ref_l)


def test_nope_full_size_sampled(gpu):
    """The sparse workload's shape and index rows without the rotary part, on sampled tokens."""
    import dataclasses
    w = dataclasses.replace(W.WORKLOADS[4], name="sparse_mla_nope", d_rope=0, scale=1.0 / math.sqrt(512.0))
    inp = W.make_sparse(w)
    out, lse = run_sparse(inp)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    T = inp["q"].shape[0]
    cu = np.concatenate([[0], np.cumsum(inp["lengths"])])
    rng = np.random.default_rng(2)
    toks = list(rng.integers(0, T, 500))
    for d in range(len(cu) - 1):
        s, e = int(cu[d]), int(cu[d + 1])
        toks += [s, s + 31, s + 2048, e - 1]
    toks = np.array(sorted(set(t for t in toks if 0 <= t < T)))
    ref_o, ref_l = sparse_mla_ref_rows(inp["q"], inp["latent"], inp["k_pe"], inp["indices"], inp["doc_ids"],
                                       inp["scale"], toks)
    check(out[toks], lse[toks], ref_o, ref_l)


def torch_sparse_rows(q, lat, kpe, idx, ids, scale, t0, t1):
    """A plain fp32 restatement of the sparse MLA definition on the GPU (torch ops only) for
    tokens t0 .. t1 - 1: slot k of token t is valid iff 0 <= idx < T, idx <= t and both tokens
    lie in the same document (doc id >= 0); scores scale * q . [latent, k_pe] over the valid
    slots; out = softmax-weighted latent rows, lse = log of the denominator; empty rows give
    zeros and -inf."""
    T = q.shape[0]
    ii = idx[t0:t1].long()
    tt = torch.arange(t0, t1, device=q.device)[:, None]
    ic = ii.clamp(0, T - 1)
    valid = (ii >= 0) & (ii < T) & (ii <= tt) & (ids[ic] == ids[t0:t1, None]) & (ids[t0:t1, None] >= 0)
    keys = torch.cat([lat, kpe], dim=1)[ic]                                  # [C, K, 512 + d_rope]
    s = torch.bmm(q[t0:t1], keys.transpose(1, 2).contiguous()) * scale        # [C, H, K]
    s = s.masked_fill(~valid[:, None, :], float("-inf"))
    lse = torch.logsumexp(s, dim=-1)                                          # -inf for empty rows
    p = torch.exp(s - lse[..., None]).nan_to_num(0.0)
    out = torch.bmm(p, lat[ic].contiguous())                                  # [C, H, 512]
    return out, lse


def full_rows_against_torch(inp, chunk=256, n_pin=48, seed=5):
    """Every row of the full-size kernel output against torch_sparse_rows; that reference is first
    pinned to the fp64 oracle on sampled tokens."""
    f = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to("cuda:0").float()
    q, lat, kpe = f(inp["q"]), f(inp["latent"]), f(inp["k_pe"])
    idx = torch.from_numpy(np.ascontiguousarray(inp["indices"])).to("cuda:0")
    ids = torch.from_numpy(np.ascontiguousarray(inp["doc_ids"])).to("cuda:0")
    T = q.shape[0]
    rng = np.random.default_rng(seed)
    pin = np.unique(rng.integers(0, T, n_pin))
    ref_o, ref_l = sparse_mla_ref_rows(inp["q"], inp["latent"], inp["k_pe"], inp["indices"], inp["doc_ids"],
                                       inp["scale"], pin)
    for j, t in enumerate(pin):
        o_t, l_t = torch_sparse_rows(q, lat, kpe, idx, ids, inp["scale"], int(t), int(t) + 1)
        np.testing.assert_allclose(o_t[0].cpu().numpy(), ref_o[j], rtol=0, atol=1e-4)
        assert_lse_match(l_t[0].cpu().numpy().astype(np.float64), ref_l[j], 1e-4, "torch reference lse")
    out, lse = run_sparse(inp)
    worst_o, worst_l = 0.0, 0.0
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        o_ref, l_ref = torch_sparse_rows(q, lat, kpe, idx, ids, inp["scale"], t0, t1)
        o_ref, l_ref = o_ref.cpu().numpy(), l_ref.cpu().numpy().astype(np.float64)
        worst_o = max(worst_o, float(np.abs(out[t0:t1] - o_ref).max()))
        assert_lse_match(lse[t0:t1], l_ref, BF16_MAX_ABS)
        fin = np.isfinite(l_ref)
        if fin.any():
            worst_l = max(worst_l, float(np.abs(lse[t0:t1][fin] - l_ref[fin]).max()))
    assert worst_o <= BF16_MAX_ABS, f"out max abs error {worst_o:.3e} over all rows"
    return worst_o, worst_l


def test_full_size_every_row_against_a_pinned_gpu_fp32_reference(gpu):
    """All 16384 x 128 rows of the full-size workload (the oracle finishes only sampled rows at
    this size)."""
    full_rows_against_torch(W.make_sparse(W.WORKLOADS[4]))


def test_nope_full_size_every_row_against_a_pinned_gpu_fp32_reference(gpu):
    import dataclasses
    w = dataclasses.replace(W.WORKLOADS[4], name="sparse_mla_nope", d_rope=0, scale=1.0 / math.sqrt(512.0))
    full_rows_against_torch(W.make_sparse(w))
