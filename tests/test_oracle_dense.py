"""Pins for the dense fp64 oracle: hand cases, closed forms, invariants, brute force, SDPA.

None of these re-types the oracle's formula: each checks it against something
the definition fixes independently (a hand-derived value, a special case with
a known answer, a symmetry, a second code path or torch's own attention).
"""
import math

import numpy as np
import pytest
import torch

from oracle import varlen_attn_bruteforce, varlen_attn_ref, varlen_attn_ref_rows
from tests.golden_util import load


def rand_problem(lengths, T=None, Hq=4, Hkv=2, D=8, seed=0, sinks=False):
    rng = np.random.default_rng(seed)
    T = T if T is not None else int(sum(lengths))
    q = rng.standard_normal((T, Hq, D))
    k = rng.standard_normal((T, Hkv, D))
    v = rng.standard_normal((T, Hkv, D))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    s = rng.standard_normal(Hq) if sinks else None
    return q, k, v, cu, s


def assert_lse_equal(a, b, tol=1e-12):
    assert np.array_equal(np.isneginf(a), np.isneginf(b))
    fin = np.isfinite(a)
    np.testing.assert_allclose(a[fin], b[fin], rtol=0, atol=tol)


# --------------------------------------------------------------------------- hand cases
@pytest.mark.parametrize("case", load("dense_hand_cases.json"), ids=lambda c: c["name"])
def test_hand_cases(case):
    q = np.array(case["q"], dtype=np.float64)
    k = np.array(case["k"], dtype=np.float64)
    v = np.array(case["v"], dtype=np.float64)
    sinks = None if case["sinks"] is None else np.array(case["sinks"])
    out, lse = varlen_attn_ref(q, k, v, case["cu_seqlens"], case["window"], case["scale"], sinks)
    np.testing.assert_allclose(out[..., 0], case["out_expected"], rtol=0, atol=1e-14)
    assert_lse_equal(lse, case["lse_expected"], 1e-14)
    # the row-wise variant and the brute-force path must agree with the same closed forms
    T, Hq = lse.shape
    tok, hd = np.meshgrid(np.arange(T), np.arange(Hq), indexing="ij")
    o2, l2 = varlen_attn_ref_rows(q, k, v, case["cu_seqlens"], case["window"], case["scale"], sinks,
                                  tok.ravel(), hd.ravel())
    np.testing.assert_allclose(o2[:, 0].reshape(T, Hq), case["out_expected"], rtol=0, atol=1e-14)
    assert_lse_equal(l2.reshape(T, Hq), case["lse_expected"], 1e-14)
    o3, l3 = varlen_attn_bruteforce(q, k, v, case["cu_seqlens"], case["window"], case["scale"], sinks)
    np.testing.assert_allclose(o3[..., 0], case["out_expected"], rtol=0, atol=1e-14)
    assert_lse_equal(l3, case["lse_expected"], 1e-14)


# --------------------------------------------------------------------------- closed forms
def test_one_token_documents_return_their_v_row():
    q, k, v, cu, _ = rand_problem([1] * 7, Hq=6, Hkv=3, D=5, seed=1)
    out, lse = varlen_attn_ref(q, k, v, cu, 0, 0.37)
    for t in range(7):
        for h in range(6):
            g = h // 2
            np.testing.assert_allclose(out[t, h], v[t, g], rtol=0, atol=1e-14)
            assert lse[t, h] == pytest.approx(0.37 * float(q[t, h] @ k[t, g]), abs=1e-13)


def test_one_token_with_sink_is_a_sigmoid():
    q, k, v, cu, s = rand_problem([1] * 5, Hq=2, Hkv=1, D=3, seed=2, sinks=True)
    out, lse = varlen_attn_ref(q, k, v, cu, 0, 0.5, s)
    for t in range(5):
        for h in range(2):
            sc = 0.5 * float(q[t, h] @ k[t, 0])
            p = 1.0 / (1.0 + math.exp(s[h] - sc))
            np.testing.assert_allclose(out[t, h], p * v[t, 0], rtol=1e-13, atol=1e-14)
            assert lse[t, h] == pytest.approx(math.log(math.exp(sc) + math.exp(s[h])), abs=1e-13)


@pytest.mark.parametrize("window", [0, 1, 3, 10])
def test_tied_scores_average_the_visible_values(window):
    lengths = [9, 4]
    q, k, v, cu, _ = rand_problem(lengths, Hq=2, Hkv=2, D=4, seed=3)
    k[:] = 0.0  # every score ties at 0
    out, lse = varlen_attn_ref(q, k, v, cu, window, 1.3)
    start = 0
    for L in lengths:
        for p in range(L):
            t = start + p
            lo = start if window == 0 else max(start, t - window + 1)
            n = t - lo + 1
            for h in range(2):
                np.testing.assert_allclose(out[t, h], v[lo:t + 1, h].mean(axis=0), rtol=0, atol=1e-13)
                assert lse[t, h] == pytest.approx(math.log(n), abs=1e-13)
        start += L


# --------------------------------------------------------------------------- invariants
@pytest.mark.parametrize("window", [0, 2, 5])
def test_packing_equals_running_documents_separately(window):
    lengths = [3, 11, 1, 7]
    q, k, v, cu, s = rand_problem(lengths, Hq=4, Hkv=2, D=6, seed=4, sinks=True)
    out, lse = varlen_attn_ref(q, k, v, cu, window, 0.4, s)
    start = 0
    for L in lengths:
        sl = slice(start, start + L)
        o1, l1 = varlen_attn_ref(q[sl], k[sl], v[sl], [0, L], window, 0.4, s)
        np.testing.assert_allclose(out[sl], o1, rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse[sl], l1, rtol=0, atol=1e-14)
        start += L


def test_window_at_least_document_length_equals_full_causal():
    lengths = [6, 13, 2]
    q, k, v, cu, s = rand_problem(lengths, seed=5, sinks=True)
    o0, l0 = varlen_attn_ref(q, k, v, cu, 0, 0.3, s)
    for w in (13, 14, 100):
        o1, l1 = varlen_attn_ref(q, k, v, cu, w, 0.3, s)
        np.testing.assert_array_equal(o0, o1)
        np.testing.assert_array_equal(l0, l1)
    # a window shorter than the longest document does change the result
    o2, _ = varlen_attn_ref(q, k, v, cu, 12, 0.3, s)
    assert np.abs(o2 - o0).max() > 1e-6


def test_window_one_is_self_attention():
    q, k, v, cu, _ = rand_problem([5, 8], Hq=4, Hkv=1, seed=6)
    out, lse = varlen_attn_ref(q, k, v, cu, 1, 0.9)
    for h in range(4):
        np.testing.assert_allclose(out[:, h], v[:, 0], rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse[:, h], 0.9 * np.einsum("td,td->t", q[:, h], k[:, 0]), atol=1e-13)


def test_sink_of_minus_infinity_equals_no_sink():
    q, k, v, cu, _ = rand_problem([4, 9], seed=7)
    o0, l0 = varlen_attn_ref(q, k, v, cu, 3, 0.5)
    o1, l1 = varlen_attn_ref(q, k, v, cu, 3, 0.5, np.full(4, -np.inf))
    np.testing.assert_array_equal(o0, o1)
    np.testing.assert_array_equal(l0, l1)


def test_gqa_equals_mha_on_repeated_kv():
    q, k, v, cu, s = rand_problem([5, 12], Hq=6, Hkv=2, D=4, seed=8, sinks=True)
    o0, l0 = varlen_attn_ref(q, k, v, cu, 4, 0.7, s)
    k_rep = np.repeat(k, 3, axis=1)  # repeat_kv: KV head g serves query heads 3g..3g+2
    v_rep = np.repeat(v, 3, axis=1)
    o1, l1 = varlen_attn_ref(q, k_rep, v_rep, cu, 4, 0.7, s)
    np.testing.assert_allclose(o0, o1, rtol=0, atol=1e-14)
    np.testing.assert_allclose(l0, l1, rtol=0, atol=1e-14)


def test_constant_values_leave_the_sink_share():
    q, k, v, cu, s = rand_problem([6, 3], Hq=2, Hkv=1, seed=9, sinks=True)
    v[:] = 1.0
    out, lse = varlen_attn_ref(q, k, v, cu, 0, 0.8, s)
    p_sink = np.exp(s[None, :] - lse)
    np.testing.assert_allclose(out[..., 0], 1.0 - p_sink, rtol=0, atol=1e-13)
    # adding c to every V row adds c * (1 - p_sink)
    q, k, v, cu, s = rand_problem([6, 3], Hq=2, Hkv=1, seed=9, sinks=True)
    o0, l0 = varlen_attn_ref(q, k, v, cu, 0, 0.8, s)
    o1, _ = varlen_attn_ref(q, k, v + 2.5, cu, 0, 0.8, s)
    expect = 2.5 * (1.0 - np.exp(s[None, :] - l0))[..., None]
    np.testing.assert_allclose(o1 - o0, np.broadcast_to(expect, o0.shape), rtol=0, atol=1e-12)


def test_lse_bounds_the_largest_visible_score():
    lengths = [7, 10]
    q, k, v, cu, _ = rand_problem(lengths, Hq=2, Hkv=1, seed=10)
    _, lse = varlen_attn_ref(q, k, v, cu, 4, 1.0)
    start = 0
    for L in lengths:
        for p in range(L):
            t = start + p
            lo = max(start, t - 3)
            for h in range(2):
                sc = k[lo:t + 1, 0] @ q[t, h]
                assert lse[t, h] >= sc.max() - 1e-12
                assert lse[t, h] <= sc.max() + math.log(len(sc)) + 1e-12
        start += L


# --------------------------------------------------------------------------- second code paths
@pytest.mark.parametrize("seed", range(6))
def test_bruteforce_mask_path_agrees(seed):
    rng = np.random.default_rng(100 + seed)
    n_docs = int(rng.integers(1, 6))
    lengths = [int(x) for x in rng.integers(0, 14, n_docs)]
    pad = int(rng.integers(0, 4))
    Hkv = int(rng.choice([1, 2, 3]))
    G = int(rng.choice([1, 2, 4]))
    window = int(rng.choice([0, 1, 2, 5, 20]))
    q, k, v, cu, s = rand_problem(lengths, T=sum(lengths) + pad, Hq=Hkv * G, Hkv=Hkv, D=5,
                                  seed=seed, sinks=bool(seed % 2))
    o0, l0 = varlen_attn_ref(q, k, v, cu, window, 0.6, s, block=4)
    o1, l1 = varlen_attn_bruteforce(q, k, v, cu, window, 0.6, s)
    np.testing.assert_allclose(o0, o1, rtol=0, atol=1e-13)
    assert_lse_equal(l0, l1, 1e-13)


@pytest.mark.parametrize("window,sinks", [(0, False), (3, False), (0, True), (6, True)])
def test_torch_sdpa_fp64_cross_check(window, sinks):
    lengths = [13, 1, 20, 6]
    Hq, Hkv, D = 6, 2, 16
    q, k, v, cu, s = rand_problem(lengths, Hq=Hq, Hkv=Hkv, D=D, seed=11, sinks=sinks)
    out, lse = varlen_attn_ref(q, k, v, cu, window, 0.25, s, block=8)
    G = Hq // Hkv
    start = 0
    for L in lengths:
        sl = slice(start, start + L)
        qt = torch.from_numpy(q[sl]).permute(1, 0, 2)                      # [Hq, L, D]
        kt = torch.from_numpy(np.repeat(k[sl], G, axis=1)).permute(1, 0, 2)
        vt = torch.from_numpy(np.repeat(v[sl], G, axis=1)).permute(1, 0, 2)
        i = torch.arange(L)[:, None]
        j = torch.arange(L)[None, :]
        allow = j <= i
        if window:
            allow &= (i - j) < window
        if sinks:
            # sink = one extra key whose score is the sink logit and whose value is zero
            bias = torch.where(allow, 0.0, -math.inf).to(torch.float64)
            bias = bias[None].repeat(Hq, 1, 1)
            sink_col = torch.from_numpy(s)[:, None, None].expand(Hq, L, 1)
            bias = torch.cat([bias, sink_col], dim=2)
            kt = torch.cat([kt, torch.zeros(Hq, 1, D, dtype=torch.float64)], dim=1)
            vt = torch.cat([vt, torch.zeros(Hq, 1, D, dtype=torch.float64)], dim=1)
            # the zero key scores 0, so the bias alone sets the (unscaled) sink logit
            ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=bias, scale=0.25)
        else:
            ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=allow, scale=0.25)
        np.testing.assert_allclose(out[sl], ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)
        start += L


def test_row_variant_matches_block_variant():
    lengths = [40, 3, 77]
    q, k, v, cu, s = rand_problem(lengths, T=125, Hq=8, Hkv=2, D=8, seed=12, sinks=True)
    o0, l0 = varlen_attn_ref(q, k, v, cu, 9, 0.35, s, block=16)
    rng = np.random.default_rng(0)
    tok = rng.integers(0, 125, 60)
    hd = rng.integers(0, 8, 60)
    o1, l1 = varlen_attn_ref_rows(q, k, v, cu, 9, 0.35, s, tok, hd)
    np.testing.assert_allclose(o1, o0[tok, hd], rtol=0, atol=1e-13)
    assert_lse_equal(l1, l0[tok, hd], 1e-13)


def test_padding_tokens_are_zero_with_minus_inf_lse():
    q, k, v, cu, s = rand_problem([3, 4], T=10, seed=13, sinks=True)
    out, lse = varlen_attn_ref(q, k, v, cu, 0, 1.0, s)
    assert np.all(out[7:] == 0) and np.all(np.isneginf(lse[7:]))
    assert np.all(np.isfinite(lse[:7]))
