"""Pins for the sparse MLA fp64 oracle: hand cases, reduction to dense, slot invariances."""
import numpy as np
import pytest

from oracle import mla_value_proj_ref, sparse_mla_ref, sparse_mla_ref_rows, sparse_mla_value_ref, varlen_attn_ref
from tests.golden_util import load


def rand_sparse(lengths, H=3, d_l=6, d_r=2, topk=None, seed=0):
    rng = np.random.default_rng(seed)
    T = int(sum(lengths))
    q = rng.standard_normal((T, H, d_l + d_r))
    latent = rng.standard_normal((T, d_l))
    k_pe = rng.standard_normal((T, d_r))
    doc_ids = np.repeat(np.arange(len(lengths)), lengths).astype(np.int32)
    return q, latent, k_pe, doc_ids


def all_causal_indices(lengths, topk):
    T = int(sum(lengths))
    idx = np.full((T, topk), -1, dtype=np.int32)
    s = 0
    for L in lengths:
        for p in range(L):
            idx[s + p, :p + 1] = np.arange(s, s + p + 1)
        s += L
    return idx


@pytest.mark.parametrize("case", load("sparse_hand_cases.json"), ids=lambda c: c["name"])
def test_hand_cases(case):
    q = np.array(case["q"], dtype=np.float64)
    latent = np.array(case["latent"], dtype=np.float64)
    k_pe = np.array(case["k_pe"], dtype=np.float64)
    idx = np.array(case["indices"], dtype=np.int32)
    ids = np.array(case["doc_ids"], dtype=np.int32)
    out, lse = sparse_mla_ref(q, latent, k_pe, idx, ids, case["scale"])
    np.testing.assert_allclose(out, case["out_expected"], rtol=0, atol=1e-14)
    assert np.array_equal(np.isneginf(lse), np.isneginf(case["lse_expected"]))
    fin = np.isfinite(lse)
    np.testing.assert_allclose(lse[fin], case["lse_expected"][fin], rtol=0, atol=1e-14)
    o2, l2 = sparse_mla_ref_rows(q, latent, k_pe, idx, ids, case["scale"], np.arange(case["T"]))
    np.testing.assert_array_equal(o2, out)
    np.testing.assert_array_equal(l2, lse)


def test_all_causal_keys_selected_equals_dense_causal_mqa():
    """The expanded-KV reference: selecting every causal same-document key is dense attention."""
    lengths = [5, 12, 1, 9]
    H, d_l, d_r = 4, 8, 3
    q, latent, k_pe, ids = rand_sparse(lengths, H, d_l, d_r, seed=1)
    idx = all_causal_indices(lengths, 16)
    out, lse = sparse_mla_ref(q, latent, k_pe, idx, ids, 0.3)
    # dense MQA: one KV head, key = [latent, k_pe], value = [latent, 0]
    k = np.concatenate([latent, k_pe], axis=1)[:, None, :]
    v = np.concatenate([latent, np.zeros_like(k_pe)], axis=1)[:, None, :]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    od, ld = varlen_attn_ref(q, k, v, cu, 0, 0.3)
    np.testing.assert_allclose(out, od[..., :d_l], rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, ld, rtol=0, atol=1e-13)
    assert np.all(od[..., d_l:] == 0)


def test_slot_order_and_padding_do_not_matter():
    lengths = [20, 15]
    q, latent, k_pe, ids = rand_sparse(lengths, seed=2)
    rng = np.random.default_rng(3)
    T = 35
    idx = np.full((T, 8), -1, dtype=np.int32)
    s = 0
    for L in lengths:
        for p in range(L):
            n = min(p + 1, 6)
            idx[s + p, :n] = s + rng.choice(p + 1, n, replace=False)
        s += L
    o0, l0 = sparse_mla_ref(q, latent, k_pe, idx, ids, 0.5)
    perm = np.stack([rng.permutation(8) for _ in range(T)])
    idx_p = np.take_along_axis(idx, perm, axis=1)
    o1, l1 = sparse_mla_ref(q, latent, k_pe, idx_p, ids, 0.5)
    np.testing.assert_allclose(o1, o0, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l1, l0, rtol=0, atol=1e-13)
    idx_w = np.concatenate([np.full((T, 3), -1, np.int32), idx, np.full((T, 2), -1, np.int32)], axis=1)
    o2, l2 = sparse_mla_ref(q, latent, k_pe, idx_w, ids, 0.5)
    np.testing.assert_array_equal(o2, o0)
    np.testing.assert_array_equal(l2, l0)


def test_boundary_violating_slots_are_ignored():
    """Future keys, other documents' keys and out-of-range indices act like -1."""
    lengths = [10, 10]
    q, latent, k_pe, ids = rand_sparse(lengths, seed=4)
    base = all_causal_indices(lengths, 10)
    o0, l0 = sparse_mla_ref(q, latent, k_pe, base, ids, 0.7)
    bad = base.copy()
    for t in range(20):
        row = bad[t]
        free = np.where(row < 0)[0]
        junk = [t + 1 if t + 1 < 20 else -5, 19 - t if ids[19 - t] != ids[t] else 1000, 20, -2]
        for f, j in zip(free, junk):
            row[f] = j
    o1, l1 = sparse_mla_ref(q, latent, k_pe, bad, ids, 0.7)
    np.testing.assert_array_equal(o1, o0)
    np.testing.assert_array_equal(l1, l0)


def test_duplicate_slots_count_twice():
    lengths = [4]
    q, latent, k_pe, ids = rand_sparse(lengths, H=1, seed=5)
    idx = np.array([[0, -1], [0, 1], [2, 2], [3, 0]], dtype=np.int32)
    out, lse = sparse_mla_ref(q, latent, k_pe, idx, ids, 1.0)
    s22 = float(q[2, 0, :6] @ latent[2] + q[2, 0, 6:] @ k_pe[2])
    # two copies of one key: weight 1 on that row, log-sum-exp gains log 2
    np.testing.assert_allclose(out[2, 0], latent[2], rtol=0, atol=1e-14)
    assert lse[2, 0] == pytest.approx(s22 + np.log(2.0), abs=1e-13)


def test_padding_query_tokens_are_empty():
    lengths = [3]
    q, latent, k_pe, _ = rand_sparse([5], seed=6)
    ids = np.array([0, 0, 0, -1, -1], dtype=np.int32)
    idx = all_causal_indices([5], 5)
    out, lse = sparse_mla_ref(q, latent, k_pe, idx, ids, 1.0)
    assert np.all(out[3:] == 0) and np.all(np.isneginf(lse[3:]))
    assert np.all(np.isfinite(lse[:3]))


def test_nope_rows_equal_dense_without_rotary_part():
    """NoPE layers (k_pe [T, 0], q of width d_l): the all-causal selection is dense MQA on latent."""
    lengths = [7, 3, 11]
    H, d_l = 2, 8
    q, latent, k_pe, ids = rand_sparse(lengths, H, d_l, 0, seed=9)
    assert k_pe.shape[1] == 0
    idx = all_causal_indices(lengths, 12)
    out, lse = sparse_mla_ref(q, latent, k_pe, idx, ids, 0.45)
    cu = np.concatenate([[0], np.cumsum(lengths)])
    od, ld = varlen_attn_ref(q, latent[:, None, :], latent[:, None, :], cu, 0, 0.45)
    np.testing.assert_allclose(out, od, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, ld, rtol=0, atol=1e-13)


def test_value_projection_scalar_loop():
    """out_v[t, h, v] = sum_d value_weight[h, v, d] * o[t, h, d], written as a scalar loop."""
    rng = np.random.default_rng(21)
    T, H, d_l, d_v = 3, 2, 5, 4
    o = rng.standard_normal((T, H, d_l))
    w = rng.standard_normal((H, d_v, d_l))
    got = mla_value_proj_ref(o, w)
    for t in range(T):
        for h in range(H):
            for v in range(d_v):
                acc = 0.0
                for d in range(d_l):
                    acc += w[h, v, d] * o[t, h, d]
                assert got[t, h, v] == pytest.approx(acc, abs=1e-12)


def test_value_projection_identity_and_zero_heads():
    """[I | 0] weights copy the first d_v latent coordinates; a zero head gives zeros."""
    rng = np.random.default_rng(22)
    T, H, d_l, d_v = 6, 3, 10, 4
    o = rng.standard_normal((T, H, d_l))
    w = np.zeros((H, d_v, d_l))
    w[0, :, :d_v] = np.eye(d_v)
    w[2, :, d_l - d_v:] = np.eye(d_v)  # the last d_v coordinates, in order
    got = mla_value_proj_ref(o, w)
    np.testing.assert_array_equal(got[:, 0], o[:, 0, :d_v])
    np.testing.assert_array_equal(got[:, 1], np.zeros((T, d_v)))
    np.testing.assert_array_equal(got[:, 2], o[:, 2, d_l - d_v:])


def test_sparse_mla_value_composes_and_keeps_empty_rows_zero():
    lengths = [6, 4]
    H, d_l, d_r, d_v = 3, 6, 2, 5
    q, latent, k_pe, ids = rand_sparse(lengths, H, d_l, d_r, seed=23)
    idx = all_causal_indices(lengths, 6)
    idx[4] = -1  # an empty query row
    w = np.random.default_rng(24).standard_normal((H, d_v, d_l))
    out_v, lse = sparse_mla_value_ref(q, latent, k_pe, idx, ids, w, 0.6)
    o, l = sparse_mla_ref(q, latent, k_pe, idx, ids, 0.6)
    np.testing.assert_allclose(out_v, np.einsum("hvd,thd->thv", w, o), rtol=0, atol=1e-12)
    np.testing.assert_array_equal(lse, l)
    assert np.all(out_v[4] == 0) and np.isneginf(lse[4]).all()
