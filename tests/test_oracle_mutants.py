"""Plant one mistake at a time in a copy of the oracle's source and show the pins catch it.

Each mutant is a plausible slip (an off-by-one window, a wrong GQA head map, a
dropped or scaled sink, a transposed operand, a missing scale, a leaked
document boundary ...).  The pin battery is the same evidence the oracle is
trusted on: hand-derived closed forms, the brute-force mask path and torch's
fp64 SDPA.  Only copies are mutated, on the CPU.
"""
import math
import os
import types

import numpy as np
import pytest
import torch

import oracle.dense
import oracle.mask
import oracle.sparse
from tests.golden_util import load

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def mutated(module, old, new):
    """Copy of ``module`` with each ``old`` snippet replaced by ``new`` (str or tuples of str)."""
    src = open(module.__file__).read()
    olds = (old,) if isinstance(old, str) else old
    news = (new,) if isinstance(new, str) else new
    for o, n in zip(olds, news):
        assert src.count(o) >= 1, f"mutation anchor not found: {o!r}"
        src = src.replace(o, n)
    mod = types.ModuleType(module.__name__ + "_mutant")
    mod.__file__ = module.__file__
    exec(compile(src, module.__file__, "exec"), mod.__dict__)
    return mod


def _close(a, b, tol=1e-12):
    a, b = np.asarray(a, float), np.asarray(b, float)
    if a.shape != b.shape or not np.array_equal(np.isneginf(a), np.isneginf(b)):
        return False
    fin = np.isfinite(a) & np.isfinite(b)
    return bool(np.all(np.abs(a[fin] - b[fin]) <= tol)) and np.array_equal(np.isfinite(a), np.isfinite(b))


def dense_pins_hold(mod) -> bool:
    try:
        for c in load("dense_hand_cases.json"):
            q, k, v = (np.array(c[n], dtype=np.float64) for n in ("q", "k", "v"))
            s = None if c["sinks"] is None else np.array(c["sinks"])
            o, l = mod.varlen_attn_ref(q, k, v, c["cu_seqlens"], c["window"], c["scale"], s)
            if not (_close(o[..., 0], c["out_expected"]) and _close(l, c["lse_expected"])):
                return False
            T, Hq = l.shape
            tok, hd = np.meshgrid(np.arange(T), np.arange(Hq), indexing="ij")
            o2, l2 = mod.varlen_attn_ref_rows(q, k, v, c["cu_seqlens"], c["window"], c["scale"], s,
                                              tok.ravel(), hd.ravel())
            if not (_close(o2[:, 0].reshape(T, Hq), c["out_expected"]) and _close(l2.reshape(T, Hq), c["lse_expected"])):
                return False
        rng = np.random.default_rng(7)
        for window, sinks in ((0, False), (3, True), (1, False), (6, True)):
            lengths, T = [5, 0, 9, 4], 21
            Hq, Hkv, D = 6, 2, 4
            q = rng.standard_normal((T, Hq, D))
            k = rng.standard_normal((T, Hkv, D))
            v = rng.standard_normal((T, Hkv, D))
            cu = np.concatenate([[0], np.cumsum(lengths)])
            s = rng.standard_normal(Hq) if sinks else None
            o0, l0 = mod.varlen_attn_ref(q, k, v, cu, window, 0.45, s, block=4)
            o1, l1 = oracle.mask.varlen_attn_bruteforce(q, k, v, cu, window, 0.45, s)
            if not (_close(o0, o1) and _close(l0, l1)):
                return False
            tok = np.arange(T).repeat(Hq)
            hd = np.tile(np.arange(Hq), T)
            o2, l2 = mod.varlen_attn_ref_rows(q, k, v, cu, window, 0.45, s, tok, hd)
            if not (_close(o2.reshape(T, Hq, D), o1) and _close(l2.reshape(T, Hq), l1)):
                return False
        # torch SDPA on one causal document
        L = 11
        q = rng.standard_normal((L, 4, 8))
        k = rng.standard_normal((L, 2, 8))
        v = rng.standard_normal((L, 2, 8))
        o, _ = mod.varlen_attn_ref(q, k, v, [0, L], 0, 0.3)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q).permute(1, 0, 2), torch.from_numpy(np.repeat(k, 2, 1)).permute(1, 0, 2),
            torch.from_numpy(np.repeat(v, 2, 1)).permute(1, 0, 2), is_causal=True, scale=0.3)
        return _close(o, ref.permute(1, 0, 2).numpy())
    except Exception:
        return False  # a crash is a caught mistake too


def sparse_pins_hold(mod) -> bool:
    try:
        for c in load("sparse_hand_cases.json"):
            args = [np.array(c[n], dtype=np.float64) for n in ("q", "latent", "k_pe")]
            o, l = mod.sparse_mla_ref(*args, np.array(c["indices"]), np.array(c["doc_ids"]), c["scale"])
            if not (_close(o, c["out_expected"]) and _close(l, c["lse_expected"])):
                return False
        rng = np.random.default_rng(3)
        lengths = [6, 9]
        T, H, dl, dr = 15, 2, 5, 3
        q = rng.standard_normal((T, H, dl + dr))
        lat = rng.standard_normal((T, dl))
        kpe = rng.standard_normal((T, dr))
        ids = np.repeat([0, 1], lengths)
        idx = np.full((T, 12), -1)
        s0 = 0
        for L in lengths:
            for p in range(L):
                idx[s0 + p, :p + 1] = rng.permutation(np.arange(s0, s0 + p + 1))
            s0 += L
        o, l = mod.sparse_mla_ref(q, lat, kpe, idx, ids, 0.6)
        kk = np.concatenate([lat, kpe], 1)[:, None]
        vv = np.concatenate([lat, np.zeros_like(kpe)], 1)[:, None]
        od, ld = oracle.dense.varlen_attn_ref(q, kk, vv, [0, 6, 15], 0, 0.6)
        if not (_close(o, od[..., :dl]) and _close(l, ld)):
            return False
        o2, l2 = mod.sparse_mla_ref_rows(q, lat, kpe, idx, ids, 0.6, np.arange(T))
        return _close(o2, o) and _close(l2, l)
    except Exception:
        return False


def value_pins_hold(mod) -> bool:
    """Scalar-loop and identity-weight pins of the value up-projection, plus its composition."""
    try:
        rng = np.random.default_rng(31)
        T, H, dl, dv = 3, 3, 5, 4
        o = rng.standard_normal((T, H, dl))
        w = rng.standard_normal((H, dv, dl))
        got = mod.mla_value_proj_ref(o, w)
        want = np.zeros((T, H, dv))
        for t in range(T):
            for h in range(H):
                for v in range(dv):
                    want[t, h, v] = sum(w[h, v, d] * o[t, h, d] for d in range(dl))
        if not _close(got, want):
            return False
        eye = np.zeros((H, dv, dl))
        eye[:, :, :dv] = np.eye(dv)
        if not _close(mod.mla_value_proj_ref(o, eye), o[..., :dv], 0.0):
            return False
        lengths = [4, 3]
        q = rng.standard_normal((7, H, dl + 2))
        lat = rng.standard_normal((7, dl))
        kpe = rng.standard_normal((7, 2))
        ids = np.repeat([0, 1], lengths)
        idx = np.array([[0, -1, -1, -1], [0, 1, -1, -1], [0, 1, 2, -1], [0, 1, 2, 3],
                        [4, -1, -1, -1], [4, 5, -1, -1], [4, 5, 6, -1]])
        ov, lv = mod.sparse_mla_value_ref(q, lat, kpe, idx, ids, w, 0.5)
        oo, ll = oracle.sparse.sparse_mla_ref(q, lat, kpe, idx, ids, 0.5)
        return _close(ov, np.einsum("hvd,thd->thv", w, oo)) and _close(lv, ll)
    except Exception:
        return False


DENSE_MUTANTS = [
    ("window off by one", "ok &= (i - j) < window", "ok &= (i - j) <= window"),
    ("window off by one (rows)", "lo = s if window == 0 else max(s, i - window + 1)",
     "lo = s if window == 0 else max(s, i - window)"),
    ("strictly causal", "ok = (j >= s) & (j <= i)", "ok = (j >= s) & (j < i)"),
    # the block path guards the document start twice (key range and mask): remove both
    ("document boundary leak", ("lo = s if window == 0 else max(s, i0 - window + 1)", "ok = (j >= s) & (j <= i)"),
     ("lo = 0 if window == 0 else max(0, i0 - window + 1)", "ok = (j <= i)")),
    ("rows: document boundary leak", "lo = s if window == 0 else max(s, i - window + 1)",
     "lo = 0 if window == 0 else max(0, i - window + 1)"),
    ("GQA modulo map", "return h // (Hq // Hkv)", "return h % Hkv"),
    ("sink dropped from normaliser", "Z = Z + np.exp(sk[h] - m)", "Z = Z"),
    ("sink scaled", "Z = Z + np.exp(sk[h] - m)", "Z = Z + np.exp(scale * sk[h] - m)"),
    # (leaving the sink out of the row max is an exact rewrite, not a mistake: not listed)
    ("sink carries a value", "out[i0:i1, h, :] = (E @ v[lo:hi, g, :]) / Z[:, None]",
     "out[i0:i1, h, :] = (E @ v[lo:hi, g, :] + (0 if sk is None else np.exp(sk[h] - m))[..., None]) / Z[:, None]"),
    ("lse without max", "lse[i0:i1, h] = m + np.log(Z)", "lse[i0:i1, h] = np.log(Z)"),
    ("missing scale", "S = scale * (q[i0:i1, h, :] @ k[lo:hi, g, :].T)", "S = (q[i0:i1, h, :] @ k[lo:hi, g, :].T)"),
    ("value operand swapped", "(E @ v[lo:hi, g, :]) / Z[:, None]", "(E @ k[lo:hi, g, :]) / Z[:, None]"),
    ("unnormalised", "(E @ v[lo:hi, g, :]) / Z[:, None]", "(E @ v[lo:hi, g, :])"),
    ("rows: wrong kv head", "g = kv_head_of(h, Hq, Hkv)\n        kk", "g = h % Hkv\n        kk"),
    ("rows: sink dropped", "Z += np.exp(float(sinks[h]) - m)", "Z += 0.0"),
]

SPARSE_MUTANTS = [
    ("strictly causal slots", "ok = (idx >= 0) & (idx < T) & (idx <= t)", "ok = (idx >= 0) & (idx < T) & (idx < t)"),
    ("no document check", "ok &= np.asarray(doc_ids)[safe] == doc_ids[t]", "ok &= True"),
    ("rotary part dropped", "S = scale * (qt[:, :d_l] @ lat.T + qt[:, d_l:] @ rope.T)", "S = scale * (qt[:, :d_l] @ lat.T)"),
    ("rotary part on wrong coords", "qt[:, d_l:] @ rope.T", "qt[:, :rope.shape[1]] @ rope.T"),
    ("missing scale", "S = scale * (qt[:, :d_l] @ lat.T + qt[:, d_l:] @ rope.T)", "S = (qt[:, :d_l] @ lat.T + qt[:, d_l:] @ rope.T)"),
    ("empty row lse zero", "return np.zeros((H, d_l)), np.full(H, -np.inf)", "return np.zeros((H, d_l)), np.zeros(H)"),
    ("value rows reversed", "return (E @ lat) / Z[:, None]", "return (E @ lat[::-1]) / Z[:, None]"),
    ("duplicates collapsed", "sel = np.asarray(indices[t], dtype=np.int64)[ok]",
     "sel = np.unique(np.asarray(indices[t], dtype=np.int64)[ok])"),
]


VALUE_MUTANTS = [
    ("wrong head's weight", "out[:, h, :] = o[:, h, :] @ w[h].T", "out[:, h, :] = o[:, h, :] @ w[(h + 1) % H].T"),
    ("latent coordinates reversed", "out[:, h, :] = o[:, h, :] @ w[h].T", "out[:, h, :] = o[:, h, ::-1] @ w[h].T"),
    ("projection skipped", "return mla_value_proj_ref(o, value_weight), lse",
     "return o[..., :np.asarray(value_weight).shape[1]], lse"),
]


def test_unmutated_oracle_passes_the_battery():
    assert dense_pins_hold(oracle.dense)
    assert sparse_pins_hold(oracle.sparse)
    assert value_pins_hold(oracle.sparse)


@pytest.mark.parametrize("name,old,new", VALUE_MUTANTS, ids=[m[0] for m in VALUE_MUTANTS])
def test_value_mutant_is_caught(name, old, new):
    assert not value_pins_hold(mutated(oracle.sparse, old, new)), f"pins missed mutant: {name}"


@pytest.mark.parametrize("name,old,new", DENSE_MUTANTS, ids=[m[0] for m in DENSE_MUTANTS])
def test_dense_mutant_is_caught(name, old, new):
    assert not dense_pins_hold(mutated(oracle.dense, old, new)), f"pins missed mutant: {name}"


@pytest.mark.parametrize("name,old,new", SPARSE_MUTANTS, ids=[m[0] for m in SPARSE_MUTANTS])
def test_sparse_mutant_is_caught(name, old, new):
    assert not sparse_pins_hold(mutated(oracle.sparse, old, new)), f"pins missed mutant: {name}"
