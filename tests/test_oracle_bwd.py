"""Pins of the fp64 backward oracle (oracle.dense_bwd), none of which retypes its formulas.

* central finite differences of the forward oracle, element by element, on tiny
  packed problems (documents, padding, window, sinks, GQA);
* torch fp64 autograd through a plainly masked softmax with the sink as an
  extra logit column (a library routine doing the differentiation);
* closed forms for one-token documents;
* invariants: key-shift invariance of dq without sinks, the column sum rule of
  dv, GQA = summed gradients of repeated-KV MHA, window >= document length;
* planted mistakes in copies of the oracle, each caught by the pins.
"""
import numpy as np
import pytest
import torch

import oracle.dense_bwd
from oracle import varlen_attn_bwd_ref, varlen_attn_ref
from tests.test_oracle_mutants import mutated


def problem(seed, T=9, cu=(0, 3, 8), Hq=4, Hkv=2, D=3, sinks=True):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, Hq, D))
    k = rng.standard_normal((T, Hkv, D))
    v = rng.standard_normal((T, Hkv, D))
    do = rng.standard_normal((T, Hq, D))
    s = rng.standard_normal(Hq) if sinks else None
    return q, k, v, do, np.array(cu), s


def loss(q, k, v, do, cu, window, scale, s):
    out, _ = varlen_attn_ref(q, k, v, cu, window, scale, s)
    return float((out * do).sum())


def finite_difference_grads(q, k, v, do, cu, window, scale, s, eps=1e-6):
    grads = []
    for name in ("q", "k", "v", "s"):
        x = {"q": q, "k": k, "v": v, "s": s}[name]
        if x is None:
            grads.append(None)
            continue
        g = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            args = {"q": q, "k": k, "v": v, "s": s}
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args[name] = xp
            lp = loss(args["q"], args["k"], args["v"], do, cu, window, scale, args["s"])
            args[name] = xm
            lm = loss(args["q"], args["k"], args["v"], do, cu, window, scale, args["s"])
            g[idx] = (lp - lm) / (2 * eps)
        grads.append(g)
    return grads


def fd_pin_holds(bwd, seed, window, sinks, Hq=4, Hkv=2, tol=1e-7) -> bool:
    q, k, v, do, cu, s = problem(seed, Hq=Hq, Hkv=Hkv, sinks=sinks)
    dq, dk, dv, ds, _ = bwd(q, k, v, do, cu, window, 0.7, s)
    fq, fk, fv, fs = finite_difference_grads(q, k, v, do, cu, window, 0.7, s)
    ok = np.abs(dq - fq).max() <= tol and np.abs(dk - fk).max() <= tol and np.abs(dv - fv).max() <= tol
    if sinks:
        ok = ok and ds is not None and np.abs(ds - fs).max() <= tol
    return bool(ok)


@pytest.mark.parametrize("window,sinks", [(0, False), (0, True), (2, True), (1, False)])
def test_finite_differences_of_the_forward(window, sinks):
    assert fd_pin_holds(varlen_attn_bwd_ref, seed=window + 10 * sinks, window=window, sinks=sinks)


def test_finite_differences_mha_and_single_kv_head():
    assert fd_pin_holds(varlen_attn_bwd_ref, seed=3, window=0, sinks=True, Hq=2, Hkv=2)
    assert fd_pin_holds(varlen_attn_bwd_ref, seed=4, window=3, sinks=False, Hq=3, Hkv=1)


def torch_grads(q, k, v, do, cu, window, scale, s):
    """Autograd through a plainly masked softmax over the full T x T matrix (fp64, CPU)."""
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    doc = np.full(T, -1)
    for d in range(len(cu) - 1):
        doc[cu[d]:cu[d + 1]] = d
    i, j = np.arange(T)[:, None], np.arange(T)[None, :]
    allowed = (doc[:, None] == doc[None, :]) & (doc[:, None] >= 0) & (j <= i)
    if window:
        allowed &= (i - j) < window
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    ts = None if s is None else torch.tensor(s, dtype=torch.float64, requires_grad=True)
    mask = torch.tensor(allowed)
    outs = []
    for h in range(Hq):
        logits = scale * tq[:, h, :] @ tk[:, h // G, :].T
        logits = logits.masked_fill(~mask, float("-inf"))
        if ts is not None:
            logits = torch.cat([logits, ts[h].expand(T, 1)], dim=1)
        rows = mask.any(dim=1) if ts is None else torch.ones(T, dtype=torch.bool)
        p = torch.softmax(logits.masked_fill(~rows[:, None], 0.0), dim=1)[:, :T]
        p = p * rows[:, None] * torch.tensor(doc >= 0)[:, None]
        outs.append(p @ tv[:, h // G, :])
    out = torch.stack(outs, dim=1)
    (out * torch.tensor(do)).sum().backward()
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy(), None if ts is None else ts.grad.numpy()


@pytest.mark.parametrize("window,sinks", [(0, False), (5, True), (1, True)])
def test_torch_autograd_fp64(window, sinks):
    lengths = [7, 1, 20, 9]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    q, k, v, do, _, s = problem(20 + window, T=40, cu=cu, Hq=4, Hkv=2, D=8, sinks=sinks)
    dq, dk, dv, ds, _ = varlen_attn_bwd_ref(q, k, v, do, cu, window, 0.35, s)
    tq, tk, tv, ts = torch_grads(q, k, v, do, cu, window, 0.35, s)
    np.testing.assert_allclose(dq, tq, atol=1e-12)
    np.testing.assert_allclose(dk, tk, atol=1e-12)
    np.testing.assert_allclose(dv, tv, atol=1e-12)
    if sinks:
        np.testing.assert_allclose(ds, ts, atol=1e-12)


def test_one_token_documents_closed_forms():
    T, Hq, Hkv, D = 5, 4, 2, 3
    q, k, v, do, _, s = problem(30, T=T, cu=(0, 5), Hq=Hq, Hkv=Hkv, D=D, sinks=True)
    cu = np.arange(T + 1)
    # no sink: the softmax over one key is 1, so no gradient reaches q or k and dv = summed dout
    dq, dk, dv, ds, delta = varlen_attn_bwd_ref(q, k, v, do, cu, 0, 0.9, None)
    assert np.all(dq == 0) and np.all(dk == 0) and ds is None
    np.testing.assert_allclose(dv, do.reshape(T, Hkv, 2, D).sum(axis=2), atol=1e-15)
    # with a sink: p = sigmoid(score - sink), out = p v
    dq, dk, dv, ds, delta = varlen_attn_bwd_ref(q, k, v, do, cu, 0, 0.9, s)
    for t in range(T):
        for h in range(Hq):
            g = h // 2
            p = 1.0 / (1.0 + np.exp(-(0.9 * q[t, h] @ k[t, g] - s[h])))
            dpv = do[t, h] @ v[t, g]
            np.testing.assert_allclose(delta[t, h], p * dpv, atol=1e-14)
            np.testing.assert_allclose(dq[t, h], 0.9 * p * (1 - p) * dpv * k[t, g], atol=1e-14)
    ref_ds = [-sum((1 - 1 / (1 + np.exp(-(0.9 * q[t, h] @ k[t, h // 2] - s[h])))) * delta[t, h] for t in range(T))
              for h in range(Hq)]
    np.testing.assert_allclose(ds, ref_ds, atol=1e-14)


def test_key_shift_invariance_and_dv_column_sum():
    lengths = [12, 30]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    q, k, v, do, _, s = problem(40, T=42, cu=cu, Hq=4, Hkv=2, D=6, sinks=False)
    dq, dk, dv, _, _ = varlen_attn_bwd_ref(q, k, v, do, cu, 0, 0.5, None)
    c = np.random.default_rng(1).standard_normal(6)
    dq2, _, dv2, _, _ = varlen_attn_bwd_ref(q, k + c, v, do, cu, 0, 0.5, None)
    np.testing.assert_allclose(dq2, dq, atol=1e-12)
    np.testing.assert_allclose(dv2, dv, atol=1e-12)
    # every row's probabilities sum to 1 - p_sink: summed over keys, dv collects summed dout
    for d in range(2):
        sl = slice(cu[d], cu[d + 1])
        np.testing.assert_allclose(dv[sl].sum(axis=0), do[sl].reshape(-1, 2, 2, 6).sum(axis=(0, 2)), atol=1e-12)


def test_gqa_equals_summed_repeated_kv_mha():
    lengths = [10, 14]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    q, k, v, do, _, s = problem(50, T=24, cu=cu, Hq=6, Hkv=2, D=4, sinks=True)
    dq, dk, dv, ds, _ = varlen_attn_bwd_ref(q, k, v, do, cu, 4, 0.6, s)
    kr, vr = np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1)
    mq, mk, mv, ms, _ = varlen_attn_bwd_ref(q, kr, vr, do, cu, 4, 0.6, s)
    np.testing.assert_allclose(dq, mq, atol=1e-12)
    np.testing.assert_allclose(ds, ms, atol=1e-12)
    np.testing.assert_allclose(dk, mk.reshape(24, 2, 3, 4).sum(axis=2), atol=1e-12)
    np.testing.assert_allclose(dv, mv.reshape(24, 2, 3, 4).sum(axis=2), atol=1e-12)


def test_window_at_least_document_length_equals_causal_and_padding_is_inert():
    q, k, v, do, cu, s = problem(60, T=12, cu=(0, 5, 9), sinks=True)
    a = varlen_attn_bwd_ref(q, k, v, do, cu, 0, 0.8, s)
    b = varlen_attn_bwd_ref(q, k, v, do, cu, 5, 0.8, s)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
    dq, dk, dv, _, delta = a
    assert np.all(dq[9:] == 0) and np.all(dk[9:] == 0) and np.all(dv[9:] == 0) and np.all(delta[9:] == 0)


def test_query_blocking_does_not_change_the_result():
    lengths = [300, 45]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    q, k, v, do, _, s = problem(70, T=345, cu=cu, Hq=2, Hkv=1, D=4, sinks=True)
    a = varlen_attn_bwd_ref(q, k, v, do, cu, 70, 0.4, s, block=256)
    b = varlen_attn_bwd_ref(q, k, v, do, cu, 70, 0.4, s, block=17)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, atol=1e-12)


# ---------------------------------------------------------------- planted mistakes
BWD_MUTANTS = {
    "delta dropped": ("dS = P * (dP - dl[:, None])", "dS = P * dP"),
    "dk without scale": ("dk[lo:hi, g, :] += scale * (dS.T @", "dk[lo:hi, g, :] += (dS.T @"),
    "dsink sign": ("dsink[h] -= ", "dsink[h] += "),
    "dv from dS": ("dv[lo:hi, g, :] += P.T @ do", "dv[lo:hi, g, :] += dS.T @ do"),
    "interleaved head map": ("g = kv_head_of(h, Hq, Hkv)", "g = h % Hkv"),
    "dq through v": ("dq[i0:i1, h, :] = scale * (dS @ k[lo:hi, g, :])", "dq[i0:i1, h, :] = scale * (dS @ v[lo:hi, g, :])"),
    "dk overwritten across heads": ("dk[lo:hi, g, :] += ", "dk[lo:hi, g, :] = "),
    "delta unnormalised": ("dl = (P * dP).sum(axis=1)", "dl = (E * dP).sum(axis=1)"),
    "sink probability unnormalised": ("np.exp(sk[h] - m) / Z * dl", "np.exp(sk[h] - m) * dl"),
}


def bwd_pins_hold(mod) -> bool:
    try:
        return (fd_pin_holds(mod.varlen_attn_bwd_ref, seed=1, window=0, sinks=True)
                and fd_pin_holds(mod.varlen_attn_bwd_ref, seed=2, window=2, sinks=True))
    except Exception:
        return False


def test_pins_hold_for_the_oracle_itself():
    assert bwd_pins_hold(oracle.dense_bwd)


@pytest.mark.parametrize("name", sorted(BWD_MUTANTS))
def test_pins_catch_planted_mistake(name):
    old, new = BWD_MUTANTS[name]
    assert not bwd_pins_hold(mutated(oracle.dense_bwd, old, new)), name
