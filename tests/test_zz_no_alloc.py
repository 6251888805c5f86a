"""varlen_attn_bwd_noalloc (through the C ABI) against varlen_attn_bwd on the same inputs.

The no-allocation entry point runs the same kernels with its per-row workspace in the
library's device array instead of a caller buffer, so its gradients must equal those of
varlen_attn_bwd bit for bit: on two calls in a row, the second with a smaller input (the
array keeps the first call's contents), and with and without sinks.  A call beyond the
array's limit is refused before anything is enqueued.
"""
import ctypes
import math

import numpy as np
import pytest
import torch

from sliding_window_gqa_varlen_amd import binding, workloads as W
from sliding_window_gqa_varlen_amd.binding import describe
from tests.gpu_util import dev

pytestmark = pytest.mark.gpu


def case(lengths, T, Hq, Hkv, D, window, sinks, seed):
    w = W.DenseWorkload("noalloc", "bf16", T=T, Hq=Hq, Hkv=Hkv, D=D, window=window, scale=1.0 / math.sqrt(D),
                        seed=seed, doc_lengths=tuple(lengths), sinks=sinks)
    inp = W.make_dense(w)
    t = {n: dev(inp[n], torch.bfloat16) for n in ("q", "k", "v")}
    t["cu"] = torch.from_numpy(inp["cu_seqlens"]).cuda()
    t["sinks"] = None if inp["sinks"] is None else torch.from_numpy(np.asarray(inp["sinks"], np.float32)).cuda()
    t["dout"] = dev(W.make_dout(seed, inp["q"].shape), torch.bfloat16)
    t["out"], t["lse"] = binding.varlen_attn_fwd(t["q"], t["k"], t["v"], t["cu"], inp["n_docs"], window, w.scale,
                                                 t["sinks"])
    return w, inp, t


def run_both(w, inp, t):
    ref = binding.varlen_attn_bwd(t["q"], t["k"], t["v"], t["out"], t["dout"], t["lse"], t["cu"], inp["n_docs"],
                                  w.window, w.scale, t["sinks"])
    dq, dk, dv = torch.full_like(t["q"], 7.0), torch.full_like(t["k"], 7.0), torch.full_like(t["v"], 7.0)
    dsinks = None if t["sinks"] is None else torch.full((w.Hq,), 7.0, device="cuda", dtype=torch.float32)
    got = binding.varlen_attn_bwd_noalloc(t["q"], t["k"], t["v"], t["out"], t["dout"], t["lse"], t["cu"],
                                          inp["n_docs"], w.window, w.scale, t["sinks"], dq=dq, dk=dk, dv=dv,
                                          dsinks=dsinks)
    torch.cuda.synchronize()
    return ref, got


def assert_bitwise(ref, got):
    for name, a, b in zip(("dq", "dk", "dv", "dsinks"), ref, got):
        if a is None:
            assert b is None
            continue
        x, y = a.float().cpu().numpy(), b.float().cpu().numpy()
        assert np.all(np.isfinite(y)), name
        np.testing.assert_array_equal(x, y, err_msg=name)


def test_two_calls_in_a_row_second_smaller(gpu):
    first = case([300, 7, 129, 64, 1], T=520, Hq=16, Hkv=2, D=128, window=90, sinks=True, seed=41)
    assert_bitwise(*run_both(*first))
    second = case([40, 33, 90], T=170, Hq=4, Hkv=1, D=64, window=0, sinks=False, seed=42)
    assert_bitwise(*run_both(*second))
    third = case([17, 50], T=80, Hq=8, Hkv=4, D=128, window=0, sinks=True, seed=43)
    assert_bitwise(*run_both(*third))


def test_full_size_window128_workload(gpu):
    """The 65536-token, 64-head window-128 backward with sinks: T * Hq = 2^22, the array's limit."""
    w = W.WORKLOADS[3]
    inp = W.make_dense(w)
    t = {n: dev(inp[n], torch.bfloat16) for n in ("q", "k", "v")}
    t["cu"] = torch.from_numpy(inp["cu_seqlens"]).cuda()
    t["sinks"] = torch.from_numpy(np.asarray(inp["sinks"], np.float32)).cuda()
    t["dout"] = dev(W.make_dout(w.seed, inp["q"].shape), torch.bfloat16)
    t["out"], t["lse"] = binding.varlen_attn_fwd(t["q"], t["k"], t["v"], t["cu"], inp["n_docs"], w.window, w.scale,
                                                 t["sinks"])
    assert w.T * w.Hq == 1 << 22
    assert_bitwise(*run_both(w, inp, t))


def test_beyond_the_limit_is_refused_before_any_launch(gpu):
    lib = binding.load_library()
    T, Hq = (1 << 22) + 16, 1
    q = torch.empty(16, 1, 64, dtype=torch.bfloat16, device="cuda")
    d = describe(q)
    d.shape[0] = T  # only the descriptor is oversized; the call must refuse it on the host
    st = lib.varlen_attn_bwd_noalloc(ctypes.byref(d), ctypes.byref(d), ctypes.byref(d), ctypes.byref(d),
                                     ctypes.byref(d), None, None, 0, 0, 0.125, None, ctypes.byref(d),
                                     ctypes.byref(d), ctypes.byref(d), None, None)
    assert st == -5
    assert b"4,194,304" in lib.swa_last_error()
    assert T * Hq > 1 << 22
