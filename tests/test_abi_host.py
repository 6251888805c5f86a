"""The C ABI on the host: the library loads, exports what include/*.h declare,
and rejects every malformed call before touching the GPU (no compute call here)."""
import ctypes
import glob
import math
import os
import re
import subprocess

import pytest
import torch

from sliding_window_gqa_varlen_amd import binding
from sliding_window_gqa_varlen_amd.binding import SwaError, describe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))

SWA_OK, SWA_ERR_NULL, SWA_ERR_DTYPE, SWA_ERR_SHAPE, SWA_ERR_ARG, SWA_ERR_UNSUPPORTED, SWA_ERR_LAYOUT = \
    0, -1, -2, -3, -4, -5, -6


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M))
    return sorted(names)


def test_header_declares_the_expected_entry_points():
    assert declared_functions() == sorted(binding.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", binding.library_path()], capture_output=True, text=True)
    exported = {line.split()[-1] for line in out.stdout.splitlines() if " T " in line}
    for name in declared_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_version_and_error_strings(lib):
    assert lib.swa_abi_version() == 1
    for code in (0, -1, -2, -3, -4, -5, -6, -7, 12345):
        assert len(lib.swa_strerror(code)) > 0
    assert lib.swa_strerror(0) == b"success"


# ---------------------------------------------------------------- dense argument checks
def dense_args(T=16, Hq=4, Hkv=2, D=64, dtype=torch.bfloat16):
    q = torch.zeros(T, Hq, D, dtype=dtype)
    k = torch.zeros(T, Hkv, D, dtype=dtype)
    v = torch.zeros(T, Hkv, D, dtype=dtype)
    out = torch.zeros(T, Hq, D, dtype=dtype)
    cu = torch.tensor([0, T], dtype=torch.int32)
    return dict(q=q, k=k, v=v, out=out, cu=cu)


def call_dense(lib, a, n_docs=1, window=0, scale=0.125, sinks=None, lse=None, descs=None, cu="default"):
    d = descs or {n: describe(a[n]) for n in ("q", "k", "v", "out")}
    ref = lambda x: None if x is None else ctypes.byref(x)  # noqa: E731
    cu_ptr = ctypes.c_void_p(a["cu"].data_ptr()) if cu == "default" else cu
    return lib.varlen_attn_fwd(ref(d["q"]), ref(d["k"]), ref(d["v"]), cu_ptr, n_docs, window, scale,
                               sinks, ref(d["out"]), lse, None)


def test_dense_rejects_null_descriptors(lib):
    a = dense_args()
    for name in ("q", "k", "v", "out"):
        d = {n: describe(a[n]) for n in ("q", "k", "v", "out")}
        d[name] = None
        assert call_dense(lib, a, descs=d) == SWA_ERR_NULL
        assert name in lib.swa_last_error().decode()


def test_dense_rejects_null_cu_seqlens_with_documents(lib):
    assert call_dense(lib, dense_args(), cu=None) == SWA_ERR_NULL


def test_dense_rejects_bad_ranks_shapes_and_dtypes(lib):
    a = dense_args()
    d = {n: describe(a[n]) for n in ("q", "k", "v", "out")}
    d["q"].ndim = 2
    assert call_dense(lib, a, descs=d) == SWA_ERR_SHAPE
    b = dense_args()
    b["k"] = torch.zeros(15, 2, 64, dtype=torch.bfloat16)
    assert call_dense(lib, b) == SWA_ERR_SHAPE
    b = dense_args(Hq=3, Hkv=2)
    assert call_dense(lib, b) == SWA_ERR_SHAPE
    assert "multiple" in lib.swa_last_error().decode()
    b = dense_args()
    b["out"] = torch.zeros(16, 4, 64, dtype=torch.float32)
    assert call_dense(lib, b) == SWA_ERR_DTYPE
    b = dense_args(dtype=torch.int32)
    assert call_dense(lib, b) == SWA_ERR_DTYPE
    b = dense_args()
    b["v"] = torch.zeros(16, 2, 128, dtype=torch.bfloat16)
    assert call_dense(lib, b) == SWA_ERR_SHAPE


@pytest.mark.parametrize("D,dtype", [(32, torch.bfloat16), (96, torch.bfloat16), (512, torch.bfloat16),
                                     (256, torch.float32)])
def test_dense_rejects_unsupported_head_dim(lib, D, dtype):
    """head_dim 64 and 128 for both dtypes, 256 for bf16 only."""
    assert call_dense(lib, dense_args(D=D, dtype=dtype)) == SWA_ERR_UNSUPPORTED


@pytest.mark.parametrize("kw,code", [
    (dict(window=-1), SWA_ERR_ARG), (dict(n_docs=-1), SWA_ERR_ARG), (dict(scale=0.0), SWA_ERR_ARG),
    (dict(scale=-0.5), SWA_ERR_ARG), (dict(scale=math.nan), SWA_ERR_ARG), (dict(scale=math.inf), SWA_ERR_ARG)])
def test_dense_rejects_bad_scalars(lib, kw, code):
    assert call_dense(lib, dense_args(), **kw) == code


def test_dense_rejects_misaligned_or_strided_layouts(lib):
    a = dense_args()
    base = torch.zeros(16 * 4 * 64 + 1, dtype=torch.bfloat16)
    a["q"] = base[1:].view(16, 4, 64)  # 2-byte offset: not 16-byte aligned
    assert call_dense(lib, a) == SWA_ERR_LAYOUT
    a = dense_args()
    a["k"] = torch.zeros(16, 2, 128, dtype=torch.bfloat16)[:, :, ::2]  # innermost stride 2
    assert call_dense(lib, a) == SWA_ERR_LAYOUT
    a = dense_args()
    a["v"] = torch.zeros(16, 2, 68, dtype=torch.bfloat16)[:, :, :64]  # row stride 136 bytes
    assert call_dense(lib, a) == SWA_ERR_LAYOUT


@pytest.mark.parametrize("dim", [0, 1])
def test_dense_rejects_out_strides_beyond_32_bit_store_offsets(lib, dim):
    """The bf16 output tile leaves by buffer stores whose offsets from the wave's first row are
    32-bit: token and head strides of out must stay below 2^24 elements (refused before any
    launch; only the descriptor's stride is changed, no memory is touched)."""
    a = dense_args()
    d = {n: describe(a[n]) for n in ("q", "k", "v", "out")}
    d["out"].stride[dim] = 1 << 24
    assert call_dense(lib, a, descs=d) == SWA_ERR_UNSUPPORTED
    assert "out" in lib.swa_last_error().decode()


def test_dense_rejects_output_aliasing_an_input(lib):
    a = dense_args(Hq=2, Hkv=2)
    a["out"] = a["q"]
    assert call_dense(lib, a) == SWA_ERR_ARG


def test_dense_empty_problem_is_a_no_op(lib):
    a = dense_args(T=0)
    assert call_dense(lib, a, n_docs=0) == SWA_OK


def test_library_detail_reaches_swa_last_error(lib):
    a = dense_args()
    assert call_dense(lib, a, window=-3) == SWA_ERR_ARG
    assert b"window" in lib.swa_last_error()


def test_binding_refuses_host_tensors_before_any_call():
    """A host tensor would give the kernel a host address: the binding refuses it."""
    a = dense_args()
    with pytest.raises(ValueError, match="GPU"):
        binding.varlen_attn_fwd(a["q"], a["k"], a["v"], a["cu"], window=0, stream=0)
    b = bwd_args()
    with pytest.raises(ValueError, match="GPU"):
        binding.varlen_attn_bwd(b["q"], b["k"], b["v"], b["out"], b["dout"], torch.zeros(16, 4), b["cu"], stream=0)
    s = sparse_args()
    with pytest.raises(ValueError, match="GPU"):
        binding.sparse_mla_fwd(s["q"], s["latent"], s["k_pe"], s["idx"], s["ids"], stream=0)
    v = vproj_args()
    with pytest.raises(ValueError, match="GPU"):
        binding.mla_value_proj(v["o"], v["w"], stream=0)
    with pytest.raises(ValueError, match="GPU"):
        binding.peak_copy(torch.zeros(16), torch.zeros(16), stream=0)


class _FakeGpu(torch.Tensor):
    """A host tensor that reports a GPU device, to drive the binding's size and layout checks
    on a host without a GPU (they run before the library is called, so nothing reads it)."""

    @staticmethod
    def __new__(cls, t, device="cuda:0"):
        r = torch.Tensor._make_subclass(cls, t)
        r._fake_device = torch.device(device)
        return r

    @property
    def device(self):
        return self._fake_device


def test_binding_size_and_layout_checks():
    g = _FakeGpu
    a = dense_args(T=16, Hq=4)
    q, k, v, out = g(a["q"]), g(a["k"]), g(a["v"]), g(a["out"])
    lse = g(torch.zeros(16, 4))
    with pytest.raises(ValueError, match="cu_seqlens must hold at least 3"):
        binding.varlen_attn_fwd(q, k, v, g(torch.tensor([0, 16], dtype=torch.int32)), n_docs=2, out=out, lse=lse,
                                stream=0)
    with pytest.raises(ValueError, match="cu_seqlens must be contiguous"):
        binding.varlen_attn_fwd(q, k, v, g(torch.zeros(8, dtype=torch.int32)[::2]), n_docs=2, out=out, lse=lse,
                                stream=0)
    with pytest.raises(ValueError, match=r"sinks must have shape \(4,\)"):
        binding.varlen_attn_fwd(q, k, v, g(a["cu"]), n_docs=1, sinks=g(torch.zeros(3)), out=out, lse=lse, stream=0)
    with pytest.raises(ValueError, match="cu_seqlens is required"):
        binding.varlen_attn_fwd(q, k, v, None, n_docs=1, out=out, lse=lse, stream=0)
    with pytest.raises(ValueError, match="is on cuda:1"):
        binding.varlen_attn_fwd(q, g(a["k"], "cuda:1"), v, g(a["cu"]), n_docs=1, out=out, lse=lse, stream=0)
    with pytest.raises(ValueError, match=r"lse must have shape \(16, 4\)"):
        binding.varlen_attn_fwd(q, k, v, g(a["cu"]), n_docs=1, out=out, lse=g(torch.zeros(16, 3)), stream=0)
    b = {n: g(x) for n, x in bwd_args().items() if x is not None}
    with pytest.raises(ValueError, match=r"dsinks must"):
        binding.varlen_attn_bwd(b["q"], b["k"], b["v"], b["out"], b["dout"], g(torch.zeros(16, 4)), b["cu"], n_docs=1,
                                sinks=g(torch.zeros(4)), dq=b["dq"], dk=b["dk"], dv=b["dv"], dsinks=g(torch.zeros(3)),
                                delta=g(torch.zeros(16, 4)), stream=0)
    sp = sparse_args(T=8)
    with pytest.raises(ValueError, match=r"doc_ids must have shape \(8,\)"):
        binding.sparse_mla_fwd(g(sp["q"]), g(sp["latent"]), g(sp["k_pe"]), g(sp["idx"]),
                               g(torch.zeros(7, dtype=torch.int32)), out=g(sp["out"]), lse=g(torch.zeros(8, 16)),
                               stream=0)


# ---------------------------------------------------------------- sparse argument checks
def sparse_args(T=8, H=16, topk=4):
    return dict(q=torch.zeros(T, H, 576, dtype=torch.bfloat16), latent=torch.zeros(T, 512, dtype=torch.bfloat16),
                k_pe=torch.zeros(T, 64, dtype=torch.bfloat16), idx=torch.zeros(T, topk, dtype=torch.int32),
                ids=torch.zeros(T, dtype=torch.int32), out=torch.zeros(T, H, 512, dtype=torch.bfloat16))


def call_sparse(lib, a, scale=0.05, ids="default"):
    d = {n: describe(a[n]) for n in ("q", "latent", "k_pe", "idx", "out")}
    ids_ptr = ctypes.c_void_p(a["ids"].data_ptr()) if ids == "default" else ids
    return lib.sparse_mla_fwd(ctypes.byref(d["q"]), ctypes.byref(d["latent"]), ctypes.byref(d["k_pe"]),
                              ctypes.byref(d["idx"]), ids_ptr, scale, ctypes.byref(d["out"]), None, None)


def test_sparse_rejects_bad_arguments(lib):
    assert call_sparse(lib, sparse_args(), ids=None) == SWA_ERR_NULL
    a = sparse_args()
    a["idx"] = torch.zeros(8, 4, dtype=torch.float32)
    assert call_sparse(lib, a) == SWA_ERR_DTYPE
    a = sparse_args()
    a["q"] = torch.zeros(8, 16, 512, dtype=torch.bfloat16)
    assert call_sparse(lib, a) == SWA_ERR_SHAPE
    a = sparse_args(H=12)
    assert call_sparse(lib, a) == SWA_ERR_UNSUPPORTED
    a = sparse_args(topk=0)
    assert call_sparse(lib, a) == SWA_ERR_ARG
    assert call_sparse(lib, sparse_args(), scale=-1.0) == SWA_ERR_ARG
    a = sparse_args()
    a["out"] = torch.zeros(8, 16, 512, dtype=torch.float32)
    assert call_sparse(lib, a) == SWA_ERR_DTYPE
    a = sparse_args()
    a["latent"] = torch.zeros(8, 256, dtype=torch.bfloat16)
    assert call_sparse(lib, a) == SWA_ERR_SHAPE


def test_sparse_nope_shapes(lib):
    """Rotary width 0 (q 512 wide, k_pe [T, 0]) is accepted; other rotary widths are not."""
    a = sparse_args(T=0)
    a["q"], a["k_pe"] = torch.zeros(0, 16, 512, dtype=torch.bfloat16), torch.zeros(0, 0, dtype=torch.bfloat16)
    assert call_sparse(lib, a) == SWA_OK
    a = sparse_args()
    a["q"], a["k_pe"] = torch.zeros(8, 16, 544, dtype=torch.bfloat16), torch.zeros(8, 32, dtype=torch.bfloat16)
    assert call_sparse(lib, a) == SWA_ERR_UNSUPPORTED
    a = sparse_args()
    a["k_pe"] = torch.zeros(8, 0, dtype=torch.bfloat16)  # q still 576 wide
    assert call_sparse(lib, a) == SWA_ERR_SHAPE


def test_sparse_empty_problem_is_a_no_op(lib):
    assert call_sparse(lib, sparse_args(T=0)) == SWA_OK


# ---------------------------------------------------------------- value projection argument checks
def vproj_args(T=8, H=4, Dv=128, Dl=512):
    return dict(o=torch.zeros(T, H, Dl, dtype=torch.bfloat16), w=torch.zeros(H, Dv, Dl, dtype=torch.bfloat16),
                out=torch.zeros(T, H, Dv, dtype=torch.bfloat16))


def call_vproj(lib, a, descs=None):
    d = descs or {n: describe(a[n]) for n in ("o", "w", "out")}
    ref = lambda x: None if x is None else ctypes.byref(x)  # noqa: E731
    return lib.mla_value_proj(ref(d["o"]), ref(d["w"]), ref(d["out"]), None)


def test_value_proj_rejects_bad_arguments(lib):
    for name in ("o", "w", "out"):
        a = vproj_args()
        d = {n: describe(a[n]) for n in ("o", "w", "out")}
        d[name] = None
        assert call_vproj(lib, a, descs=d) == SWA_ERR_NULL
    a = vproj_args()
    a["w"] = torch.zeros(4, 128, 512, dtype=torch.float32)
    assert call_vproj(lib, a) == SWA_ERR_DTYPE
    a = vproj_args()
    a["out"] = torch.zeros(8, 4, 128, dtype=torch.float32)
    assert call_vproj(lib, a) == SWA_ERR_DTYPE
    a = vproj_args()
    a["w"] = torch.zeros(5, 128, 512, dtype=torch.bfloat16)
    assert call_vproj(lib, a) == SWA_ERR_SHAPE
    a = vproj_args()
    a["out"] = torch.zeros(8, 4, 64, dtype=torch.bfloat16)
    assert call_vproj(lib, a) == SWA_ERR_SHAPE
    a = vproj_args()
    a["o"] = torch.zeros(8, 2048, dtype=torch.bfloat16)  # rank 2
    assert call_vproj(lib, a) == SWA_ERR_SHAPE
    assert call_vproj(lib, vproj_args(Dl=256)) == SWA_ERR_UNSUPPORTED
    assert call_vproj(lib, vproj_args(Dv=96)) == SWA_ERR_UNSUPPORTED
    a = vproj_args()
    a["o"] = a["o"][:, :, :-8]  # innermost extent 504 is checked before any layout question
    assert call_vproj(lib, a) == SWA_ERR_SHAPE
    a = vproj_args()
    a["o"] = torch.zeros(8, 4, 520, dtype=torch.bfloat16)[:, :, 4:516]  # 8-byte misaligned base
    assert call_vproj(lib, a) == SWA_ERR_LAYOUT
    a = vproj_args()
    a["out"] = torch.zeros(8, 4, 256, dtype=torch.bfloat16)[:, :, ::2]  # innermost stride 2
    assert call_vproj(lib, a) == SWA_ERR_LAYOUT


def test_value_proj_rejects_output_aliasing_an_input(lib):
    a = vproj_args(Dv=128)
    buf = torch.zeros(8, 4, 512, dtype=torch.bfloat16)
    a["o"] = buf
    a["out"] = buf[:, :, :128]
    assert call_vproj(lib, a) == SWA_ERR_ARG


def test_value_proj_empty_problem_is_a_no_op(lib):
    assert call_vproj(lib, vproj_args(T=0)) == SWA_OK
    a = vproj_args(T=0)
    with pytest.raises(ValueError, match="GPU"):  # the binding refuses host tensors even when empty
        binding.mla_value_proj(a["o"], a["w"], stream=0)


# ---------------------------------------------------------------- backward argument checks
def bwd_args(T=16, Hq=4, Hkv=2, D=128, dtype=torch.bfloat16):
    a = {n: torch.zeros(T, Hq, D, dtype=dtype) for n in ("q", "out", "dout", "dq")}
    a.update({n: torch.zeros(T, Hkv, D, dtype=dtype) for n in ("k", "v", "dk", "dv")})
    a.update(lse=torch.zeros(T, Hq), delta=torch.zeros(T, Hq), cu=torch.tensor([0, T], dtype=torch.int32),
             sinks=None, dsinks=None)
    return a


def call_bwd(lib, a, window=0, scale=0.125, lse="default", delta="default", mutate=None):
    d = {n: describe(a[n]) for n in ("q", "k", "v", "out", "dout", "dq", "dk", "dv")}
    if mutate is not None:
        mutate(d)
    ptr = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())  # noqa: E731
    lse_p = ptr(a["lse"]) if lse == "default" else lse
    delta_p = ptr(a["delta"]) if delta == "default" else delta
    return lib.varlen_attn_bwd(*(ctypes.byref(d[n]) for n in ("q", "k", "v", "out", "dout")), lse_p,
                               ptr(a["cu"]), 1, window, scale, ptr(a["sinks"]),
                               *(ctypes.byref(d[n]) for n in ("dq", "dk", "dv")), ptr(a["dsinks"]), delta_p, None)


@pytest.mark.parametrize("dim", [0, 1])
def test_bwd_rejects_dq_strides_beyond_32_bit_store_offsets(lib, dim):
    def big(d):
        d["dq"].stride[dim] = 1 << 24
    assert call_bwd(lib, bwd_args(), mutate=big) == SWA_ERR_UNSUPPORTED
    assert "dq" in lib.swa_last_error().decode()


def test_bwd_rejects_bad_arguments(lib):
    assert call_bwd(lib, bwd_args(), lse=None) == SWA_ERR_NULL
    assert call_bwd(lib, bwd_args(), delta=None) == SWA_ERR_NULL
    a = bwd_args()
    a["sinks"] = torch.zeros(4)
    assert call_bwd(lib, a) == SWA_ERR_NULL  # dsinks required with sinks
    assert call_bwd(lib, bwd_args(dtype=torch.float32)) == SWA_ERR_DTYPE
    for D in (32, 256):
        assert call_bwd(lib, bwd_args(D=D)) == SWA_ERR_UNSUPPORTED
    a = bwd_args()
    a["dk"] = torch.zeros(16, 4, 128, dtype=torch.bfloat16)
    assert call_bwd(lib, a) == SWA_ERR_SHAPE
    a = bwd_args()
    a["dout"] = torch.zeros(15, 4, 128, dtype=torch.bfloat16)
    assert call_bwd(lib, a) == SWA_ERR_SHAPE
    assert call_bwd(lib, bwd_args(Hq=3, Hkv=2)) == SWA_ERR_SHAPE
    assert call_bwd(lib, bwd_args(), window=-1) == SWA_ERR_ARG
    assert call_bwd(lib, bwd_args(), scale=0.0) == SWA_ERR_ARG
    a = bwd_args()
    a["dq"] = a["q"]
    assert call_bwd(lib, a) == SWA_ERR_ARG  # gradient aliases an input
    a = bwd_args(Hq=2, Hkv=2)
    a["dv"] = a["dk"]
    assert call_bwd(lib, a) == SWA_ERR_ARG  # two gradients share storage


def test_bwd_empty_problem_is_a_no_op(lib):
    assert call_bwd(lib, bwd_args(T=0)) == SWA_OK
