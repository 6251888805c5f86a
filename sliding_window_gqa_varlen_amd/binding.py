"""ctypes binding of libswattn.so (argument marshalling only).

The functions here turn torch tensors into ``swa_tensor`` descriptors, pick the
current HIP stream and call the C entry points of the same name.  No step of
the attention runs here; if the library is missing or a call fails, they
raise — there is no fallback.
"""
from __future__ import annotations

import ctypes
import math
import os
import threading
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libswattn.so"
_lock = threading.Lock()
_lib = None

SWA_DTYPE_F32, SWA_DTYPE_BF16, SWA_DTYPE_I32 = 0, 1, 2
_DTYPES = {torch.float32: SWA_DTYPE_F32, torch.bfloat16: SWA_DTYPE_BF16, torch.int32: SWA_DTYPE_I32}

# functions the header declares, with their ctypes signatures
EXPORTS = ("varlen_attn_fwd", "varlen_attn_bwd", "sparse_mla_fwd", "mla_value_proj", "swa_strerror", "swa_last_error",
           "swa_abi_version", "varlen_attn_bwd_noalloc", "swa_peak_mfma_bf16", "swa_peak_mfma_bf16_flops", "swa_peak_copy", "swa_peak_read")


class SwaTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 3), ("stride", ctypes.c_int64 * 3)]


class SwaError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str, text: str):
        super().__init__(f"{fn} failed with status {status} ({text}): {detail}")
        self.status = status


def library_path() -> str:
    return os.environ.get("SWATTN_LIB", os.path.join(_HERE, _LIB_NAME))


def load_library():
    """Load libswattn.so once; raise if it was not built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} not found: build it with `python -m sliding_window_gqa_varlen_amd.build`")
        lib = ctypes.CDLL(path)
        P = ctypes.POINTER(SwaTensor)
        vp, i32, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float
        lib.varlen_attn_fwd.argtypes = [P, P, P, vp, i32, i32, f32, vp, P, vp, vp]
        lib.varlen_attn_fwd.restype = i32
        lib.varlen_attn_bwd.argtypes = [P, P, P, P, P, vp, vp, i32, i32, f32, vp, P, P, P, vp, vp, vp]
        lib.varlen_attn_bwd.restype = i32
        lib.varlen_attn_bwd_noalloc.argtypes = [P, P, P, P, P, vp, vp, i32, i32, f32, vp, P, P, P, vp, vp]
        lib.varlen_attn_bwd_noalloc.restype = i32
        lib.sparse_mla_fwd.argtypes = [P, P, P, P, vp, f32, P, vp, vp]
        lib.sparse_mla_fwd.restype = i32
        lib.mla_value_proj.argtypes = [P, P, P, vp]
        lib.mla_value_proj.restype = i32
        lib.swa_strerror.argtypes = [i32]
        lib.swa_strerror.restype = ctypes.c_char_p
        lib.swa_last_error.argtypes = []
        lib.swa_last_error.restype = ctypes.c_char_p
        lib.swa_abi_version.argtypes = []
        lib.swa_abi_version.restype = i32
        i64 = ctypes.c_int64
        lib.swa_peak_mfma_bf16.argtypes = [vp, i32, vp]
        lib.swa_peak_mfma_bf16.restype = i32
        lib.swa_peak_mfma_bf16_flops.argtypes = [i32]
        lib.swa_peak_mfma_bf16_flops.restype = ctypes.c_double
        lib.swa_peak_copy.argtypes = [vp, vp, i64, vp]
        lib.swa_peak_copy.restype = i32
        lib.swa_peak_read.argtypes = [vp, i64, vp, vp]
        lib.swa_peak_read.restype = i32
        _lib = lib
        return lib


def describe(t: Optional[torch.Tensor]) -> Optional[SwaTensor]:
    """swa_tensor view of a torch tensor (rank <= 3; strides in elements)."""
    if t is None:
        return None
    if t.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {t.dtype}")
    if t.dim() > 3:
        raise ValueError("rank > 3")
    d = SwaTensor()
    d.data = t.data_ptr() if t.numel() > 0 else None
    d.dtype = _DTYPES[t.dtype]
    d.ndim = t.dim()
    for i in range(t.dim()):
        d.shape[i] = t.shape[i]
        d.stride[i] = t.stride(i)
    return d


def _on_gpu(name: str, t: torch.Tensor, device: torch.device, dtype=None, contiguous: bool = False,
            shape=None, min_numel: Optional[int] = None) -> None:
    """Raise unless t is a tensor on `device` (a GPU) with the stated dtype / layout / size.

    A host tensor would hand the kernel a host address, and a short or strided buffer behind
    a raw pointer would be read out of bounds: both are refused before the library is called.
    """
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU (got {t.device})")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, the operands on {device}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError(f"{name} must hold at least {min_numel} elements (got {t.numel()})")


def _operand_device(t: torch.Tensor) -> torch.device:
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"operands must be GPU tensors (got {getattr(t, 'device', type(t))})")
    return t.device


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _check(fn: str, status: int):
    if status != 0:
        lib = load_library()
        raise SwaError(fn, status, lib.swa_last_error().decode(), lib.swa_strerror(status).decode())


def varlen_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens: Optional[torch.Tensor],
                    n_docs: Optional[int] = None, window: int = 0, scale: Optional[float] = None,
                    sinks: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                    lse: Optional[torch.Tensor] = None, stream=None, return_lse: bool = True):
    """Packed varlen causal / sliding-window GQA attention forward on the GPU.

    q [T, Hq, D], k/v [T, Hkv, D] (bf16 or f32, on the GPU); cu_seqlens int32
    [n_docs + 1] on the GPU; window 0 = full causal; scale defaults to
    D ** -0.5; sinks optional fp32 [Hq].  Returns (out, lse) — lse is None when
    ``return_lse`` is False and no ``lse`` buffer is given.
    """
    lib = load_library()
    T, Hq, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if n_docs is None:
        n_docs = 0 if cu_seqlens is None else cu_seqlens.numel() - 1
    if out is None:
        out = torch.empty((T, Hq, D), dtype=q.dtype, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((T, Hq), dtype=torch.float32, device=q.device)
    dev = _operand_device(q)
    for name, x in (("k", k), ("v", v), ("out", out)):
        _on_gpu(name, x, dev)
    if int(n_docs) > 0:
        if cu_seqlens is None:
            raise ValueError("cu_seqlens is required when n_docs > 0")
        _on_gpu("cu_seqlens", cu_seqlens, dev, torch.int32, contiguous=True, min_numel=int(n_docs) + 1)
    elif cu_seqlens is not None:
        _on_gpu("cu_seqlens", cu_seqlens, dev, torch.int32, contiguous=True)
    if sinks is not None:
        _on_gpu("sinks", sinks, dev, torch.float32, contiguous=True, shape=(Hq,))
    if lse is not None:
        _on_gpu("lse", lse, dev, torch.float32, contiguous=True, shape=(T, Hq))
    dq, dk, dv, do = describe(q), describe(k), describe(v), describe(out)
    st = lib.varlen_attn_fwd(ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv), _ptr(cu_seqlens),
                             int(n_docs), int(window), float(scale), _ptr(sinks), ctypes.byref(do),
                             _ptr(lse), _stream(stream))
    _check("varlen_attn_fwd", st)
    return out, lse


def varlen_attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor, dout: torch.Tensor,
                    lse: torch.Tensor, cu_seqlens: Optional[torch.Tensor], n_docs: Optional[int] = None,
                    window: int = 0, scale: Optional[float] = None, sinks: Optional[torch.Tensor] = None,
                    dq: Optional[torch.Tensor] = None, dk: Optional[torch.Tensor] = None,
                    dv: Optional[torch.Tensor] = None, dsinks: Optional[torch.Tensor] = None,
                    delta: Optional[torch.Tensor] = None, stream=None):
    """Backward of varlen_attn_fwd (bf16, head_dim 64 or 128) from its out and lse.

    Returns (dq, dk, dv, dsinks) — dsinks is None without sinks.  ``delta`` is a
    [T, Hq] fp32 workspace (allocated here when not given; contents unspecified on return).
    """
    lib = load_library()
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if n_docs is None:
        n_docs = 0 if cu_seqlens is None else cu_seqlens.numel() - 1
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty((T, Hkv, D), dtype=q.dtype, device=q.device) if dk is None else dk
    dv = torch.empty((T, Hkv, D), dtype=q.dtype, device=q.device) if dv is None else dv
    if sinks is not None and dsinks is None:
        dsinks = torch.empty(Hq, dtype=torch.float32, device=q.device)
    if delta is None:
        delta = torch.empty((T, Hq), dtype=torch.float32, device=q.device)
    dev = _operand_device(q)
    for name, x in (("k", k), ("v", v), ("out", out), ("dout", dout), ("dq", dq), ("dk", dk), ("dv", dv)):
        _on_gpu(name, x, dev)
    for name, x in (("lse", lse), ("delta", delta)):
        _on_gpu(name, x, dev, torch.float32, contiguous=True, shape=(T, Hq))
    if int(n_docs) > 0:
        if cu_seqlens is None:
            raise ValueError("cu_seqlens is required when n_docs > 0")
        _on_gpu("cu_seqlens", cu_seqlens, dev, torch.int32, contiguous=True, min_numel=int(n_docs) + 1)
    elif cu_seqlens is not None:
        _on_gpu("cu_seqlens", cu_seqlens, dev, torch.int32, contiguous=True)
    if sinks is not None:
        _on_gpu("sinks", sinks, dev, torch.float32, contiguous=True, shape=(Hq,))
        _on_gpu("dsinks", dsinks, dev, torch.float32, contiguous=True, shape=(Hq,))
    ds = [describe(x) for x in (q, k, v, out, dout, dq, dk, dv)]
    st = lib.varlen_attn_bwd(*(ctypes.byref(d) for d in ds[:5]), _ptr(lse), _ptr(cu_seqlens), int(n_docs),
                             int(window), float(scale), _ptr(sinks), *(ctypes.byref(d) for d in ds[5:]),
                             _ptr(dsinks), _ptr(delta), _stream(stream))
    _check("varlen_attn_bwd", st)
    return dq, dk, dv, (dsinks if sinks is not None else None)


def varlen_attn_bwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor,
                            dout: torch.Tensor, lse: torch.Tensor, cu_seqlens: Optional[torch.Tensor],
                            n_docs: Optional[int] = None, window: int = 0, scale: Optional[float] = None,
                            sinks: Optional[torch.Tensor] = None, dq: torch.Tensor = None, dk: torch.Tensor = None,
                            dv: torch.Tensor = None, dsinks: Optional[torch.Tensor] = None, stream=None):
    """varlen_attn_bwd with its workspace in the library's device array (no allocation anywhere:
    dq, dk, dv and, with sinks, dsinks must be given).  Returns (dq, dk, dv, dsinks)."""
    lib = load_library()
    T, Hq, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if n_docs is None:
        n_docs = 0 if cu_seqlens is None else cu_seqlens.numel() - 1
    if dq is None or dk is None or dv is None or (sinks is not None and dsinks is None):
        raise ValueError("varlen_attn_bwd_noalloc allocates nothing: pass dq, dk, dv (and dsinks with sinks)")
    dev = _operand_device(q)
    for name, x in (("k", k), ("v", v), ("out", out), ("dout", dout), ("dq", dq), ("dk", dk), ("dv", dv)):
        _on_gpu(name, x, dev)
    _on_gpu("lse", lse, dev, torch.float32, contiguous=True, shape=(T, Hq))
    if int(n_docs) > 0:
        if cu_seqlens is None:
            raise ValueError("cu_seqlens is required when n_docs > 0")
        _on_gpu("cu_seqlens", cu_seqlens, dev, torch.int32, contiguous=True, min_numel=int(n_docs) + 1)
    if sinks is not None:
        _on_gpu("sinks", sinks, dev, torch.float32, contiguous=True, shape=(Hq,))
        _on_gpu("dsinks", dsinks, dev, torch.float32, contiguous=True, shape=(Hq,))
    ds = [describe(x) for x in (q, k, v, out, dout, dq, dk, dv)]
    st = lib.varlen_attn_bwd_noalloc(*(ctypes.byref(d) for d in ds[:5]), _ptr(lse), _ptr(cu_seqlens), int(n_docs),
                                     int(window), float(scale), _ptr(sinks), *(ctypes.byref(d) for d in ds[5:]),
                                     _ptr(dsinks), _stream(stream))
    _check("varlen_attn_bwd_noalloc", st)
    return dq, dk, dv, (dsinks if sinks is not None else None)


def sparse_mla_fwd(q: torch.Tensor, latent: torch.Tensor, k_pe: torch.Tensor, indices: torch.Tensor,
                   doc_ids: torch.Tensor, scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                   lse: Optional[torch.Tensor] = None, stream=None, return_lse: bool = True):
    """Sparse MLA forward: gathered top-k latent (512) + rotary (64) keys, value = latent.

    q [T, H, 576] bf16, latent [T, 512] bf16, k_pe [T, 64] bf16, indices int32
    [T, topk] (-1 = empty slot), doc_ids int32 [T]; scale defaults to q.shape[-1] ** -0.5.
    NoPE variant: q [T, H, 512] with k_pe [T, 0].
    Returns (out [T, H, 512] bf16, lse [T, H] fp32 or None).
    """
    lib = load_library()
    T, H, Dqk = q.shape
    Dl = latent.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(Dqk)
    if out is None:
        out = torch.empty((T, H, Dl), dtype=q.dtype, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((T, H), dtype=torch.float32, device=q.device)
    dev = _operand_device(q)
    for name, x in (("latent", latent), ("k_pe", k_pe), ("indices", indices), ("out", out)):
        _on_gpu(name, x, dev)
    _on_gpu("doc_ids", doc_ids, dev, torch.int32, contiguous=True, shape=(T,))
    if lse is not None:
        _on_gpu("lse", lse, dev, torch.float32, contiguous=True, shape=(T, H))
    dq, dl, dr, di, do = describe(q), describe(latent), describe(k_pe), describe(indices), describe(out)
    st = lib.sparse_mla_fwd(ctypes.byref(dq), ctypes.byref(dl), ctypes.byref(dr), ctypes.byref(di),
                            _ptr(doc_ids), float(scale), ctypes.byref(do), _ptr(lse), _stream(stream))
    _check("sparse_mla_fwd", st)
    return out, lse


def mla_value_proj(o_latent: torch.Tensor, value_weight: torch.Tensor, out: Optional[torch.Tensor] = None,
                   stream=None) -> torch.Tensor:
    """Value up-projection: out[t, h] = value_weight[h] @ o_latent[t, h].

    o_latent [T, H, 512] bf16, value_weight [H, Dv, 512] bf16 (Dv in {64, 128});
    returns out [T, H, Dv] bf16.
    """
    lib = load_library()
    T, H, _ = o_latent.shape
    Dv = value_weight.shape[1]
    if out is None:
        out = torch.empty((T, H, Dv), dtype=o_latent.dtype, device=o_latent.device)
    dev = _operand_device(o_latent)
    _on_gpu("value_weight", value_weight, dev)
    _on_gpu("out", out, dev)
    do, dw, dout = describe(o_latent), describe(value_weight), describe(out)
    st = lib.mla_value_proj(ctypes.byref(do), ctypes.byref(dw), ctypes.byref(dout), _stream(stream))
    _check("mla_value_proj", st)
    return out


def sparse_mla(q: torch.Tensor, latent: torch.Tensor, k_pe: torch.Tensor, indices: torch.Tensor,
               doc_ids: torch.Tensor, value_weight: torch.Tensor, scale: Optional[float] = None, stream=None,
               return_lse: bool = True):
    """Sparse MLA with the value up-projection: sparse_mla_fwd, then mla_value_proj.

    Returns (out [T, H, Dv] bf16, lse [T, H] fp32 or None).  The latent-space
    intermediate [T, H, 512] is a torch allocation on the same stream.
    """
    o, lse = sparse_mla_fwd(q, latent, k_pe, indices, doc_ids, scale, stream=stream, return_lse=return_lse)
    return mla_value_proj(o, value_weight, stream=stream), lse


# ------------------------------------------------------------- achievable-peak probes
def peak_mfma_bf16(iters: int, sink: torch.Tensor, stream=None) -> float:
    """Enqueue the bf16 MFMA-only loop (swa_peak_mfma_bf16); returns the flops it performs."""
    lib = load_library()
    _on_gpu("sink", sink, _operand_device(sink), torch.float32, min_numel=1)
    _check("swa_peak_mfma_bf16", lib.swa_peak_mfma_bf16(_ptr(sink), int(iters), _stream(stream)))
    return float(lib.swa_peak_mfma_bf16_flops(int(iters)))


def peak_copy(src: torch.Tensor, dst: torch.Tensor, stream=None) -> int:
    """Enqueue a streaming copy of src's bytes into dst; returns the bytes moved (read + write)."""
    lib = load_library()
    dev = _operand_device(src)
    _on_gpu("src", src, dev, contiguous=True)
    _on_gpu("dst", dst, dev, contiguous=True)
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < n:
        raise ValueError("dst is smaller than src")
    _check("swa_peak_copy", lib.swa_peak_copy(_ptr(src), _ptr(dst), n, _stream(stream)))
    return 2 * n


def peak_read(src: torch.Tensor, sink: torch.Tensor, stream=None) -> int:
    """Enqueue a streaming read of src; returns the bytes read."""
    lib = load_library()
    dev = _operand_device(src)
    _on_gpu("src", src, dev, contiguous=True)
    _on_gpu("sink", sink, dev, torch.float32, min_numel=1)
    n = src.numel() * src.element_size()
    _check("swa_peak_read", lib.swa_peak_read(_ptr(src), n, _ptr(sink), _stream(stream)))
    return n
