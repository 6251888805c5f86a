"""Packed variable-length causal / sliding-window GQA attention forward for MI355X (gfx950).

The compute lives in the HIP library ``libswattn.so`` built from ``csrc/``;
``binding`` marshals torch tensors into its C ABI.  Importing this package
does not load the library: the first call does, and it raises if the library
was not built (there is no fallback path).
"""
__all__ = ["varlen_attn_fwd", "varlen_attn_bwd", "sparse_mla_fwd", "mla_value_proj", "sparse_mla", "library_path"]


def __getattr__(name):
    if name in __all__:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
