"""Sparse latent attention with a per-head attention sink on MI355X (gfx950).

The kernels live in libsparse_attn.so (C ABI: include/sparse_attn.h); this
package holds the thin binding (``api``), the in-tree build (``build``) and
the seeded input generators (``workloads``).
"""
__all__ = ["sparse_attn", "sparse_attn_rope", "sparse_attn_2src", "sparse_attn_2src_fp4", "fp4_record_bytes", "sparse_attn_partial", "sparse_attn_combine", "check_idxs", "topk",
           "plan_splits", "plan_kernel", "workspace_bytes"]


def __getattr__(name):
    if name in __all__:
        from . import api
        return getattr(api, name)
    raise AttributeError(name)
