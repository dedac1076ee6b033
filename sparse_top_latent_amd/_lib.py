"""ctypes view of libsparse_attn.so (the C ABI declared in include/sparse_attn.h).

Loading fails loudly when the library has not been built: there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsparse_attn.so")

SYMBOLS = (
    "sparse_attn_plan_splits",
    "sparse_attn_workspace_bytes",
    "sparse_attn_workspace_bytes_splits",
    "sparse_attn_fwd",
    "sparse_attn_fwd_splits",
    "sparse_attn_fwd_noalloc",
    "sparse_attn_noalloc_max_bytes",
    "sparse_attn_fwd_rope",
    "sparse_attn_fwd_2src",
    "sparse_attn_fwd_2src_fp4",
    "sparse_attn_fp4_record_bytes",
    "sparse_attn_fwd_partial",
    "sparse_attn_fwd_combine",
    "sparse_attn_check_idxs",
    "sparse_attn_topk",
    "sparse_attn_plan_kernel",
    "sparse_attn_status_str",
)

STATUS = {0: "SA_OK", 1: "SA_ERR_NULL", 2: "SA_ERR_SHAPE", 3: "SA_ERR_UNSUPPORTED",
          4: "SA_ERR_ALIGN", 5: "SA_ERR_WORKSPACE", 6: "SA_ERR_INDEX_RANGE", 7: "SA_ERR_HIP",
          8: "SA_ERR_SPLITS"}
SA_ERR_INDEX_RANGE = 6


class SaDims(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32),
                ("D", ctypes.c_int32), ("N", ctypes.c_int32), ("K", ctypes.c_int32)]


_lib = None


def lib():
    """The loaded library; raises if it was never built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build the HIP library first "
                "(python -c 'import __graft_entry__ as g; g.build()')")
        L = ctypes.CDLL(LIB_PATH)
        P, F, I32, SZ = ctypes.c_void_p, ctypes.c_float, ctypes.c_int32, ctypes.c_size_t
        D = ctypes.POINTER(SaDims)
        L.sparse_attn_plan_splits.argtypes = [D]
        L.sparse_attn_plan_splits.restype = I32
        L.sparse_attn_workspace_bytes.argtypes = [D]
        L.sparse_attn_workspace_bytes.restype = SZ
        L.sparse_attn_workspace_bytes_splits.argtypes = [D, I32]
        L.sparse_attn_workspace_bytes_splits.restype = SZ
        L.sparse_attn_fwd.argtypes = [P, P, P, P, F, P, D, P, SZ, P]
        L.sparse_attn_fwd.restype = ctypes.c_int
        L.sparse_attn_fwd_splits.argtypes = [P, P, P, P, F, P, D, I32, P, SZ, P]
        L.sparse_attn_fwd_splits.restype = ctypes.c_int
        L.sparse_attn_fwd_noalloc.argtypes = [P, P, P, P, F, P, D, I32, P]
        L.sparse_attn_fwd_noalloc.restype = ctypes.c_int
        L.sparse_attn_noalloc_max_bytes.argtypes = []
        L.sparse_attn_noalloc_max_bytes.restype = SZ
        L.sparse_attn_fwd_rope.argtypes = [P, P, P, P, F, P, I32, P, D, I32, P, SZ, P]
        L.sparse_attn_fwd_rope.restype = ctypes.c_int
        L.sparse_attn_fwd_2src.argtypes = [P, P, I32, P, I32, I32, P, P, F, P, D, I32, P, SZ, P]
        L.sparse_attn_fwd_2src.restype = ctypes.c_int
        L.sparse_attn_fwd_2src_fp4.argtypes = [P, P, I32, P, I32, I32, P, P, F, P, D, I32, P, SZ, P]
        L.sparse_attn_fwd_2src_fp4.restype = ctypes.c_int
        L.sparse_attn_fp4_record_bytes.argtypes = [I32]
        L.sparse_attn_fp4_record_bytes.restype = I32
        L.sparse_attn_fwd_partial.argtypes = [P, P, P, F, D, I32, P, SZ, P]
        L.sparse_attn_fwd_partial.restype = ctypes.c_int
        L.sparse_attn_fwd_combine.argtypes = [P, P, D, I32, P, SZ, P]
        L.sparse_attn_fwd_combine.restype = ctypes.c_int
        L.sparse_attn_check_idxs.argtypes = [P, D, P, P]
        L.sparse_attn_check_idxs.restype = ctypes.c_int
        L.sparse_attn_topk.argtypes = [P, P, I32, I32, I32, I32, P, ctypes.c_int64, P]
        L.sparse_attn_topk.restype = ctypes.c_int
        L.sparse_attn_plan_kernel.argtypes = [D, I32]
        L.sparse_attn_plan_kernel.restype = ctypes.c_char_p
        L.sparse_attn_status_str.argtypes = [ctypes.c_int]
        L.sparse_attn_status_str.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_str(rc: int) -> str:
    return lib().sparse_attn_status_str(rc).decode()


def check(rc: int, what: str) -> None:
    if rc != 0:
        raise RuntimeError(f"{what}: {STATUS.get(rc, rc)} ({status_str(rc)})")
