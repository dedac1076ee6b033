"""Python binding of the sparse_attn C ABI.

Argument marshalling only: dtype/shape/device checks, allocation of the output
and workspace through torch, and the call on torch's current HIP stream.  All
arithmetic runs in the HIP kernels of libsparse_attn.so.

The argument order follows the call on the DeepSeek-V4.1 "Output projection"
page (Attention.forward excerpt): sparse_attn(q, kv, attn_sink, topk_idxs,
softmax_scale).
"""
from __future__ import annotations

import ctypes

import numpy as np

import torch

from . import _lib
from ._lib import SaDims


def _dims(q, kv, idxs) -> SaDims:
    if q.dim() != 4 or kv.dim() != 3 or idxs.dim() != 3:
        raise ValueError("expected q [B,T,H,D], kv [B,N,D], idxs [B,T,K]")
    B, T, H, D = q.shape
    if kv.shape[0] != B or kv.shape[2] != D:
        raise ValueError(f"kv shape {tuple(kv.shape)} does not match q {tuple(q.shape)}")
    if idxs.shape[0] != B or idxs.shape[1] != T:
        raise ValueError(f"idxs shape {tuple(idxs.shape)} does not match q {tuple(q.shape)}")
    return SaDims(B, T, H, D, kv.shape[1], idxs.shape[2])


def _check_tensors(q, kv, sink, idxs):
    if q.dtype != torch.bfloat16 or kv.dtype != torch.bfloat16:
        raise TypeError("q and kv must be bfloat16")
    if idxs.dtype != torch.int32:
        raise TypeError("idxs must be int32")
    if sink is not None and (sink.dtype != torch.float32 or sink.dim() != 1
                             or sink.shape[0] != q.shape[2]):
        raise TypeError("sink must be float32 [H] or None")
    for name, t in (("q", q), ("kv", kv), ("idxs", idxs), ("sink", sink)):
        if t is None:
            continue
        if not t.is_cuda or t.device != q.device:
            raise ValueError(f"{name} must be on the same GPU as q")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def plan_splits(q, kv, idxs) -> int:
    with torch.cuda.device(q.device):
        r = _lib.lib().sparse_attn_plan_splits(ctypes.byref(_dims(q, kv, idxs)))
    if r < 0:
        _lib.check(-r, "sparse_attn_plan_splits")
    return int(r)


def plan_kernel(q, kv, idxs, num_splits: int = 0) -> str:
    """Name of the attention kernel a call would launch (for reports)."""
    with torch.cuda.device(q.device):
        r = _lib.lib().sparse_attn_plan_kernel(ctypes.byref(_dims(q, kv, idxs)), num_splits)
    if r is None:
        raise RuntimeError("sparse_attn_plan_kernel: bad arguments or device query failed")
    return r.decode()


def workspace_bytes(q, kv, idxs, num_splits: int = 0) -> int:
    """sparse_attn_workspace_bytes (num_splits 0: the planned count) or
    sparse_attn_workspace_bytes_splits."""
    L = _lib.lib()
    with torch.cuda.device(q.device):
        dims = ctypes.byref(_dims(q, kv, idxs))
        if num_splits == 0:
            return int(L.sparse_attn_workspace_bytes(dims))
        return int(L.sparse_attn_workspace_bytes_splits(dims, num_splits))


def sparse_attn(q, kv, sink, idxs, scale: float, out=None, num_splits: int = 0,
                workspace=None, checked: bool = False):
    """o[b,t,h] = softmax over {sink_h} U {scale <q[b,t,h], kv[b,j]> : j in idxs[b,t], j >= 0}
    applied to the rows kv[b,j] (the sink carries no value).  Returns bf16 [B,T,H,D].

    num_splits 0 calls sparse_attn_fwd with the planned split count (the
    workspace it needs is allocated here when none is given); 1..64 call
    sparse_attn_fwd_splits.  checked=True first counts list entries >= N on
    the device (sparse_attn_check_idxs, which synchronises to read the count)
    and raises SA_ERR_INDEX_RANGE when there is one."""
    _check_tensors(q, kv, sink, idxs)
    dims = _dims(q, kv, idxs)
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != torch.bfloat16 or not out.is_contiguous():
        raise ValueError("out must be a contiguous bf16 tensor shaped like q")
    if checked and check_idxs(idxs, kv.shape[1]) > 0:
        _lib.check(_lib.SA_ERR_INDEX_RANGE, "sparse_attn (checked)")
    L = _lib.lib()
    with torch.cuda.device(q.device):
        need = workspace_bytes(q, kv, idxs, num_splits)
        if workspace is None and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        if num_splits == 0:
            rc = L.sparse_attn_fwd(_ptr(q), _ptr(kv), _ptr(sink), _ptr(idxs),
                                   ctypes.c_float(scale), _ptr(out), ctypes.byref(dims),
                                   _ptr(workspace), ws_bytes, _stream(q.device))
            what = "sparse_attn_fwd"
        else:
            rc = L.sparse_attn_fwd_splits(_ptr(q), _ptr(kv), _ptr(sink), _ptr(idxs),
                                          ctypes.c_float(scale), _ptr(out), ctypes.byref(dims),
                                          num_splits, _ptr(workspace), ws_bytes,
                                          _stream(q.device))
            what = "sparse_attn_fwd_splits"
    _lib.check(rc, what)
    return out


def sparse_attn_rope(q, kv, sink, idxs, scale: float, freqs, rd: int, out=None,
                     num_splits: int = 0, workspace=None):
    """sparse_attn followed by the inverse rotary step on the output's last rd
    dims: pair i (dims D-rd+2i, D-rd+2i+1) of query (b, t) as a complex number
    times the conjugate of freqs[t, i] (freqs: float32 [T, rd/2, 2] of
    (cos, sin), e.g. torch.view_as_real of the complex freqs_cis slice), fused
    into the output's rounding."""
    _check_tensors(q, kv, sink, idxs)
    dims = _dims(q, kv, idxs)
    T, D = q.shape[1], q.shape[3]
    if freqs is not None:
        if freqs.dtype != torch.float32 or not freqs.is_contiguous() \
                or tuple(freqs.shape) != (T, rd // 2, 2) or freqs.device != q.device:
            raise ValueError("freqs must be a contiguous float32 [T, rd/2, 2] tensor on q's device")
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != torch.bfloat16 or not out.is_contiguous():
        raise ValueError("out must be a contiguous bf16 tensor shaped like q")
    L = _lib.lib()
    with torch.cuda.device(q.device):
        need = int(L.sparse_attn_workspace_bytes_splits(ctypes.byref(dims), num_splits))
        if workspace is None and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        rc = L.sparse_attn_fwd_rope(_ptr(q), _ptr(kv), _ptr(sink), _ptr(idxs),
                                    ctypes.c_float(scale), _ptr(freqs), rd, _ptr(out),
                                    ctypes.byref(dims), num_splits, _ptr(workspace), ws_bytes,
                                    _stream(q.device))
    _lib.check(rc, "sparse_attn_fwd_rope")
    return out


def sparse_attn_2src(q, kv_win, kv_cmp, W: int, N: int, sink, idxs, scale: float, out=None,
                     num_splits: int = 0, workspace=None):
    """sparse_attn over rows held in two buffers: list entry j < W is kv_win[b, j],
    j >= W is kv_cmp[b, j - W] (N = the index space, W <= kv_win.shape[1],
    N - W <= kv_cmp.shape[1]); equal to sparse_attn on the concatenated rows."""
    B, T, H, D = q.shape
    for t in (kv_win, kv_cmp):
        if t.dtype != torch.bfloat16 or not t.is_contiguous() or t.dim() != 3 or t.shape[0] != B \
                or t.shape[2] != D or t.device != q.device:
            raise ValueError("kv_win and kv_cmp must be contiguous bf16 [B, rows, D] on q's device")
    _check_tensors(q, kv_win, sink, idxs)
    dims = SaDims(B, T, H, D, N, idxs.shape[2])
    if out is None:
        out = torch.empty_like(q)
    L = _lib.lib()
    with torch.cuda.device(q.device):
        need = int(L.sparse_attn_workspace_bytes_splits(ctypes.byref(dims), num_splits))
        if workspace is None and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        rc = L.sparse_attn_fwd_2src(_ptr(q), _ptr(kv_win), kv_win.shape[1], _ptr(kv_cmp),
                                    kv_cmp.shape[1], W, _ptr(sink), _ptr(idxs),
                                    ctypes.c_float(scale), _ptr(out), ctypes.byref(dims),
                                    num_splits, _ptr(workspace), ws_bytes, _stream(q.device))
    _lib.check(rc, "sparse_attn_fwd_2src")
    return out


def fp4_record_bytes(D: int) -> int:
    """Bytes of one packed FP4 compressed-row record (288 at D = 512)."""
    return int(_lib.lib().sparse_attn_fp4_record_bytes(D))


def sparse_attn_2src_fp4(q, kv_win, cmp_records, W: int, N: int, sink, idxs, scale: float,
                         out=None, num_splits: int = 0, workspace=None):
    """sparse_attn_2src with the compressed rows as packed FP4 records
    (uint8 [B, rows, fp4_record_bytes(D)]): E2M1 codes and one E4M3 scale per 16
    elements; equal to sparse_attn_2src on the decoded bf16 rows."""
    B, T, H, D = q.shape
    R = fp4_record_bytes(D)
    if kv_win.dtype != torch.bfloat16 or not kv_win.is_contiguous() or kv_win.dim() != 3 \
            or kv_win.shape[0] != B or kv_win.shape[2] != D or kv_win.device != q.device:
        raise ValueError("kv_win must be a contiguous bf16 [B, rows, D] tensor on q's device")
    if cmp_records.dtype != torch.uint8 or not cmp_records.is_contiguous() \
            or cmp_records.dim() != 3 or cmp_records.shape[0] != B or cmp_records.shape[2] != R \
            or cmp_records.device != q.device:
        raise ValueError(f"cmp_records must be a contiguous uint8 [B, rows, {R}] tensor on q's device")
    _check_tensors(q, kv_win, sink, idxs)
    dims = SaDims(B, T, H, D, N, idxs.shape[2])
    if out is None:
        out = torch.empty_like(q)
    L = _lib.lib()
    with torch.cuda.device(q.device):
        need = int(L.sparse_attn_workspace_bytes_splits(ctypes.byref(dims), num_splits))
        if workspace is None and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        rc = L.sparse_attn_fwd_2src_fp4(_ptr(q), _ptr(kv_win), kv_win.shape[1], _ptr(cmp_records),
                                        cmp_records.shape[1], W, _ptr(sink), _ptr(idxs),
                                        ctypes.c_float(scale), _ptr(out), ctypes.byref(dims),
                                        num_splits, _ptr(workspace), ws_bytes, _stream(q.device))
    _lib.check(rc, "sparse_attn_fwd_2src_fp4")
    return out


def sparse_attn_partial(q, kv, idxs, scale: float, num_splits: int, workspace):
    """First kernel of the split path: per-split partials into ``workspace``."""
    _check_tensors(q, kv, None, idxs)
    dims = _dims(q, kv, idxs)
    with torch.cuda.device(q.device):
        rc = _lib.lib().sparse_attn_fwd_partial(
            _ptr(q), _ptr(kv), _ptr(idxs), ctypes.c_float(scale), ctypes.byref(dims),
            num_splits, _ptr(workspace), workspace.numel() * workspace.element_size(),
            _stream(q.device))
    _lib.check(rc, "sparse_attn_fwd_partial")


def sparse_attn_combine(q_shape, N: int, K: int, sink, out, num_splits: int, workspace):
    """Second kernel of the split path: merge the partials with the sink into ``out``."""
    B, T, H, D = q_shape
    dims = SaDims(B, T, H, D, N, K)
    with torch.cuda.device(out.device):
        rc = _lib.lib().sparse_attn_fwd_combine(
            _ptr(sink), _ptr(out), ctypes.byref(dims), num_splits, _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream(out.device))
    _lib.check(rc, "sparse_attn_fwd_combine")


def topk(scores, k: int, offset: int = 0, lens=None, out=None):
    """Compressed segment of the index lists: for each row of scores (fp32
    [..., C]) the positions + offset of the min(k, visible) best scores in
    ascending order, -1 after; lens (int32 [...]) limits the visible positions.
    ``out`` may be a strided view (e.g. lists[..., W:W + k]) whose last
    dimension is contiguous; it is written in place."""
    if scores.dtype != torch.float32 or not scores.is_contiguous() or not scores.is_cuda:
        raise TypeError("scores must be a contiguous float32 CUDA tensor")
    lead = scores.shape[:-1]
    C = scores.shape[-1]
    Q = int(np.prod(lead)) if len(lead) else 1
    if lens is not None:
        if lens.dtype != torch.int32 or not lens.is_contiguous() or lens.shape != lead \
                or lens.device != scores.device:
            raise TypeError("lens must be a contiguous int32 tensor shaped like scores[..., 0]")
    if out is None:
        out = torch.empty(*lead, k, dtype=torch.int32, device=scores.device)
    if out.dtype != torch.int32 or out.shape != (*lead, k) or out.stride(-1) != 1:
        raise ValueError("out must be int32 [..., k] with a contiguous last dimension")
    # rows of out must be evenly spaced
    stride = out.stride(-2) if out.dim() >= 2 else k
    if out.dim() >= 2 and not all(out.stride(i) == out.stride(i + 1) * out.shape[i + 1]
                                  for i in range(out.dim() - 2)):
        raise ValueError("out rows must be evenly spaced")
    with torch.cuda.device(scores.device):
        rc = _lib.lib().sparse_attn_topk(_ptr(scores), _ptr(lens), Q, C, k, offset, _ptr(out),
                                         stride, _stream(scores.device))
    _lib.check(rc, "sparse_attn_topk")
    return out


def check_idxs(idxs, N: int) -> int:
    """Number of entries >= N (checked mode); synchronises to read the count."""
    B, T, K = idxs.shape
    dims = SaDims(B, T, 1, 128, N, K)
    bad = torch.zeros(1, dtype=torch.int32, device=idxs.device)
    with torch.cuda.device(idxs.device):
        rc = _lib.lib().sparse_attn_check_idxs(_ptr(idxs), ctypes.byref(dims), _ptr(bad),
                                                _stream(idxs.device))
    _lib.check(rc, "sparse_attn_check_idxs")
    return int(bad.item())
