"""The C-ABI library without a GPU: it loads, exports every declared entry
point, and rejects bad arguments before making any HIP call."""
import ctypes
import os
import re

import pytest

from sparse_top_latent_amd import _lib
from sparse_top_latent_amd._lib import SaDims

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparse_attn.h")

SA_OK, SA_ERR_NULL, SA_ERR_SHAPE, SA_ERR_UNSUPPORTED, SA_ERR_ALIGN, SA_ERR_WORKSPACE, \
    SA_ERR_INDEX_RANGE, SA_ERR_HIP, SA_ERR_SPLITS = range(9)

# fake device addresses: never dereferenced, because every call below fails its
# argument checks first
A = ctypes.c_void_p(0x10000)
A2 = ctypes.c_void_p(0x20000)
MIS = ctypes.c_void_p(0x10002)


@pytest.fixture(scope="module")
def L():
    return _lib.lib()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(sparse_attn_\w+)\s*\(", text,
                                 flags=re.M)))


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert len(names) == 17
    assert set(names) == set(_lib.SYMBOLS)
    for n in names:
        assert hasattr(L, n), n


def declared_signature(name):
    """Parameter types and names of a declaration in the header, whitespace folded."""
    text = open(HEADER).read()
    m = re.search(r"\b" + name + r"\s*\(([^)]*)\)\s*;", text)
    assert m, name
    return [" ".join(p.split()) for p in m.group(1).split(",")]


def test_boundary_signatures_as_documented():
    # the page's call sparse_attn(q, kv, attn_sink, topk_idxs, softmax_scale)
    # with out, the dims, a workspace and the stream made explicit
    assert declared_signature("sparse_attn_fwd") == [
        "const void *q", "const void *kv", "const float *sink", "const int32_t *idxs",
        "float scale", "void *out", "const sa_dims *d", "void *workspace",
        "size_t workspace_bytes", "hipStream_t stream"]
    assert declared_signature("sparse_attn_workspace_bytes") == ["const sa_dims *d"]
    assert declared_signature("sparse_attn_fwd_splits") == [
        "const void *q", "const void *kv", "const float *sink", "const int32_t *idxs",
        "float scale", "void *out", "const sa_dims *d", "int32_t num_splits", "void *workspace",
        "size_t workspace_bytes", "hipStream_t stream"]
    assert declared_signature("sparse_attn_workspace_bytes_splits") == [
        "const sa_dims *d", "int32_t num_splits"]
    assert declared_signature("sparse_attn_check_idxs") == [
        "const int32_t *idxs", "const sa_dims *d", "int32_t *d_bad_count", "hipStream_t stream"]
    assert declared_signature("sparse_attn_status_str") == ["int status"]
    text = open(HEADER).read()
    for i, name in enumerate(["SA_OK", "SA_ERR_NULL", "SA_ERR_SHAPE", "SA_ERR_UNSUPPORTED",
                              "SA_ERR_ALIGN", "SA_ERR_WORKSPACE", "SA_ERR_INDEX_RANGE",
                              "SA_ERR_HIP", "SA_ERR_SPLITS"]):
        assert re.search(r"\b%s = %d\b" % (name, i), text), name


def dims(B=2, T=3, H=64, D=512, N=100, K=40):
    return ctypes.byref(SaDims(B, T, H, D, N, K))


def fwd(L, q=A, kv=A, sink=None, idxs=A, out=A2, d=None, S=1, ws=None, wsb=0):
    return L.sparse_attn_fwd_splits(q, kv, sink, idxs, ctypes.c_float(0.1), out,
                                    dims() if d is None else d, S, ws, wsb, None)


def fwd_planned(L, q=A, kv=A, sink=None, idxs=A, out=A2, d=None, ws=None, wsb=0):
    return L.sparse_attn_fwd(q, kv, sink, idxs, ctypes.c_float(0.1), out,
                             dims() if d is None else d, ws, wsb, None)


def test_status_strings(L):
    seen = set()
    for rc in range(9):
        s = _lib.status_str(rc)
        assert s and s not in seen
        seen.add(s)
    assert _lib.status_str(99) == "unknown status"


def test_dims_errors(L):
    assert fwd(L, d=ctypes.POINTER(SaDims)()) == SA_ERR_NULL
    assert fwd(L, d=dims(H=0)) == SA_ERR_SHAPE
    assert fwd(L, d=dims(D=0)) == SA_ERR_SHAPE
    assert fwd(L, d=dims(B=-1)) == SA_ERR_SHAPE
    assert fwd(L, d=dims(K=-1)) == SA_ERR_SHAPE
    assert fwd(L, d=dims(N=-5)) == SA_ERR_SHAPE
    assert fwd(L, d=dims(D=64)) == SA_ERR_UNSUPPORTED
    assert fwd(L, d=dims(D=100)) == SA_ERR_UNSUPPORTED
    assert fwd(L, d=dims(K=2049)) == SA_ERR_UNSUPPORTED
    # output rows (query, head) are numbered in 32 bits on the device
    assert fwd(L, d=dims(B=65536, T=512, H=64)) == SA_ERR_SHAPE  # B*T*H = 2^31
    assert L.sparse_attn_workspace_bytes_splits(dims(B=65536, T=512, H=64), 2) == 0


def test_pointer_errors(L):
    assert fwd(L, q=None) == SA_ERR_NULL
    assert fwd(L, kv=None) == SA_ERR_NULL
    assert fwd(L, idxs=None) == SA_ERR_NULL
    assert fwd(L, out=None) == SA_ERR_NULL
    assert fwd(L, q=MIS) == SA_ERR_ALIGN
    assert fwd(L, kv=MIS) == SA_ERR_ALIGN
    assert fwd(L, out=MIS) == SA_ERR_ALIGN
    assert fwd(L, idxs=ctypes.c_void_p(0x10001)) == SA_ERR_ALIGN
    assert fwd(L, sink=ctypes.c_void_p(0x10002)) == SA_ERR_ALIGN


def test_split_and_workspace_errors(L):
    assert fwd(L, S=-1) == SA_ERR_SPLITS
    assert fwd(L, S=65) == SA_ERR_SPLITS
    assert fwd(L, S=2) == SA_ERR_WORKSPACE                      # no workspace
    assert fwd(L, S=2, ws=A, wsb=16) == SA_ERR_WORKSPACE        # too small
    assert fwd(L, S=2, ws=ctypes.c_void_p(0x10010), wsb=1 << 30) == SA_ERR_ALIGN
    d = dims()
    assert L.sparse_attn_fwd_partial(A, A, A, ctypes.c_float(1.0), d, 1, A, 1 << 30,
                                     None) == SA_ERR_SPLITS
    assert L.sparse_attn_fwd_combine(None, A, d, 1, A, 1 << 30, None) == SA_ERR_SPLITS
    assert L.sparse_attn_fwd_combine(None, A, d, 2, None, 1 << 30, None) == SA_ERR_WORKSPACE
    assert L.sparse_attn_fwd_combine(None, A, d, 2, A, 16, None) == SA_ERR_WORKSPACE
    assert L.sparse_attn_fwd_combine(None, None, d, 2, A, 1 << 30, None) == SA_ERR_NULL


def test_zero_queries_is_a_noop(L):
    assert fwd(L, q=None, kv=None, idxs=None, out=None, d=dims(B=0)) == SA_OK
    assert fwd(L, q=None, kv=None, idxs=None, out=None, d=dims(T=0)) == SA_OK
    assert fwd_planned(L, q=None, kv=None, idxs=None, out=None, d=dims(B=0)) == SA_OK


def test_planned_entry_point_argument_errors(L):
    # one split without a workspace: argument errors come back before any HIP call
    assert fwd_planned(L, d=ctypes.POINTER(SaDims)()) == SA_ERR_NULL
    assert fwd_planned(L, d=dims(D=100)) == SA_ERR_UNSUPPORTED
    assert fwd_planned(L, q=None) == SA_ERR_NULL
    assert fwd_planned(L, out=MIS) == SA_ERR_ALIGN
    assert fwd_planned(L, d=dims(H=0)) == SA_ERR_SHAPE


def test_workspace_size_formula(L):
    B, T, H, D, S = 3, 5, 64, 512, 4
    got = L.sparse_attn_workspace_bytes_splits(dims(B=B, T=T, H=H, D=D), S)
    up = lambda x: (x + 255) // 256 * 256
    slots = B * T * S * H
    assert got == up(slots * D * 2) + 3 * up(slots * 4) + up(B * T * 4)
    assert L.sparse_attn_workspace_bytes_splits(dims(), 1) == 0
    assert L.sparse_attn_workspace_bytes_splits(dims(D=100), 2) == 0
    assert L.sparse_attn_workspace_bytes_splits(dims(), 65) == 0
    assert L.sparse_attn_workspace_bytes(dims(D=100)) == 0


def test_check_idxs_errors(L):
    assert L.sparse_attn_check_idxs(A, ctypes.POINTER(SaDims)(), A2, None) == SA_ERR_NULL
    assert L.sparse_attn_check_idxs(None, dims(), A2, None) == SA_ERR_NULL
    assert L.sparse_attn_check_idxs(A, dims(), None, None) == SA_ERR_NULL
    assert L.sparse_attn_check_idxs(A, dims(), ctypes.c_void_p(0x10001), None) == SA_ERR_ALIGN
    assert L.sparse_attn_check_idxs(None, dims(K=0), None, None) == SA_OK


def test_binding_refuses_cpu_tensors():
    import torch
    from sparse_top_latent_amd import sparse_attn
    q = torch.zeros(1, 1, 8, 128, dtype=torch.bfloat16)
    kv = torch.zeros(1, 4, 128, dtype=torch.bfloat16)
    idx = torch.zeros(1, 1, 2, dtype=torch.int32)
    with pytest.raises(ValueError):
        sparse_attn(q, kv, None, idx, 0.1)
    with pytest.raises(TypeError):
        sparse_attn(q.float(), kv, None, idx, 0.1)


def test_plan_kernel_rejects_bad_arguments(L):
    # argument errors come back as NULL before any device query
    assert L.sparse_attn_plan_kernel(None, 1) is None
    assert L.sparse_attn_plan_kernel(dims(D=100), 1) is None
    assert L.sparse_attn_plan_kernel(dims(), 65) is None
    assert L.sparse_attn_plan_kernel(dims(), -1) is None


def fwd2(L, q=A, win=A, win_rows=100, cmp=A, cmp_rows=100, W=40, d=None, S=1):
    return L.sparse_attn_fwd_2src(q, win, win_rows, cmp, cmp_rows, W, None, A,
                                  ctypes.c_float(0.1), A2, dims() if d is None else d, S, None,
                                  0, None)


def test_two_source_argument_errors(L):
    # dims() has N=100: entries j < W come from the window buffer, j >= W from
    # the compressed one; every error is reported before any HIP call
    assert fwd2(L, W=-1) == SA_ERR_SHAPE
    assert fwd2(L, W=101) == SA_ERR_SHAPE
    assert fwd2(L, W=40, win_rows=39) == SA_ERR_SHAPE          # window buffer too short
    assert fwd2(L, W=40, cmp_rows=59) == SA_ERR_SHAPE          # compressed buffer too short
    assert fwd2(L, W=40, win=None) == SA_ERR_NULL
    assert fwd2(L, W=40, cmp=None) == SA_ERR_NULL
    assert fwd2(L, W=40, win=ctypes.c_void_p(0x10008)) == SA_ERR_ALIGN
    assert fwd2(L, W=40, S=65) == SA_ERR_SPLITS
    assert fwd2(L, d=dims(D=100)) == SA_ERR_UNSUPPORTED
    # a NULL buffer that no entry can address is fine; zero queries is a no-op
    assert fwd2(L, q=None, win=None, cmp=None, d=dims(B=0), W=0) == SA_OK


def test_fp4_record_bytes_and_errors(L):
    assert L.sparse_attn_fp4_record_bytes(512) == 288
    assert L.sparse_attn_fp4_record_bytes(256) == 144
    assert L.sparse_attn_fp4_record_bytes(128) == 80     # 72 rounded up to 16
    assert L.sparse_attn_fp4_record_bytes(100) == 0
    f = lambda **kw: L.sparse_attn_fwd_2src_fp4(
        kw.get("q", A), A, 100, kw.get("rec", A), kw.get("rows", 100), kw.get("W", 40), None, A,
        ctypes.c_float(0.1), A2, kw.get("d", dims()), 1, None, 0, None)
    assert L.sparse_attn_fwd_2src_fp4(A, A, 100, A, 100, 40, None, A, ctypes.c_float(0.1), A2,
                                      None, 1, None, 0, None) == SA_ERR_NULL
    assert f(W=101) == SA_ERR_SHAPE
    assert f(rows=59) == SA_ERR_SHAPE
    assert f(rec=None) == SA_ERR_NULL
    assert f(rec=ctypes.c_void_p(0x10008)) == SA_ERR_ALIGN
    assert f(d=dims(D=100)) == SA_ERR_UNSUPPORTED


def test_rope_argument_errors(L):
    # rotary table: rd a multiple of 8 within D, freqs present and 16-byte aligned
    F = ctypes.c_void_p(0x20000)
    r = lambda rd=64, freqs=F, d=None: L.sparse_attn_fwd_rope(
        A, A, None, A, ctypes.c_float(0.1), freqs, rd, A2, dims() if d is None else d, 1, None,
        0, None)
    assert r(rd=-8) == SA_ERR_SHAPE
    assert r(rd=12) == SA_ERR_SHAPE
    assert r(rd=520) == SA_ERR_SHAPE          # dims() has D = 512
    assert r(freqs=None) == SA_ERR_NULL
    assert r(freqs=ctypes.c_void_p(0x20008)) == SA_ERR_ALIGN
    assert r(d=dims(B=0)) == SA_OK
    assert r(d=dims(B=0), rd=12) == SA_ERR_SHAPE


def test_topk_argument_errors(L):
    t = lambda scores=A, lens=None, Q=4, C=100, k=10, out=A2, stride=10: L.sparse_attn_topk(
        scores, lens, Q, C, k, 0, out, stride, None)
    assert t(Q=-1) == SA_ERR_SHAPE
    assert t(k=-1) == SA_ERR_SHAPE
    assert t(stride=9) == SA_ERR_SHAPE                       # rows would overlap
    assert t(out=None) == SA_ERR_NULL
    assert t(scores=None) == SA_ERR_NULL
    assert t(out=ctypes.c_void_p(0x20002)) == SA_ERR_ALIGN
    assert t(Q=0, out=None, scores=None) == SA_OK            # nothing to do
    assert t(k=0, out=None) == SA_OK
    assert L.sparse_attn_topk(A, None, 1, 2**31 - 5, 10, 100, A2, 10, None) == SA_ERR_SHAPE


def test_noalloc_argument_errors(L):
    # all rejected before any HIP call
    noalloc = lambda d, S=0, q=A: L.sparse_attn_fwd_noalloc(q, A, None, A, ctypes.c_float(0.1), A2,
                                                            d, S, None)
    assert noalloc(ctypes.POINTER(SaDims)()) == SA_ERR_NULL
    assert noalloc(dims(D=100)) == SA_ERR_UNSUPPORTED
    assert noalloc(dims(), S=65) == SA_ERR_SPLITS
    assert noalloc(dims(), S=-1) == SA_ERR_SPLITS
    assert noalloc(dims(B=0)) == SA_OK
    assert noalloc(dims(B=512, T=1, K=640), S=64) == SA_ERR_WORKSPACE
    assert L.sparse_attn_noalloc_max_bytes() == 33 << 20

