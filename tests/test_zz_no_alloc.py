"""The allocation-free entry point (sparse_attn_fwd_noalloc, split workspace in
the library's static device array) against sparse_attn_fwd_splits with a
caller's workspace, on the same inputs and split counts (needs the GPU)."""
import ctypes

import numpy as np
import pytest

from sparse_top_latent_amd import _lib, workloads as wl
from sparse_top_latent_amd._lib import SaDims

pytestmark = pytest.mark.gpu


def _inputs(w, torch):
    q = torch.from_numpy(w.q.view(np.int16)).cuda().view(torch.bfloat16)
    kv = w.kv_device("cuda")
    idx = torch.from_numpy(w.idxs).cuda()
    sink = torch.from_numpy(w.sink).cuda()
    return q, kv, idx, sink


def _call(L, name, q, kv, sink, idx, scale, out, d, S, torch, ws=None):
    P = ctypes.c_void_p
    st = P(torch.cuda.current_stream().cuda_stream)
    if name == "noalloc":
        return L.sparse_attn_fwd_noalloc(P(q.data_ptr()), P(kv.data_ptr()), P(sink.data_ptr()),
                                         P(idx.data_ptr()), ctypes.c_float(scale), P(out.data_ptr()),
                                         ctypes.byref(d), S, st)
    nb = 0 if ws is None else ws.numel()
    return L.sparse_attn_fwd_splits(P(q.data_ptr()), P(kv.data_ptr()), P(sink.data_ptr()),
                                    P(idx.data_ptr()), ctypes.c_float(scale), P(out.data_ptr()),
                                    ctypes.byref(d), S, None if ws is None else P(ws.data_ptr()),
                                    nb, st)


def test_noalloc_matches_the_workspace_entry_point(ref):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L = _lib.lib()
    # two calls in a row, the second with a smaller input: the decode batch at
    # its planned split count, then 8 queries at three splits, then one split
    for w, S in ((wl.make_decode(), 0), (wl.make_decode(B=8), 3), (wl.make_decode(B=4), 1)):
        q, kv, idx, sink = _inputs(w, torch)
        d = SaDims(w.B, w.T, w.H, w.D, w.N, w.K)
        Sx = S if S else L.sparse_attn_plan_splits(ctypes.byref(d))
        nb = L.sparse_attn_workspace_bytes_splits(ctypes.byref(d), Sx)
        assert nb <= L.sparse_attn_noalloc_max_bytes()
        ws = torch.empty(max(nb, 256), dtype=torch.uint8, device="cuda")
        exp_out = torch.empty_like(q)
        got_out = torch.full_like(q, float("nan"))
        assert _call(L, "splits", q, kv, sink, idx, w.scale, exp_out, d, Sx, torch,
                     ws if nb else None) == 0
        assert _call(L, "noalloc", q, kv, sink, idx, w.scale, got_out, d, S, torch) == 0
        torch.cuda.synchronize()
        a = exp_out.view(torch.int16).cpu().numpy()
        b = got_out.view(torch.int16).cpu().numpy()
        assert np.array_equal(a, b), f"B={w.B} S={Sx}: outputs differ"
        # and the oracle's bar on the noalloc output
        got = wl.bf16_bits_to_f32(b.view(np.uint16)).astype(np.float64)
        exps = []
        for bb in range(w.B):
            q1, kv1, i1 = w.query_slice(bb, 0)
            exps.append(ref(q1, kv1, w.sink, i1, w.scale)[0, 0])
        err = np.abs(got[:, 0] - np.stack(exps))
        assert err.max() <= 1e-2 and err.mean() <= 1e-3, (err.max(), err.mean())


def test_noalloc_rejects_a_workspace_beyond_its_array():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L = _lib.lib()
    d = SaDims(512, 1, 64, 512, 1024, 640)   # 512 queries at 64 splits: ~2 GB of partials
    A = ctypes.c_void_p(0x10000)
    assert L.sparse_attn_fwd_noalloc(A, A, None, A, ctypes.c_float(0.1), A, ctypes.byref(d), 64,
                                     None) == 5   # SA_ERR_WORKSPACE, before any launch
