"""ORACLE -- test infrastructure only.

A plain double-precision CPU definition of sparse latent attention with a
per-head attention sink (the C source ``sparse_attn_ref.c`` beside this file
states the definition and the passages it follows).  Only the tests, the smoke
check and the benchmark's CPU-baseline leg import this package.  It shares no
code with the GPU library in ``sparse_top_latent_amd`` and imports nothing
from it.

``build()`` compiles the C source with gcc (-O2, OpenMP, no fast-math);
``sparse_attn_ref`` calls it through ctypes on numpy arrays.

Two readings where the pages are silent can be flipped: ``sink_scaled=True``
multiplies the sink logit by the softmax scale, and ``dedup=True`` counts a
repeated index once (the GLM index mask's reading) instead of once per
occurrence.  The defaults are the readings the GPU library implements; each
variant is pinned against its own brute force in the tests.

Parity unpinned: the pair layout of ``rotate_back`` (the pages call
apply_rotary_emb on the output's rotary dims with inverse=True but do not
show its body; the reading taken is DeepSeek's complex convention, consecutive
elements 2i, 2i+1 as real and imaginary parts).  The rotation itself is pinned.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sparse_attn_ref.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle into ``oracle/liboracle.so`` and return its path."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-Wall",
             "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _bind(path):
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.oracle_sparse_attn_f64.argtypes = [P, P, P, P, ctypes.c_float,
                                           I64, I64, I64, I64, I64, I64, P, P, P]
    lib.oracle_sparse_attn_f64.restype = ctypes.c_int
    lib.oracle_sparse_attn_f64_flags.argtypes = [P, P, P, P, ctypes.c_float,
                                                 I64, I64, I64, I64, I64, I64, ctypes.c_int,
                                                 P, P, P]
    lib.oracle_sparse_attn_f64_flags.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        _lib = _bind(_LIB_PATH)
    return _lib


def num_threads() -> int:
    """OpenMP threads the oracle uses (OMP_NUM_THREADS or all cores)."""
    return int(_load().oracle_num_threads())


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


SINK_SCALED = 1   # flag values of the C entry point
DEDUP = 2


def sparse_attn_ref(q_bits, kv_bits, sink, idxs, scale, *, weights: bool = False,
                    sink_scaled: bool = False, dedup: bool = False):
    return _call(_load(), q_bits, kv_bits, sink, idxs, scale, weights, sink_scaled, dedup)


def sparse_attn_2src_ref(q_bits, win_bits, cmp_bits, W, N, sink, idxs, scale):
    """The step over rows held in two buffers, as the pages define it: the
    window rows and the compressed rows are joined along the row axis and the
    compressed indices are offset by the window length (DeepSeek-V4.1 pages,
    "Output projection" page, Attention.forward excerpt, the cat of window_kv
    and compress_kv).  Entry j < W is win_bits[b, j]; j >= W is
    cmp_bits[b, j - W]; N is the joined row count."""
    win_bits = np.asarray(win_bits, dtype=np.uint16)
    cmp_bits = np.asarray(cmp_bits, dtype=np.uint16)
    if not (0 <= W <= N) or win_bits.shape[1] < W or cmp_bits.shape[1] < N - W:
        raise ValueError("W outside [0, N] or a buffer with too few rows")
    kv = np.concatenate([win_bits[:, :W], cmp_bits[:, :N - W]], axis=1)
    return sparse_attn_ref(q_bits, kv, sink, idxs, scale)


def e2m1_values(codes):
    """OCP MX FP4 (E2M1): bit 3 sign, bits 2-1 exponent with bias 1, bit 0
    mantissa; exponent 0 is subnormal (0 or 0.5).  The pages name FP4 for the
    compressed cache (DeepSeek-V4.1 pages, "blocks, re-index groups" page,
    compressor excerpt, fp4_act_quant with groups of 16)."""
    c = np.asarray(codes, dtype=np.int64)
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + 0.5 * m, np.maximum(e - 1, 0)))
    return np.where(c & 8, -mag, mag)


def e4m3_values(codes):
    """OCP FP8 E4M3 (float8_e4m3fn, the scale dtype of the same excerpt): bit 7
    sign, bits 6-3 exponent with bias 7, bits 2-0 mantissa; exponent 0 is
    subnormal (m * 2^-9); 0x7F and 0xFF are NaN; no infinities."""
    c = np.asarray(codes, dtype=np.int64)
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(c & 0x80, -mag, mag)


def fp4_records_to_rows(records, D):
    """Packed FP4 row records [.., R] -> float64 rows [.., D]: bytes 0..D/2-1
    hold the E2M1 codes (byte k: element 2k in the low nibble, 2k+1 in the high
    nibble), bytes D/2..D/2+D/16-1 the E4M3 scales of the groups of 16."""
    rec = np.asarray(records, dtype=np.uint8)
    codes = rec[..., :D // 2].astype(np.int64)
    el = np.stack([codes & 15, codes >> 4], axis=-1).reshape(*rec.shape[:-1], D)
    scales = e4m3_values(rec[..., D // 2:D // 2 + D // 16])
    return e2m1_values(el) * np.repeat(scales, 16, axis=-1)


def _f64_to_bf16_bits_exact(x):
    """float64 values that bf16 holds exactly (or NaN) -> bf16 bit patterns."""
    f = np.asarray(x, dtype=np.float32)
    if not np.array_equal(f.astype(np.float64), np.asarray(x, np.float64), equal_nan=True):
        raise ValueError("value not exact in float32")
    bits = f.view(np.uint32)
    nan = np.isnan(f)
    if np.any((bits & 0xFFFF)[~nan] != 0):
        raise ValueError("value not exact in bf16")
    return np.where(nan, np.uint16(0x7FC0), (bits >> 16).astype(np.uint16)).astype(np.uint16)


def sparse_attn_2src_fp4_ref(q_bits, win_bits, records, W, N, sink, idxs, scale):
    """The two-source step with the compressed rows given as packed FP4 records:
    each record is decoded to its exact values (E2M1 code times the E4M3 scale
    of its group of 16; exact in bf16), then the step is the same as for
    bf16 rows."""
    D = np.asarray(q_bits).shape[-1]
    rows = fp4_records_to_rows(records, D)
    return sparse_attn_2src_ref(q_bits, win_bits, _f64_to_bf16_bits_exact(rows), W, N, sink,
                                idxs, scale)


def topk_ref(scores, lens, k, offset):
    """The compressed segment of the index lists from indexer scores
    (DeepSeek-V4.1 pages, "blocks, re-index groups" page, _compress_topk_idxs
    excerpt: the top index_topk compressed positions per query, offset by the
    window length, -1 where fewer are visible).  Query q sees positions
    0 .. lens[q]-1 (all when lens is None); the min(k, visible) best scores are
    taken, NaN ranked below every number, -0 equal to +0, equal scores by
    ascending position; the positions + offset are listed in ascending order,
    then -1 up to k.  Returns int32 [Q, k]."""
    sc = np.asarray(scores, dtype=np.float64)
    Q, C = sc.shape
    out = np.full((Q, k), -1, dtype=np.int32)
    for qi in range(Q):
        L = C if lens is None else int(min(max(lens[qi], 0), C))
        row = sc[qi, :L]
        nan = np.isnan(row)
        # primary key: -value (NaN last), secondary: position
        primary = np.where(nan, np.inf, -np.where(row == 0, 0.0, row))
        order = np.lexsort((np.arange(L), nan.astype(np.int8), primary))
        take = np.sort(order[:min(k, L)])
        out[qi, :len(take)] = take + offset
    return out


def rotate_back(o, freqs, rd):
    """The output's rotary dims rotated back (DeepSeek-V4.1 pages, "Output
    projection" page, Attention.forward excerpt: apply_rotary_emb on
    o[..., -rd:] with freqs_cis and inverse=True).  o is float64 [B, T, H, D];
    freqs is float32 [T, rd/2, 2], the (cos, sin) of the angle of pair i at
    position t (freqs_cis[t, i] as real and imaginary parts).  Reading: pair i
    is the complex number o[..., D-rd+2i] + 1j * o[..., D-rd+2i+1], and the
    inverse multiplies it by conj(freqs_cis[t, i]).  The first D - rd dims are
    returned unchanged."""
    o = np.array(o, dtype=np.float64, copy=True)
    if rd == 0:
        return o
    D = o.shape[-1]
    f = np.asarray(freqs, dtype=np.float64)
    rot = f[..., 0] + 1j * f[..., 1]                      # freqs_cis [T, rd/2]
    z = o[..., D - rd::2] + 1j * o[..., D - rd + 1::2]    # [B, T, H, rd/2]
    z = z * np.conj(rot)[None, :, None, :]
    o[..., D - rd::2] = z.real
    o[..., D - rd + 1::2] = z.imag
    return o


def sparse_attn_rope_ref(q_bits, kv_bits, sink, idxs, scale, freqs, rd):
    """sparse_attn followed by the inverse rotation of the output's last rd
    dims (the two steps of the same excerpt, in that order)."""
    return rotate_back(sparse_attn_ref(q_bits, kv_bits, sink, idxs, scale), freqs, rd)


def ref_from_library(path):
    """The same interface over another build of the oracle's C entry point
    (the tests use it to run the pins against planted mistakes)."""
    lib = _bind(path)

    def fn(q_bits, kv_bits, sink, idxs, scale, *, weights: bool = False,
           sink_scaled: bool = False, dedup: bool = False):
        return _call(lib, q_bits, kv_bits, sink, idxs, scale, weights, sink_scaled, dedup)
    return fn


def _call(lib, q_bits, kv_bits, sink, idxs, scale, weights, sink_scaled=False, dedup=False):
    """fp64 sparse attention with a sink.

    q_bits  : uint16 bf16 bit patterns [B, T, H, D]
    kv_bits : uint16 bf16 bit patterns [B, N, D]
    sink    : float32 [H] or None (no sink)
    idxs    : int32 [B, T, K]; negative entries are unused
    scale   : Python float, rounded to float32 as the GPU boundary receives it
    sink_scaled, dedup : the alternative readings (see the module docstring)
    Returns out [B, T, H, D] float64, plus (w [B,T,H,K], w_sink [B,T,H]) when
    ``weights`` is true.  Raises ValueError on an index >= N.
    """
    q_bits = np.ascontiguousarray(q_bits, dtype=np.uint16)
    kv_bits = np.ascontiguousarray(kv_bits, dtype=np.uint16)
    idxs = np.ascontiguousarray(idxs, dtype=np.int32)
    if sink is not None:
        sink = np.ascontiguousarray(sink, dtype=np.float32)
    B, T, H, D = q_bits.shape
    Bk, N, Dk = kv_bits.shape
    Bi, Ti, K = idxs.shape
    if (Bk, Dk) != (B, D) or (Bi, Ti) != (B, T):
        raise ValueError("shape mismatch between q, kv and idxs")
    if sink is not None and sink.shape != (H,):
        raise ValueError("sink must have shape [H]")
    out = np.zeros((B, T, H, D), dtype=np.float64)
    w = np.zeros((B, T, H, K), dtype=np.float64) if weights else None
    ws = np.zeros((B, T, H), dtype=np.float64) if weights else None
    flags = (SINK_SCALED if sink_scaled else 0) | (DEDUP if dedup else 0)
    rc = lib.oracle_sparse_attn_f64_flags(
        _ptr(q_bits), _ptr(kv_bits), _ptr(sink), _ptr(idxs), ctypes.c_float(scale),
        B, T, H, D, N, K, flags, _ptr(out), _ptr(w), _ptr(ws))
    if rc == 1:
        raise ValueError("index list holds an entry >= N")
    if rc != 0:
        raise ValueError(f"oracle rejected the dimensions (code {rc})")
    if weights:
        return out, w, ws
    return out
