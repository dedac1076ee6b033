"""Seeded synthetic inputs for sparse latent attention.

This module only draws inputs: it holds none of the attention arithmetic, and
both the GPU path and the fp64 oracle are fed from it.  Shapes follow the
DeepSeek-V4.1 pages: 64 heads of width 512 with a 64-wide rotary tail
(config.json excerpt on the "blocks, re-index groups" page), a 128-row sliding
window and 512 selected compressed rows (same excerpt: window_size,
index_topk), compress ratio 2 or 1 (compress_ratios), window rows first and
compressed rows after them in one row space (Attention.forward excerpt on the
"Output projection" page: kv and the index lists are joined in that order).

Recipe (every tensor has its own stream: numpy PCG64 seeded with
SeedSequence([config_seed, tensor_id]), ids 0 = index lists, 1 = sink,
2 = q, 3 = kv):
  * q, kv: standard normal float32 rounded to bfloat16 (round to nearest even);
  * sink: standard normal float32;
  * kv rows that no index list of their sequence references hold NaN, so a
    stray read shows up in the output;
  * index lists: window segment first, then the compressed segment, each
    padded with -1 at its end (see each config below).
Only referenced rows are stored (``rows``/``vals`` per sequence), which keeps
the 2-9 GB key-value tensors of the long and ragged configs out of host memory;
``kv_device`` materialises the dense tensor on the GPU.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

BF16_NAN = np.uint16(0x7FC0)

CONFIG_SEEDS = {"tiny": 0, "decode": 1, "prefill": 2, "long": 3, "ragged": 4, "window": 5}


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def _rng(seed: int, tensor_id: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, tensor_id]))


@dataclass
class Workload:
    name: str
    B: int
    T: int
    H: int
    D: int
    N: int
    K: int
    scale: float
    seed: int
    idxs: np.ndarray                 # int32 [B, T, K]
    sink: np.ndarray                 # float32 [H]
    q: np.ndarray                    # uint16 bf16 bits [B, T, H, D]
    window_rows: int = 0             # rows [0, window_rows) are the window (raw or ring) rows
    rows: list = field(default_factory=list)   # per b: int64 sorted referenced row ids
    vals: list = field(default_factory=list)   # per b: uint16 [len(rows[b]), D]

    @property
    def queries(self) -> int:
        return self.B * self.T

    def valid_entries(self) -> int:
        return int((self.idxs >= 0).sum())

    def distinct_rows(self) -> int:
        """Distinct (sequence, row) pairs referenced by any list."""
        return int(sum(len(r) for r in self.rows))

    def kv_dense_host(self, b: int) -> np.ndarray:
        """uint16 [N, D] for sequence b (NaN in unreferenced rows)."""
        kv = np.full((self.N, self.D), BF16_NAN, dtype=np.uint16)
        kv[self.rows[b]] = self.vals[b]
        return kv

    def kv_host(self) -> np.ndarray:
        """uint16 [B, N, D]; only for configs that fit host memory comfortably."""
        return np.stack([self.kv_dense_host(b) for b in range(self.B)])

    def kv_device(self, device="cuda"):
        """Dense bf16 [B, N, D] torch tensor on ``device`` (plumbing only)."""
        import torch
        kv = torch.full((self.B, self.N, self.D), float("nan"), dtype=torch.bfloat16,
                        device=device)
        flat = kv.view(torch.int16).view(self.B * self.N, self.D)
        for b in range(self.B):
            if len(self.rows[b]) == 0:
                continue
            r = torch.from_numpy(self.rows[b] + b * self.N).to(device)
            v = torch.from_numpy(self.vals[b].view(np.int16)).to(device)
            flat.index_copy_(0, r, v)
        return kv

    def query_slice(self, b: int, t: int):
        """Inputs of the single query (b, t): q [1,1,H,D], kv [1,N,D], idxs [1,1,K]."""
        return (self.q[b:b + 1, t:t + 1], self.kv_dense_host(b)[None],
                self.idxs[b:b + 1, t:t + 1])

    def algorithmic_bytes(self) -> int:
        """Bytes the method must move: distinct KV rows, q, out, index lists, sink."""
        return (self.distinct_rows() * self.D * 2 + 2 * self.queries * self.H * self.D * 2
                + self.idxs.size * 4 + self.H * 4)

    def algorithmic_flops(self) -> int:
        """4*H*D per valid list entry (QK^T and PV multiply-adds)."""
        return 4 * self.H * self.D * self.valid_entries()


def _finish(name, B, T, H, D, N, K, scale, seed, idxs, window_rows=None) -> Workload:
    idxs = np.ascontiguousarray(idxs, dtype=np.int32)
    sink = _rng(seed, 1).standard_normal(H, dtype=np.float32)
    q = to_bf16_bits(_rng(seed, 2).standard_normal((B, T, H, D), dtype=np.float32))
    kv_rng = _rng(seed, 3)
    rows, vals = [], []
    for b in range(B):
        r = np.unique(idxs[b][idxs[b] >= 0]).astype(np.int64)
        rows.append(r)
        vals.append(to_bf16_bits(kv_rng.standard_normal((len(r), D), dtype=np.float32)))
    return Workload(name, B, T, H, D, N, K, scale, seed, idxs, sink, q,
                    N if window_rows is None else window_rows, rows, vals)


def make_tiny(seed: int = CONFIG_SEEDS["tiny"]) -> Workload:
    """B=1, T=16, H=8, D=128, K=24, N=48 (16 raw + 32 compressed rows).

    Slots 0..15: window row j when j <= t, else -1 (causal window over the 16
    raw rows).  Slots 16..23: 16 + eight distinct draws from the 32 compressed
    rows.  Then each entry becomes -1 independently with probability 0.1.
    """
    B, T, H, D, K, W, C = 1, 16, 8, 128, 24, 16, 32
    rng = _rng(seed, 0)
    idxs = np.full((B, T, K), -1, dtype=np.int32)
    for t in range(T):
        for j in range(W):
            idxs[0, t, j] = j if j <= t else -1
        idxs[0, t, W:] = W + rng.choice(C, 8, replace=False)
    drop = rng.random((B, T, K)) < 0.1
    idxs[drop] = -1
    return _finish("tiny", B, T, H, D, W + C, K, D ** -0.5, seed, idxs, W)


def make_decode(seed: int = CONFIG_SEEDS["decode"], B: int = 64, H: int = 64,
                D: int = 512) -> Workload:
    """B=64 sequences at context 16384, ratio 2: 128 ring slots + 8192 compressed rows.

    Slots 0..127 name ring rows 0..127; slots 128..639 are 128 + 512 distinct
    uniform draws from the 8192 compressed rows, in draw order.
    """
    W, C, K = 128, 8192, 640
    rng = _rng(seed, 0)
    idxs = np.empty((B, 1, K), dtype=np.int32)
    for b in range(B):
        idxs[b, 0, :W] = np.arange(W)
        idxs[b, 0, W:] = W + rng.choice(C, 512, replace=False)
    return _finish("decode", B, 1, H, D, W + C, K, 512 ** -0.5, seed, idxs, W)


def make_prefill(seed: int = CONFIG_SEEDS["prefill"], T: int = 4096, H: int = 64,
                 D: int = 512) -> Workload:
    """B=1, T=4096 from position 0, ratio 2: rows 0..T-1 raw, T..T+T/2-1 compressed.

    Query t: window rows max(0, t-127)..t, padded with -1 to 128 slots; then
    T + c for min(512, (t+1)//2) distinct draws c from the (t+1)//2 visible
    compressed rows, padded with -1 to 512 slots.
    """
    W, K = 128, 640
    C = T // 2
    rng = _rng(seed, 0)
    idxs = np.full((1, T, K), -1, dtype=np.int32)
    for t in range(T):
        lo = max(0, t - W + 1)
        n_w = t + 1 - lo
        idxs[0, t, :n_w] = np.arange(lo, t + 1)
        vis = (t + 1) // 2
        n_c = min(512, vis)
        if n_c:
            idxs[0, t, W:W + n_c] = T + rng.choice(vis, n_c, replace=False)
    return _finish("prefill", 1, T, H, D, T + C, K, 512 ** -0.5, seed, idxs, T)


def make_long(seed: int = CONFIG_SEEDS["long"], B: int = 32, H: int = 64,
              D: int = 512) -> Workload:
    """B=32, ratio 1: 128 ring rows + 65536 compressed rows per sequence.

    Compressed slots: 8 runs of 64 contiguous rows at uniform offsets in
    [0, 65536-64], redrawn until no two runs overlap; row = 128 + offset + i.
    """
    W, C, K, runs, run_len = 128, 65536, 640, 8, 64
    rng = _rng(seed, 0)
    idxs = np.empty((B, 1, K), dtype=np.int32)
    for b in range(B):
        offs: list[int] = []
        while len(offs) < runs:
            o = int(rng.integers(0, C - run_len + 1))
            if all(abs(o - p) >= run_len for p in offs):
                offs.append(o)
        idxs[b, 0, :W] = np.arange(W)
        idxs[b, 0, W:] = np.concatenate([W + o + np.arange(run_len) for o in offs])
    return _finish("long", B, 1, H, D, W + C, K, 512 ** -0.5, seed, idxs, W)


def make_ragged(seed: int = CONFIG_SEEDS["ragged"], B: int = 256, H: int = 64,
                D: int = 512) -> Workload:
    """B=256, ratio 2, context log-uniform in [256, 65536).

    ctx_b = floor(256 * 256**u), u ~ U[0,1).  Ring slots 0..127 are all valid;
    compressed slots are 128 + min(512, ctx_b//2) distinct draws from the
    ctx_b//2 visible compressed rows, padded with -1.
    """
    W, Cmax, K = 128, 32768, 640
    rng = _rng(seed, 0)
    ctx = np.floor(256.0 * 256.0 ** rng.random(B)).astype(np.int64)
    idxs = np.full((B, 1, K), -1, dtype=np.int32)
    for b in range(B):
        vis = int(ctx[b]) // 2
        n_c = min(512, vis)
        idxs[b, 0, :W] = np.arange(W)
        idxs[b, 0, W:W + n_c] = W + rng.choice(vis, n_c, replace=False)
    return _finish("ragged", B, 1, H, D, W + Cmax, K, 512 ** -0.5, seed, idxs, W)


def make_window(seed: int = CONFIG_SEEDS["window"], B: int = 64, H: int = 64,
                D: int = 512) -> Workload:
    """Pure sliding-window layer (compress ratio 0): K=128 ring slots, all valid."""
    W = 128
    idxs = np.tile(np.arange(W, dtype=np.int32), (B, 1, 1))
    return _finish("window", B, 1, H, D, W, W, 512 ** -0.5, seed, idxs)


MAKERS = {"tiny": make_tiny, "decode": make_decode, "prefill": make_prefill,
          "long": make_long, "ragged": make_ragged, "window": make_window}


def make(name: str, seed: int | None = None) -> Workload:
    fn = MAKERS[name]
    return fn() if seed is None else fn(seed)


def make_random(seed: int, B: int, T: int, H: int, D: int, N: int, K: int,
                p_unused: float = 0.2, allow_repeats: bool = False,
                scale: float | None = None) -> Workload:
    """Small generic case: each list is K draws from [0, N) (distinct unless
    ``allow_repeats``), then each entry becomes -1 with probability p_unused."""
    rng = _rng(seed, 0)
    idxs = np.empty((B, T, K), dtype=np.int32)
    for b in range(B):
        for t in range(T):
            if allow_repeats:
                idxs[b, t] = rng.integers(0, N, K)
            else:
                idxs[b, t] = rng.choice(N, K, replace=False)
    idxs[rng.random((B, T, K)) < p_unused] = -1
    sc = D ** -0.5 if scale is None else scale
    return _finish(f"random{seed}", B, T, H, D, N, K, sc, seed, idxs)


def make_freqs(seed: int, T: int, rd: int, theta: float = 10000.0) -> np.ndarray:
    """Synthetic rotary table, float32 [T, rd/2, 2] of (cos, sin): pair i at
    position p0 + t turns by (p0 + t) * theta^(-2i/rd), with the start
    position p0 drawn from [0, 65536) (tensor id 5 of the seed).  The pages
    build theirs with YaRN scaling, which only changes the angles."""
    p0 = int(_rng(seed, 5).integers(0, 65536))
    pos = np.arange(p0, p0 + T, dtype=np.float64)[:, None]
    inv = theta ** (-np.arange(0, rd, 2, dtype=np.float64) / rd)[None, :]
    ang = pos * inv
    return np.stack([np.cos(ang), np.sin(ang)], -1).astype(np.float32)


def make_fp4_records(seed: int, B: int, rows: int, D: int, R: int) -> np.ndarray:
    """Synthetic packed FP4 rows (uint8 [B, rows, R]): uniform E2M1 codes in the
    first D/2 bytes, then D/16 positive E4M3 scales with exponent field 4..5
    (2^-3 .. 2^-2 times 1 + m/8, around the amax/6 a group of 16 N(0,1) values
    gets), then zero padding.  Element RMS is about 1.  Tensor id 4 of the seed."""
    rng = _rng(seed, 4)
    rec = np.zeros((B, rows, R), dtype=np.uint8)
    rec[..., :D // 2] = rng.integers(0, 256, (B, rows, D // 2), dtype=np.uint8)
    exp = rng.integers(4, 6, (B, rows, D // 16))
    man = rng.integers(0, 8, (B, rows, D // 16))
    rec[..., D // 2:D // 2 + D // 16] = (exp << 3 | man).astype(np.uint8)
    return rec
