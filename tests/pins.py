"""Independent checks that pin the fp64 oracle to the mathematics.

Each ``check_*`` takes an oracle-like callable with the signature of
``oracle.sparse_attn_ref`` and returns a short failure message, or None when the
check passes.  The same battery runs against the real oracle (it must pass
everything) and against planted mistakes in copies of the oracle's C source
(each must fail at least one check).

The brute force and the library special case below are written from the
definitions, not from the oracle:
  * dense masked attention: the GLM-5 page's DSA path builds a boolean mask from
    the index lists, fills unselected scores with the most negative value and
    takes an fp32 softmax before multiplying by the values (eager attention
    excerpt and index-mask excerpt); here the fill is -inf, the arithmetic is
    float64, and the per-head sink is one more logit column whose value row is
    zero;
  * torch's scaled_dot_product_attention in float64, with every row valid and
    the sink folded in as an extra key (an extra feature equal to sink/scale
    against a query feature of 1) whose value row is zero;
  * gathered dense attention: the listed rows gathered entry by entry (a
    repeated index gives a repeated key and value), a dense softmax over them
    plus the sink column, times the gathered values.  With repeats this counts
    an index once per occurrence, where the index mask above counts it once;
    the two brute forces pin the two readings of repeated indices.

The sink enters every brute force as a logit column.  The default reading
takes the sink as it is; the alternative (the sink multiplied by the softmax
scale) is pinned by giving the brute forces the column scale * sink.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import scipy.special

from sparse_top_latent_amd.workloads import (bf16_bits_to_f32, make_random, make_tiny,
                                             to_bf16_bits)

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
TOL = 1e-12


def dense_masked(q_bits, kv_bits, sink, idxs, scale):
    """Brute-force dense attention over all N rows with an index-list mask."""
    q = bf16_bits_to_f32(q_bits).astype(np.float64)
    kv = bf16_bits_to_f32(kv_bits).astype(np.float64)
    B, T, H, D = q.shape
    N = kv.shape[1]
    sc = float(np.float32(scale))
    out = np.zeros((B, T, H, D))
    for b in range(B):
        for t in range(T):
            lst = idxs[b, t]
            sel = np.zeros(N, dtype=bool)
            sel[lst[lst >= 0]] = True
            V = np.where(sel[:, None], kv[b], 0.0)       # unselected rows never matter
            logits = sc * (q[b, t] @ V.T)                  # [H, N]
            logits[:, ~sel] = -np.inf
            col = (np.asarray(sink, np.float64)[:, None] if sink is not None
                   else np.full((H, 1), -np.inf))
            full = np.concatenate([logits, col], axis=1)
            for h in range(H):
                if np.all(np.isneginf(full[h])):
                    continue                               # nothing to attend to: zero
                p = scipy.special.softmax(full[h])
                out[b, t, h] = p[:N] @ V
    return out


def gathered_dense(q_bits, kv_bits, sink_logit, idxs, scale):
    """Dense softmax over the rows gathered entry by entry (repeats included),
    plus the sink logit column with a zero value row."""
    q = bf16_bits_to_f32(q_bits).astype(np.float64)
    kv = bf16_bits_to_f32(kv_bits).astype(np.float64)
    B, T, H, D = q.shape
    sc = float(np.float32(scale))
    out = np.zeros((B, T, H, D))
    for b in range(B):
        for t in range(T):
            lst = idxs[b, t]
            G = kv[b, lst[lst >= 0]]                       # [n, D], repeats kept
            for h in range(H):
                z = -np.inf if sink_logit is None else float(sink_logit[h])
                logits = np.concatenate([sc * (G @ q[b, t, h]), [z]])
                if np.all(np.isneginf(logits)):
                    continue
                p = scipy.special.softmax(logits)
                out[b, t, h] = p[:-1] @ G
    return out


def sdpa_all_rows(q_bits, kv_bits, sink, scale):
    """torch SDPA (float64, CPU) over every row of kv[b], sink as an extra key."""
    import torch
    import torch.nn.functional as F
    q = torch.from_numpy(bf16_bits_to_f32(q_bits).astype(np.float64))
    kv = torch.from_numpy(bf16_bits_to_f32(kv_bits).astype(np.float64))
    B, T, H, D = q.shape
    N = kv.shape[1]
    sc = float(np.float32(scale))
    out = torch.zeros(B, T, H, D, dtype=torch.float64)
    for b in range(B):
        qh = q[b].permute(1, 0, 2).contiguous()            # [H, T, D]
        k = kv[b].expand(H, N, D).contiguous()
        v = k.clone()
        if sink is not None:
            qh = torch.cat([qh, torch.ones(H, T, 1, dtype=torch.float64)], -1)
            k = torch.cat([k, torch.zeros(H, N, 1, dtype=torch.float64)], -1)
            extra = torch.zeros(H, 1, D + 1, dtype=torch.float64)
            extra[:, 0, D] = torch.from_numpy(np.asarray(sink, np.float64)) / sc
            k = torch.cat([k, extra], 1)
            v = torch.cat([v, torch.zeros(H, 1, D, dtype=torch.float64)], 1)
        o = F.scaled_dot_product_attention(qh, k, v, scale=sc)
        out[b] = o.permute(1, 0, 2)
    return out.numpy()


def _err(a, b):
    return float(np.max(np.abs(np.asarray(a) - np.asarray(b)))) if np.size(a) else 0.0


def _kv(w):
    return w.kv_host()


# ---------------------------------------------------------------- the battery

def check_hand_worked(ref):
    fx = json.load(open(os.path.join(GOLDEN, "hand_worked_sink_attention.json")))
    q = to_bf16_bits(np.array(fx["q"], np.float32))
    kv = to_bf16_bits(np.array(fx["kv"], np.float32))
    sink = np.array(fx["sink"], np.float32)
    idxs = np.array(fx["idxs"], np.int32)
    out, w, ws = ref(q, kv, sink, idxs, fx["scale"], weights=True)
    e = max(_err(out, fx["expected_out"]), _err(w, fx["expected_weights"]),
            _err(ws, fx["expected_sink_weight"]))
    return None if e <= TOL else f"hand-worked example off by {e:.3g}"


def check_bruteforce(ref):
    cases = [make_tiny(), make_random(11, 2, 3, 4, 32, 40, 12),
             make_random(12, 1, 2, 16, 64, 30, 30, p_unused=0.0),
             make_random(13, 3, 2, 2, 8, 9, 9, p_unused=0.5, scale=0.7)]
    for w in cases:
        kv = _kv(w)
        for sink in (w.sink, None):
            got = ref(w.q, kv, sink, w.idxs, w.scale)
            exp = dense_masked(w.q, kv, sink, w.idxs, w.scale)
            e = _err(got, exp)
            if not e <= TOL:
                return f"brute force ({w.name}, sink={sink is not None}) off by {e:.3g}"
    return None


def check_sdpa(ref):
    for seed, (B, T, H, D, N) in enumerate([(2, 3, 4, 32, 17), (1, 2, 8, 128, 40)]):
        w = make_random(20 + seed, B, T, H, D, N, N, p_unused=0.0)
        kv = _kv(w)
        rng = np.random.default_rng(seed)
        full = np.stack([np.stack([rng.permutation(N) for _ in range(T)]) for _ in range(B)])
        full = full.astype(np.int32)
        for sink in (w.sink, None):
            e = _err(ref(w.q, kv, sink, full, w.scale), sdpa_all_rows(w.q, kv, sink, w.scale))
            if not e <= TOL:
                return f"SDPA special case (sink={sink is not None}) off by {e:.3g}"
    return None


def check_weights_sum(ref):
    w = make_random(30, 2, 4, 4, 16, 25, 10, p_unused=0.3)
    kv = _kv(w)
    for sink in (w.sink, None):
        _, p, pz = ref(w.q, kv, sink, w.idxs, w.scale, weights=True)
        tot = p.sum(-1) + pz
        any_valid = (w.idxs >= 0).any(-1)[..., None] | (sink is not None)
        target = np.where(any_valid, 1.0, 0.0)
        e = _err(tot, np.broadcast_to(target, tot.shape))
        if not e <= TOL:
            return f"weights + sink weight do not sum to 1 (off by {e:.3g})"
        if (p < 0).any() or (pz < 0).any():
            return "negative weight"
    return None


def check_permutation_and_padding(ref):
    w = make_random(31, 2, 3, 4, 32, 30, 12, p_unused=0.25)
    kv = _kv(w)
    base = ref(w.q, kv, w.sink, w.idxs, w.scale)
    rng = np.random.default_rng(5)
    perm = w.idxs.copy()
    for b in range(w.B):
        for t in range(w.T):
            perm[b, t] = perm[b, t][rng.permutation(w.K)]
    if not _err(ref(w.q, kv, w.sink, perm, w.scale), base) <= TOL:
        return "permuting a list changed the output"
    padded = np.concatenate([np.full((w.B, w.T, 3), -1, np.int32), w.idxs,
                             np.full((w.B, w.T, 5), -1, np.int32)], axis=-1)
    if not _err(ref(w.q, kv, w.sink, padded, w.scale), base) <= TOL:
        return "inserting -1 entries changed the output"
    return None


def check_independence(ref):
    w = make_random(32, 3, 2, 4, 16, 20, 8, p_unused=0.2)
    kv = _kv(w)
    base = ref(w.q, kv, w.sink, w.idxs, w.scale)
    kv2 = kv.copy()
    kv2[1] = to_bf16_bits(np.random.default_rng(1).standard_normal(kv2[1].shape,
                                                                    dtype=np.float32))
    o2 = ref(w.q, kv2, w.sink, w.idxs, w.scale)
    if not (_err(o2[0], base[0]) == 0 and _err(o2[2], base[2]) == 0):
        return "output of one sequence depends on another sequence's rows"
    s2 = w.sink.copy()
    s2[2] += 3.0
    o3 = ref(w.q, kv, s2, w.idxs, w.scale)
    keep = [h for h in range(w.H) if h != 2]
    if not _err(o3[:, :, keep], base[:, :, keep]) == 0:
        return "output of one head depends on another head's sink"
    if _err(o3[:, :, 2], base[:, :, 2]) == 0:
        return "the sink of a head has no effect on it"
    return None


def check_bound(ref):
    w = make_random(33, 2, 3, 4, 16, 20, 8, p_unused=0.2)
    kv = _kv(w)
    out, _, pz = ref(w.q, kv, w.sink, w.idxs, w.scale, weights=True)
    kvf = bf16_bits_to_f32(kv).astype(np.float64)
    for b in range(w.B):
        for t in range(w.T):
            lst = w.idxs[b, t][w.idxs[b, t] >= 0]
            if len(lst) == 0:
                continue
            mx = np.abs(kvf[b, lst]).max(0)
            for h in range(w.H):
                if np.any(np.abs(out[b, t, h]) > (1 - pz[b, t, h]) * mx + 1e-12):
                    return "output outside the convex-hull bound"
    return None


def check_closed_forms(ref):
    w = make_random(34, 1, 1, 4, 16, 6, 6, p_unused=0.0)
    kv = _kv(w)
    q = bf16_bits_to_f32(w.q).astype(np.float64)
    kvf = bf16_bits_to_f32(kv).astype(np.float64)
    sc = float(np.float32(w.scale))
    # one valid entry: o = logistic(s_j - sink_h) * kv_j
    idx = np.array([[[-1, 3, -1]]], np.int32)
    out = ref(w.q, kv, w.sink, idx, w.scale)
    for h in range(w.H):
        s = sc * float(q[0, 0, h] @ kvf[0, 3])
        g = 1.0 / (1.0 + math.exp(-(s - float(w.sink[h]))))
        if not _err(out[0, 0, h], g * kvf[0, 3]) <= TOL:
            return "single-entry closed form"
    # scale 0: o = sum kv_j / (|J| + exp(sink))
    idx = np.array([[[0, 2, 5, -1]]], np.int32)
    out = ref(w.q, kv, w.sink, idx, 0.0)
    for h in range(w.H):
        exp_o = kvf[0, [0, 2, 5]].sum(0) / (3 + math.exp(float(w.sink[h])))
        if not _err(out[0, 0, h], exp_o) <= TOL:
            return "zero-scale closed form"
    # all entries unused: o = 0 with or without a sink
    idx = np.full((1, 1, 4), -1, np.int32)
    for sink in (w.sink, None):
        if np.any(ref(w.q, kv, sink, idx, w.scale) != 0):
            return "all-unused list must give zero"
    # empty list (K = 0)
    if np.any(ref(w.q, kv, w.sink, np.zeros((1, 1, 0), np.int32), w.scale) != 0):
        return "empty list must give zero"
    # n copies of one row (gather semantics): o = v * n e^c / (n e^c + e^sink)
    n = 4
    idx = np.full((1, 1, n), 1, np.int32)
    out = ref(w.q, kv, w.sink, idx, w.scale)
    for h in range(w.H):
        c = sc * float(q[0, 0, h] @ kvf[0, 1])
        f = n * math.exp(c) / (n * math.exp(c) + math.exp(float(w.sink[h])))
        if not _err(out[0, 0, h], f * kvf[0, 1]) <= TOL:
            return "repeated-row closed form"
    # a huge sink takes all the weight
    big = np.full(w.H, 80.0, np.float32)
    if np.abs(ref(w.q, kv, big, w.idxs, w.scale)).max() > 1e-20:
        return "sink of +80 should leave essentially nothing for the rows"
    return None


def check_repeated_index_readings(ref):
    """Lists with repeated indices: by default each occurrence counts (the
    gathered brute force); with dedup=True an index counts once (the index-mask
    brute force).  The case is chosen so that the two readings differ."""
    w = make_random(35, 2, 3, 4, 16, 6, 10, p_unused=0.2, allow_repeats=True)
    kv = _kv(w)
    sc = float(np.float32(w.scale))
    for sink in (w.sink, None):
        per_occ = gathered_dense(w.q, kv, sink, w.idxs, w.scale)
        once = dense_masked(w.q, kv, sink, w.idxs, w.scale)
        if not _err(per_occ, once) > 1e-3:
            return "test case does not separate the two readings"
        e = _err(ref(w.q, kv, sink, w.idxs, w.scale), per_occ)
        if not e <= TOL:
            return f"repeated indices (per occurrence) off by {e:.3g}"
        e = _err(ref(w.q, kv, sink, w.idxs, w.scale, dedup=True), once)
        if not e <= TOL:
            return f"repeated indices (dedup) off by {e:.3g}"
        # both alternative readings at once
        z = None if sink is None else sc * np.asarray(sink, np.float64)
        e = _err(ref(w.q, kv, sink, w.idxs, w.scale, dedup=True, sink_scaled=True),
                 dense_masked(w.q, kv, z, w.idxs, w.scale))
        if not e <= TOL:
            return f"dedup with scaled sink off by {e:.3g}"
    return None


def check_scaled_sink_reading(ref):
    """sink_scaled=True: the sink logit is scale * sink (brute force with that
    column, and the single-entry closed form logistic(s_j - scale*sink))."""
    w = make_random(36, 2, 2, 4, 16, 20, 8, p_unused=0.2, scale=0.37)
    kv = _kv(w)
    sc = float(np.float32(w.scale))
    z = sc * np.asarray(w.sink, np.float64)
    got = ref(w.q, kv, w.sink, w.idxs, w.scale, sink_scaled=True)
    e = _err(got, dense_masked(w.q, kv, z, w.idxs, w.scale))
    if not e <= TOL:
        return f"scaled sink brute force off by {e:.3g}"
    if not _err(got, ref(w.q, kv, w.sink, w.idxs, w.scale)) > 1e-6:
        return "scaling the sink made no difference"
    q = bf16_bits_to_f32(w.q).astype(np.float64)
    kvf = bf16_bits_to_f32(kv).astype(np.float64)
    idx = np.full((w.B, w.T, 3), -1, np.int32)
    idx[:, :, 1] = 4
    out = ref(w.q, kv, w.sink, idx, w.scale, sink_scaled=True)
    for b in range(w.B):
        for t in range(w.T):
            for h in range(w.H):
                s = sc * float(q[b, t, h] @ kvf[b, 4])
                g = 1.0 / (1.0 + math.exp(-(s - z[h])))
                if not _err(out[b, t, h], g * kvf[b, 4]) <= TOL:
                    return "single-entry closed form with a scaled sink"
    return None


BATTERY = [check_hand_worked, check_bruteforce, check_sdpa, check_weights_sum,
           check_permutation_and_padding, check_independence, check_bound,
           check_closed_forms, check_repeated_index_readings, check_scaled_sink_reading]


def run_battery(ref):
    """Names and messages of the checks that fail for ``ref``."""
    fails = []
    for chk in BATTERY:
        try:
            msg = chk(ref)
        except Exception as exc:          # a crash of the oracle under test counts as a catch
            msg = f"raised {type(exc).__name__}: {exc}"
        if msg is not None:
            fails.append((chk.__name__, msg))
    return fails
