"""The seeded workloads against the shapes the pages fix (CPU only)."""
import json
import os

import numpy as np
import pytest

from sparse_top_latent_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def cfg():
    return json.load(open(os.path.join(GOLDEN, "deepseek_v41_attention_config.json")))


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1.0 + 2 ** -8 + 2 ** -20],
                 np.float32)
    back = wl.bf16_bits_to_f32(wl.to_bf16_bits(x))
    # 1+2^-8 is a tie between 1 and 1+2^-7 -> even (1); 1+3*2^-8 ties up to 1+2^-6;
    # just above the first tie rounds up
    np.testing.assert_array_equal(back, np.array([1.0, 1.0, 1.0 + 2 ** -6, -2.5,
                                                  1.0 + 2 ** -7], np.float32))


def test_decode_shapes_follow_config():
    c = cfg()
    w = wl.make_decode(B=4)
    assert (w.H, w.D) == (c["n_heads"], c["head_dim"])
    assert w.K == c["window_size"] + c["index_topk"]
    assert w.N == c["window_size"] + 16384 // 2
    assert w.scale == c["head_dim"] ** -0.5
    assert (w.idxs >= 0).all()
    for b in range(w.B):
        assert len(np.unique(w.idxs[b, 0])) == w.K          # distinct rows
        np.testing.assert_array_equal(w.idxs[b, 0, :128], np.arange(128))


def test_prefill_lists():
    c = cfg()
    w = wl.make_prefill(T=300, H=4, D=16)
    W = c["window_size"]
    for t in [0, 1, 2, 127, 128, 299]:
        lst = w.idxs[0, t]
        win = lst[:W][lst[:W] >= 0]
        np.testing.assert_array_equal(win, np.arange(max(0, t - W + 1), t + 1))
        comp = lst[W:][lst[W:] >= 0]
        assert len(comp) == min(c["index_topk"], (t + 1) // 2)
        assert len(np.unique(comp)) == len(comp)
        assert ((comp >= 300) & (comp < 300 + (t + 1) // 2)).all()
        # -1 only at the end of each segment
        assert (lst[:W][len(win):] == -1).all() and (lst[W:][len(comp):] == -1).all()


def test_long_runs_do_not_overlap():
    w = wl.make_long(B=3, H=4, D=16)
    for b in range(w.B):
        comp = w.idxs[b, 0, 128:]
        assert len(np.unique(comp)) == 512
        runs = comp.reshape(8, 64)
        assert (np.diff(runs, axis=1) == 1).all()
        assert ((comp >= 128) & (comp < w.N)).all()


def test_ragged_contexts_and_padding():
    w = wl.make_ragged(B=64, H=4, D=16)
    valid = (w.idxs >= 0).sum(-1).ravel()
    assert valid.min() >= 128 + 128 and valid.max() == 640
    assert (valid < 640).any()


def test_tiny_recipe():
    w = wl.make_tiny()
    assert (w.B, w.T, w.H, w.D, w.N, w.K) == (1, 16, 8, 128, 48, 24)
    frac = (w.idxs < 0).mean()
    assert 0.05 < frac < 0.5
    for t in range(16):
        win = w.idxs[0, t, :16]
        assert ((win == -1) | (win == np.arange(16))).all()
        assert (win[t + 1:] == -1).all()


def test_unreferenced_rows_are_nan_and_referenced_rows_finite():
    w = wl.make_random(3, 2, 2, 4, 16, 50, 6)
    kv = w.kv_host()
    f = wl.bf16_bits_to_f32(kv)
    for b in range(w.B):
        ref_rows = np.unique(w.idxs[b][w.idxs[b] >= 0])
        assert np.isfinite(f[b, ref_rows]).all()
        other = np.setdiff1d(np.arange(w.N), ref_rows)
        assert np.isnan(f[b, other]).all()


def test_generation_is_deterministic():
    a, b = wl.make_tiny(), wl.make_tiny()
    np.testing.assert_array_equal(a.idxs, b.idxs)
    np.testing.assert_array_equal(a.q, b.q)
    np.testing.assert_array_equal(a.kv_host(), b.kv_host())
