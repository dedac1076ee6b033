"""HIP path against the fp64 oracle on the same seeded inputs (needs the GPU).

Bar (floating point): max-abs error <= 1e-2 and mean-abs error <= 1e-3 over
every compared output element, on inputs ~N(0,1).  The oracle is fp64; the GPU
path rounds the output to bf16 and feeds the softmax weights to the MFMA in
bf16, which keeps the expected error near 1e-4.
"""
import numpy as np
import pytest

from sparse_top_latent_amd import workloads as wl

pytestmark = pytest.mark.gpu

MAX_ABS = 1e-2
MEAN_ABS = 1e-3


def torch_mod():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def to_dev(w, idxs=None, sink=True, q_bits=None):
    torch = torch_mod()
    q = torch.from_numpy((w.q if q_bits is None else q_bits).view(np.int16)).cuda()
    q = q.view(torch.bfloat16)
    kv = w.kv_device("cuda")
    idx = torch.from_numpy(np.ascontiguousarray(w.idxs if idxs is None else idxs)).cuda()
    sk = torch.from_numpy(w.sink).cuda() if sink is True else (
        None if sink is None or sink is False else torch.from_numpy(np.asarray(sink, np.float32)).cuda())
    return q, kv, sk, idx


def run_gpu(w, num_splits=0, idxs=None, sink=True, q_bits=None):
    torch = torch_mod()
    from sparse_top_latent_amd import sparse_attn
    q, kv, sk, idx = to_dev(w, idxs, sink, q_bits)
    out = sparse_attn(q, kv, sk, idx, w.scale, num_splits=num_splits)
    torch.cuda.synchronize()
    bits = out.view(torch.int16).cpu().numpy().view(np.uint16)
    return wl.bf16_bits_to_f32(bits).astype(np.float64)


def sink_of(w, sink):
    if sink is True:
        return w.sink
    if sink is None or sink is False:
        return None
    return np.asarray(sink, np.float32)


def assert_close(got, exp, what=""):
    """max |err| / max(1, |exp|) <= 1e-2 and mean |err| <= 1e-3.

    On the configured workloads |exp| < 1 everywhere, so this is exactly the
    absolute bar.  Edge cases whose outputs exceed 1 in magnitude (one valid
    row, a huge query) get the bar relative to |exp|: a bf16 output holds 8
    significant bits, so its own rounding is up to 2^-9 |exp|."""
    assert got.shape == exp.shape
    assert np.isfinite(got).all(), f"{what}: non-finite GPU output"
    err = np.abs(got - exp)
    rel = err / np.maximum(1.0, np.abs(exp))
    mx = float(rel.max()) if err.size else 0.0
    mean = float(err.mean()) if err.size else 0.0
    print(f"{what}: max_abs={float(err.max()) if err.size else 0.0:.3e} "
          f"max_scaled={mx:.3e} mean_abs={mean:.3e}", flush=True)
    assert mx <= MAX_ABS and mean <= MEAN_ABS, f"{what}: max {mx:.3e} mean {mean:.3e}"


def check(ref, w, num_splits=0, idxs=None, sink=True, q_bits=None, what=""):
    lst = w.idxs if idxs is None else idxs
    got = run_gpu(w, num_splits, lst, sink, q_bits)
    exp = ref(w.q if q_bits is None else q_bits, w.kv_host(), sink_of(w, sink), lst, w.scale)
    assert_close(got, exp, what or f"{w.name} S={num_splits}")
    return got


# ------------------------------------------------------------------ small cases

@pytest.mark.parametrize("S", [0, 1, 2, 3])
@pytest.mark.parametrize("sink", [True, None])
def test_tiny(ref, S, sink):
    check(ref, wl.make_tiny(), S, sink=sink, what=f"tiny S={S} sink={sink is not None}")


@pytest.mark.parametrize("H,D", [(8, 128), (16, 256), (32, 512), (48, 512), (64, 512),
                                 (64, 128), (64, 256), (1, 128)])
@pytest.mark.parametrize("S", [1, 3])
def test_shapes_span_tiles_and_tail(ref, H, D, S):
    # K=173 with ~30% unused: several 32-row chunks and a ragged tail per split
    w = wl.make_random(100 + H + D, 2, 2, H, D, 300, 173, p_unused=0.3)
    check(ref, w, S, what=f"H={H} D={D} S={S}")


def test_empty_and_all_unused(ref):
    w = wl.make_random(7, 2, 3, 64, 512, 50, 8, p_unused=0.0)
    for S in (0, 1, 2):
        for sink in (True, None):
            got = run_gpu(w, S, np.full((2, 3, 8), -1, np.int32), sink)
            assert np.all(got == 0)
            got0 = run_gpu(w, S, np.zeros((2, 3, 0), np.int32), sink)
            assert got0.shape == (2, 3, 64, 512) and np.all(got0 == 0)


def test_single_entry_and_short_lists(ref):
    w = wl.make_random(8, 2, 2, 64, 512, 700, 641, p_unused=0.0)
    for K in (1, 24, 33, 641):
        lst = np.ascontiguousarray(w.idxs[..., :K])
        check(ref, w, 0, idxs=lst, what=f"K={K}")


@pytest.mark.parametrize("sinkval", [30.0, -30.0])
def test_extreme_sinks(ref, sinkval):
    w = wl.make_random(9, 2, 2, 64, 512, 200, 150, p_unused=0.2)
    for S in (1, 2):
        check(ref, w, S, sink=np.full(64, sinkval), what=f"sink={sinkval} S={S}")


def test_large_norm_queries(ref):
    w = wl.make_random(10, 2, 2, 64, 512, 200, 150, p_unused=0.2)
    q8 = wl.to_bf16_bits(wl.bf16_bits_to_f32(w.q) * 8.0)  # scores ~8x: stresses max rescaling
    for S in (1, 3):
        check(ref, w, S, q_bits=q8, what=f"8x query S={S}")


def test_large_magnitude_rows_on_the_split_path(ref):
    # rows ~2^20: a split's partial output would overflow fp16 without the
    # per-row power-of-two scale
    import copy
    w = copy.deepcopy(wl.make_random(15, 2, 2, 64, 512, 300, 200, p_unused=0.1))
    w.vals = [wl.to_bf16_bits(wl.bf16_bits_to_f32(v) * np.float32(2.0 ** 20)) for v in w.vals]
    # q scaled down by the same power of two keeps the scores (and the softmax)
    # as in the unscaled case, so the outputs are ~2^20 times a typical output
    q_small = wl.to_bf16_bits(wl.bf16_bits_to_f32(w.q) * np.float32(2.0 ** -20))
    exp = ref(q_small, w.kv_host(), w.sink, w.idxs, w.scale)
    assert np.abs(exp).max() > 65504.0   # beyond fp16 without the scale
    for S in (1, 2, 3):
        got = run_gpu(w, S, q_bits=q_small)
        # the output is linear in the rows: compare at the unscaled magnitude
        assert_close(got * 2.0 ** -20, exp * 2.0 ** -20, f"rows x 2^20 S={S}")


def test_small_magnitude_rows_on_the_split_path(ref):
    # rows ~2^-20: a split's partial output would sink into fp16 subnormals
    # (or flush to zero) unless each row is scaled up by its power of two
    import copy
    w = copy.deepcopy(wl.make_random(16, 2, 2, 64, 512, 300, 200, p_unused=0.1))
    w.vals = [wl.to_bf16_bits(wl.bf16_bits_to_f32(v) * np.float32(2.0 ** -20)) for v in w.vals]
    q_big = wl.to_bf16_bits(wl.bf16_bits_to_f32(w.q) * np.float32(2.0 ** 20))
    exp = ref(q_big, w.kv_host(), w.sink, w.idxs, w.scale)
    assert np.abs(exp).max() < 2.0 ** -14   # fp16 subnormal range without the scale
    for S in (1, 2, 3):
        got = run_gpu(w, S, q_bits=q_big)
        # the output is linear in the rows: compare at the unscaled magnitude
        assert_close(got * 2.0 ** 20, exp * 2.0 ** 20, f"rows x 2^-20 S={S}")


def test_sink_minus_infinity(ref):
    # a sink of -inf removes the sink from the softmax; with no valid entry as
    # well there is nothing to attend to and the output is 0 (never NaN), on
    # the one-split path as on the split path
    w = wl.make_random(17, 2, 2, 64, 512, 60, 8, p_unused=0.0)
    ninf = np.full(64, -np.inf, np.float32)
    one = np.full((2, 2, 8), -1, np.int32)
    one[..., 3] = w.idxs[..., 3]
    for S in (1, 2):
        got = run_gpu(w, S, np.full((2, 2, 8), -1, np.int32), ninf)
        assert np.all(got == 0), f"all unused, sink -inf, S={S}"
        check(ref, w, S, idxs=one, sink=ninf, what=f"one entry, sink -inf, S={S}")
        check(ref, w, S, sink=ninf, what=f"full lists, sink -inf, S={S}")


def test_permuted_lists_and_scattered_unused(ref):
    w = wl.make_random(11, 2, 2, 64, 512, 400, 300, p_unused=0.3)
    rng = np.random.default_rng(0)
    perm = w.idxs.copy()
    for b in range(2):
        for t in range(2):
            perm[b, t] = perm[b, t][rng.permutation(300)]
    a = check(ref, w, 0, what="unpermuted")
    b = check(ref, w, 0, idxs=perm, what="permuted")
    assert np.abs(a - b).max() <= 2 * MAX_ABS


def test_repeated_indices_count_per_occurrence(ref):
    w = wl.make_random(12, 1, 2, 64, 512, 20, 64, allow_repeats=True, p_unused=0.1)
    check(ref, w, 0, what="repeats")
    check(ref, w, 2, what="repeats S=2")


def test_entries_beyond_n_are_skipped(ref):
    w = wl.make_random(13, 2, 2, 64, 512, 200, 100, p_unused=0.1)
    bad = w.idxs.copy()
    bad[0, 0, 5] = w.N
    bad[1, 1, 50] = w.N + 1000
    clean = np.where(bad >= w.N, -1, bad).astype(np.int32)
    got = run_gpu(w, 0, bad)
    exp = ref(w.q, w.kv_host(), w.sink, clean, w.scale)
    assert_close(got, exp, "beyond-N skipped")


@pytest.mark.parametrize("S", [1, 2, 3, 4, 5, 6, 7, 8])
def test_split_counts_agree(ref, S):
    w = wl.make_decode(B=4)
    check(ref, w, S, what=f"decode B=4 S={S}")


def test_one_workspace_serves_many_calls(ref):
    # one workspace, calls with different split counts and batch sizes in a
    # row, each checked against the oracle
    torch = torch_mod()
    from sparse_top_latent_amd import api
    big = wl.make_decode(B=8)
    qb, kvb, skb, idxb = to_dev(big)
    ws = torch.empty(api.workspace_bytes(qb, kvb, idxb, 8), dtype=torch.uint8, device=qb.device)
    for B, S in ((8, 4), (8, 8), (3, 3), (8, 2), (8, 4)):
        w = wl.make_decode(B=B)
        q, kv, sk, idx = to_dev(w)
        out = api.sparse_attn(q, kv, sk, idx, w.scale, num_splits=S, workspace=ws)
        torch.cuda.synchronize()
        got = wl.bf16_bits_to_f32(out.view(torch.int16).cpu().numpy().view(np.uint16))
        exp = ref(w.q, w.kv_host(), w.sink, w.idxs, w.scale)
        assert_close(got.astype(np.float64), exp, f"shared workspace B={B} S={S}")


@pytest.mark.parametrize("S", [4, 6])
def test_combine_ignores_stale_workspace_slots(ref, S):
    # queries with 640 / 20 / 0 / 200 / 1 valid entries use 4 / 1 / 1 / 2 / 1
    # of the S split slots; the merge reads every slot's partial and scalars
    # before the plan entry arrives and masks the ones the plan leaves out, so
    # a workspace filled with NaN bits (0xFF bytes) must not reach the output.
    # H = 41 leaves lanes past the last output row in the merge's last block.
    torch = torch_mod()
    from sparse_top_latent_amd import api
    w = wl.make_random(460 + S, 5, 1, 41, 512, 700, 640, p_unused=0.0)
    idx = w.idxs.copy()
    for b, n in enumerate((640, 20, 0, 200, 1)):
        idx[b, 0, n:] = -1
    q, kv, sk, di = to_dev(w, idx)
    ws = torch.full((api.workspace_bytes(q, kv, di, S),), 0xFF, dtype=torch.uint8, device=q.device)
    for rep in range(2):
        out = api.sparse_attn(q, kv, sk, di, w.scale, num_splits=S, workspace=ws)
        torch.cuda.synchronize()
        got = wl.bf16_bits_to_f32(out.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
        assert_close(got, ref(w.q, w.kv_host(), w.sink, idx, w.scale), f"stale workspace S={S} call {rep}")
        ws.fill_(0xFF)


def test_bitwise_deterministic():
    w = wl.make_decode(B=8)
    for S in (1, 4):
        runs = [run_gpu(w, S) for _ in range(3)]
        assert np.array_equal(runs[0], runs[1]) and np.array_equal(runs[0], runs[2])


def test_check_idxs_counts_out_of_range():
    torch = torch_mod()
    from sparse_top_latent_amd import check_idxs
    w = wl.make_random(14, 3, 4, 8, 128, 100, 50, p_unused=0.2)
    bad = w.idxs.copy()
    bad[0, 0, 0] = 100
    bad[2, 3, 49] = 12345
    bad[1, 2, 7] = 100
    assert check_idxs(torch.from_numpy(w.idxs).cuda(), w.N) == 0
    assert check_idxs(torch.from_numpy(bad).cuda(), w.N) == 3


# ------------------------------------------------- many-query path (prefill)
# Launches with at least two workgroups per compute unit run the many-query
# kernel (two workgroups share a compute unit); these cases reach it at sizes
# the oracle finishes quickly.

def many_query_T(B=2):
    torch = torch_mod()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    return (2 * cus + 8 + B - 1) // B


@pytest.mark.parametrize("H,D", [(64, 512), (48, 512), (32, 256), (20, 128)])
def test_many_query_path(ref, H, D):
    # K=75 with ~30% unused: one full 32-row chunk, a ragged one, varying counts
    w = wl.make_random(200 + H + D, 2, many_query_T(), H, D, 160, 75, p_unused=0.3)
    check(ref, w, 0, what=f"many-query H={H} D={D}")


def test_plan_kernel_names_the_dispatch():
    import ctypes
    torch = torch_mod()
    from sparse_top_latent_amd import api, _lib
    w = wl.make_decode(B=4)
    q, kv, _, idx = to_dev(w)
    # few workgroups: 32 heads per workgroup (two of them per query and split)
    assert api.plan_kernel(q, kv, idx, 4) == "attn_fwd_kernel<512,2,1,false>"
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        # 64 queries x 4 splits fill the device with 64-head workgroups
        d = _lib.SaDims(64, 1, 64, 512, 8320, 640)
        name = _lib.lib().sparse_attn_plan_kernel(ctypes.byref(d), 4)
        assert name.decode() == "attn_fwd_kernel<512,4,1,false>"
    wm = wl.make_random(212, 2, many_query_T(), 64, 512, 60, 20)
    q, kv, _, idx = to_dev(wm)
    assert api.plan_kernel(q, kv, idx, 0) == "attn_fwd_mq_kernel<512,2,false>"


@pytest.mark.parametrize("S", [2, 3])
def test_sixty_four_head_workgroups(ref, S):
    # 80 queries: at 2 or 3 splits the 32-head workgroups would not fit 256
    # compute units in one round, so the 64-head shape runs (on such a
    # device); K=173 with ~30% unused spans several chunks and a ragged tail
    torch = torch_mod()
    from sparse_top_latent_amd import api
    w = wl.make_random(300 + S, 4, 20, 64, 512, 300, 173, p_unused=0.3)
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        q, kv, _, idx = to_dev(w)
        assert api.plan_kernel(q, kv, idx, S) == "attn_fwd_kernel<512,4,1,false>"
    check(ref, w, S, what=f"64-head workgroups S={S}")


# The split counts the planner gives the benchmark shapes on a 256-CU device
# (H=64, D=512; the planner reads only B, T, H and K): the counts the split
# sweeps measured fastest.  Other devices skip.
@pytest.mark.parametrize("B,T,K,expected", [
    (64, 1, 640, 4),     # decode
    (32, 1, 640, 4),     # long context
    (64, 1, 128, 1),     # sliding window only (head split)
    (64, 1, 384, 1),     # short decode lists (head split)
    (64, 1, 512, 1),     # the longest lists the head split takes
    (256, 1, 640, 1),    # ragged batch
    (1, 4096, 640, 1),   # prefill
    (1, 1, 640, 4),      # a single query: more splits cost more in the combine
    (1, 1, 128, 1),      # a single short query
    (8, 1, 32, 1),       # shorter than two chunks
])
def test_planned_split_counts(B, T, K, expected):
    import ctypes
    torch = torch_mod()
    from sparse_top_latent_amd import _lib
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("split counts pinned for a 256-CU device")
    d = _lib.SaDims(B, T, 64, 512, 8320, K)
    assert _lib.lib().sparse_attn_plan_splits(ctypes.byref(d)) == expected


def test_many_query_splits_stress_and_long_lists(ref):
    T = many_query_T()
    w = wl.make_random(210, 2, T, 64, 512, 120, 40, p_unused=0.2)
    check(ref, w, 2, what="many-query S=2")
    q8 = wl.to_bf16_bits(wl.bf16_bits_to_f32(w.q) * 8.0)
    check(ref, w, 0, q_bits=q8, what="many-query 8x query")
    check(ref, w, 0, sink=np.full(64, 30.0), what="many-query sink=30")
    got = run_gpu(w, 0, np.full(w.idxs.shape, -1, np.int32))
    assert np.all(got == 0)
    got0 = run_gpu(w, 0, np.zeros((2, T, 0), np.int32))
    assert np.all(got0 == 0)
    # the longest supported list (2048 entries, compacted in place), mostly unused
    wl2 = wl.make_random(211, 1, 2 * T, 64, 512, 2100, 2048, p_unused=0.97)
    check(ref, wl2, 0, what="many-query K=2048")


# ------------------------------------------------- head-split path (one split, short lists)
# Unsplit launches at D=512 with K <= 512 whose (query, 16 heads) units all fit
# the compute units at once run the head-split kernel; every case here is
# such a launch (a few queries), checked against the oracle.

HS = "attn_fwd_hs_kernel<512,false>"


def plan_name(B, T, H, D, K, S, N=8320):
    import ctypes
    from sparse_top_latent_amd import _lib
    d = _lib.SaDims(B, T, H, D, N, K)
    return _lib.lib().sparse_attn_plan_kernel(ctypes.byref(d), S).decode()


def test_head_split_dispatch():
    import ctypes
    torch = torch_mod()
    from sparse_top_latent_amd import _lib
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert plan_name(4, 1, 64, 512, 128, 0) == HS
    assert plan_name(4, 1, 64, 512, 512, 1) == HS
    assert plan_name(4, 1, 64, 512, 513, 1) != HS      # longer lists: deep-gather kernel
    assert plan_name(4, 1, 64, 512, 128, 2) != HS      # explicit splits
    assert plan_name(4, 1, 64, 256, 128, 0) != HS      # D = 256
    assert plan_name(cus // 4, 1, 64, 512, 128, 1) == HS
    assert plan_name(cus // 4 + 1, 1, 64, 512, 128, 1) != HS   # 4 units per query overflow
    assert plan_name(3, 2, 40, 512, 200, 0) == HS      # 3 head groups, the last one partial
    d = _lib.SaDims(4, 1, 64, 512, 8320, 384)
    assert _lib.lib().sparse_attn_plan_splits(ctypes.byref(d)) == 1


@pytest.mark.parametrize("K", [1, 16, 47, 48, 49, 96, 143, 144, 145, 200, 448, 512])
def test_head_split_round_boundaries(ref, K):
    # lists around one 48-entry round and three rounds (the LDS buffers' reuse)
    w = wl.make_random(400 + K, 2, 2, 64, 512, 600, K, p_unused=0.0)
    assert plan_name(2, 2, 64, 512, K, 1, N=600) == HS
    check(ref, w, 1, what=f"head split K={K}")


@pytest.mark.parametrize("H", [8, 16, 17, 33])
def test_head_split_head_counts(ref, H):
    # a head tile half empty (8), exactly one (16), one head over a tile (17:
    # a second group with 15 heads beyond H), three groups (33)
    w = wl.make_random(420 + H, 2, 3, H, 512, 260, 150, p_unused=0.2)
    assert plan_name(2, 3, H, 512, 150, 0, N=260) == HS
    check(ref, w, 0, what=f"head split H={H}")


def test_head_split_partial_head_group_unused_and_repeats(ref):
    # H=40: the last head group holds 8 heads beyond H; ~30% unused entries,
    # repeats, and entries beyond N skipped; planned and explicit one split
    w = wl.make_random(410, 3, 2, 40, 512, 300, 200, p_unused=0.3, allow_repeats=True)
    bad = w.idxs.copy()
    bad[0, 0, 3] = w.N
    bad[2, 1, 100] = w.N + 7
    clean = np.where(bad >= w.N, -1, bad).astype(np.int32)
    got = run_gpu(w, 0, bad)
    assert_close(got, ref(w.q, w.kv_host(), w.sink, clean, w.scale), "head split H=40")
    check(ref, w, 1, sink=None, what="head split H=40 no sink")


def test_head_split_rising_scores(ref):
    # every list holds all 400 rows in ascending order; row r has r/400 in
    # dim 0 and every q has 315 there, so the scores rise by ~20 log2 units
    # along the list (the rest of each score stays ~N(0, 1)): each head's max
    # keeps rising from round to round and within rounds, the reference moves
    # and blocks go through the scaled path, while the outputs stay O(1)
    import copy
    w = copy.deepcopy(wl.make_random(411, 2, 2, 64, 512, 400, 400, p_unused=0.0))
    w.idxs = np.sort(w.idxs, axis=-1).astype(np.int32)
    for b in range(w.B):
        w.vals[b] = w.vals[b].copy()
        w.vals[b][:, 0] = wl.to_bf16_bits((w.rows[b] / 400.0).astype(np.float32))
    q = w.q.copy()
    q[..., 0] = wl.to_bf16_bits(np.float32(315.0))
    check(ref, w, 1, q_bits=q, what="head split rising scores")
    check(ref, w, 0, q_bits=q, sink=np.full(64, 25.0), what="head split rising scores, sink 25")
    check(ref, w, 3, q_bits=q, what="deep gather S=3, rising scores")


def test_head_split_fp4_rows_decode_batch():
    # 64 queries, 128-entry window + 256 compressed entries, FP4 compressed
    # rows: bit for bit the bf16 two-source result, both on the head split
    torch = torch_mod()
    w = wl.make_random(412, 64, 1, 64, 512, 640, 384, p_unused=0.1)
    if torch.cuda.get_device_properties(0).multi_processor_count >= 256:
        assert plan_name(64, 1, 64, 512, 384, 0, N=640) == HS
    check_fp4(w, 128, 0, "head split fp4 64 queries")


def test_head_split_deterministic_and_close_to_deep_gather(ref):
    w = wl.make_random(413, 4, 2, 64, 512, 600, 300, p_unused=0.2)
    runs = [run_gpu(w, 1) for _ in range(3)]
    assert np.array_equal(runs[0], runs[1]) and np.array_equal(runs[0], runs[2])
    split = run_gpu(w, 3)   # the deep-gather kernel with partials
    exp = ref(w.q, w.kv_host(), w.sink, w.idxs, w.scale)
    assert_close(runs[0], exp, "head split")
    assert_close(split, exp, "deep gather S=3")
    assert np.abs(runs[0] - split).max() <= 2 * MAX_ABS


# ------------------------------------------------- two-source rows (window + compressed)

def split_sources(w, W, spare=(3, 5)):
    """The workload's rows as two buffers with NaN spare rows: window rows
    [0, W) and compressed rows [W, N) (host bits and device tensors)."""
    torch = torch_mod()
    kvh = w.kv_host()
    nan = np.uint16(0x7FC0)
    win_h = np.full((w.B, W + spare[0], w.D), nan, np.uint16)
    cmp_h = np.full((w.B, w.N - W + spare[1], w.D), nan, np.uint16)
    win_h[:, :W] = kvh[:, :W]
    cmp_h[:, :w.N - W] = kvh[:, W:]
    dev = lambda a: torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return win_h, cmp_h, dev(win_h), dev(cmp_h)


def check_two_source(ref2, w, W, S, what):
    torch = torch_mod()
    from sparse_top_latent_amd import api
    q, kv, sk, idx = to_dev(w)
    win_h, cmp_h, win, cmp_ = split_sources(w, W)
    one = api.sparse_attn(q, kv, sk, idx, w.scale, num_splits=S)
    two = api.sparse_attn_2src(q, win, cmp_, W, w.N, sk, idx, w.scale, num_splits=S)
    torch.cuda.synchronize()
    # the same rows in the same order: bit for bit the one-buffer result
    assert torch.equal(one.view(torch.int16), two.view(torch.int16)), f"{what}: differs from one buffer"
    got = wl.bf16_bits_to_f32(two.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
    exp = ref2(w.q, win_h, cmp_h, W, w.N, w.sink, w.idxs, w.scale)
    assert_close(got, exp, what)


@pytest.fixture(scope="module")
def ref2():
    import oracle
    oracle.build(force=False)
    return oracle.sparse_attn_2src_ref


@pytest.mark.parametrize("W", [0, 128, 300])
@pytest.mark.parametrize("S", [1, 3])
def test_two_source_rows(ref2, W, S):
    w = wl.make_random(220, 2, 3, 64, 512, 300, 173, p_unused=0.3)
    check_two_source(ref2, w, W, S, f"two-source W={W} S={S}")


def test_two_source_many_query_path(ref2):
    w = wl.make_random(221, 2, many_query_T(), 64, 512, 160, 75, p_unused=0.3)
    check_two_source(ref2, w, 40, 0, "two-source many-query W=40")


def test_two_source_full_decode():
    # the decode shape as the model holds it: a 128-row window ring and the
    # compressed cache; bit for bit the one-buffer result on every query
    torch = torch_mod()
    from sparse_top_latent_amd import api
    w = wl.make("decode")
    q, kv, sk, idx = to_dev(w)
    win = kv[:, :128].contiguous()
    cmp_ = torch.full((w.B, w.N - 128 + 64, w.D), float("nan"), dtype=torch.bfloat16, device="cuda")
    cmp_[:, :w.N - 128] = kv[:, 128:]
    one = api.sparse_attn(q, kv, sk, idx, w.scale)
    two = api.sparse_attn_2src(q, win, cmp_, 128, w.N, sk, idx, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(one.view(torch.int16), two.view(torch.int16))


# ------------------------------------------------- FP4 compressed rows (E2M1 + E4M3 group scales)

def fp4_records_for(w, W, spare=2):
    """Packed FP4 records for the compressed rows [W, N) of workload w (plus
    spare rows); rows no list references get NaN scale codes, so a stray read
    shows in the output."""
    from sparse_top_latent_amd import api
    R = api.fp4_record_bytes(w.D)
    rec = wl.make_fp4_records(w.seed, w.B, w.N - W + spare, w.D, R)
    D16 = w.D // 16
    for b in range(w.B):
        used = np.unique(w.idxs[b][w.idxs[b] >= W]) - W
        poison = np.ones(rec.shape[1], bool)
        poison[used] = False
        rec[b, poison, w.D // 2:w.D // 2 + D16] = 0x7F
    return rec


def check_fp4(w, W, S, what):
    torch = torch_mod()
    import oracle
    from sparse_top_latent_amd import api
    oracle.build(force=False)
    q, kv, sk, idx = to_dev(w)
    win_h, _, win, _ = split_sources(w, W)
    rec_h = fp4_records_for(w, W)
    rec = torch.from_numpy(rec_h).cuda()
    got_t = api.sparse_attn_2src_fp4(q, win, rec, W, w.N, sk, idx, w.scale, num_splits=S)
    # the same rows decoded (by the oracle's decoder) and given as bf16
    cmp_bits = oracle._f64_to_bf16_bits_exact(oracle.fp4_records_to_rows(rec_h, w.D))
    cmp_t = torch.from_numpy(cmp_bits.view(np.int16)).cuda().view(torch.bfloat16)
    bf = api.sparse_attn_2src(q, win, cmp_t, W, w.N, sk, idx, w.scale, num_splits=S)
    torch.cuda.synchronize()
    assert torch.equal(got_t.view(torch.int16), bf.view(torch.int16)), f"{what}: differs from bf16 rows"
    got = wl.bf16_bits_to_f32(got_t.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
    exp = oracle.sparse_attn_2src_fp4_ref(w.q, win_h, rec_h, W, w.N, w.sink, w.idxs, w.scale)
    assert_close(got, exp, what)


@pytest.mark.parametrize("W,S", [(128, 1), (128, 3), (0, 2), (300, 1)])
def test_fp4_compressed_rows(W, S):
    w = wl.make_random(230, 2, 3, 64, 512, 300, 173, p_unused=0.3)
    check_fp4(w, W, S, f"fp4 W={W} S={S}")


@pytest.mark.parametrize("H,D", [(16, 128), (32, 256)])
def test_fp4_other_head_dims(H, D):
    w = wl.make_random(231 + D, 2, 2, H, D, 200, 90, p_unused=0.2)
    check_fp4(w, 64, 1, f"fp4 H={H} D={D}")


def test_fp4_many_query_path():
    w = wl.make_random(233, 2, many_query_T(), 64, 512, 160, 75, p_unused=0.3)
    check_fp4(w, 40, 0, "fp4 many-query")


def test_fp4_full_decode():
    # decode shape: 128-row bf16 window ring + FP4 compressed cache; every query
    # bit for bit the bf16 two-source result on the decoded rows
    torch = torch_mod()
    import oracle
    from sparse_top_latent_amd import api
    w = wl.make("decode")
    q, kv, sk, idx = to_dev(w)
    win = kv[:, :128].contiguous()
    R = api.fp4_record_bytes(w.D)
    rec_h = wl.make_fp4_records(w.seed, w.B, w.N - 128, w.D, R)
    rec = torch.from_numpy(rec_h).cuda()
    cmp_bits = oracle._f64_to_bf16_bits_exact(oracle.fp4_records_to_rows(rec_h, w.D))
    cmp_t = torch.from_numpy(cmp_bits.view(np.int16)).cuda().view(torch.bfloat16)
    a = api.sparse_attn_2src_fp4(q, win, rec, 128, w.N, sk, idx, w.scale)
    b = api.sparse_attn_2src(q, win, cmp_t, 128, w.N, sk, idx, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


# ------------------------------------------ the output's inverse rotary step, fused

def run_rope(w, freqs, rd, S=0):
    """(fused rope output, plain sparse_attn output) as bf16 bit patterns."""
    torch = torch_mod()
    from sparse_top_latent_amd import api
    q, kv, sk, idx = to_dev(w)
    f = None if freqs is None else torch.from_numpy(freqs).cuda()
    out = api.sparse_attn_rope(q, kv, sk, idx, w.scale, f, rd, num_splits=S)
    plain = api.sparse_attn(q, kv, sk, idx, w.scale, num_splits=S)
    torch.cuda.synchronize()
    return (out.view(torch.int16).cpu().numpy().view(np.uint16),
            plain.view(torch.int16).cpu().numpy().view(np.uint16))


def check_rope(w, rd, S, what):
    import oracle
    freqs = wl.make_freqs(w.seed, w.T, rd)
    bits, pbits = run_rope(w, freqs, rd, S)
    # the dims before the rotary part are sparse_attn's, bit for bit
    assert np.array_equal(bits[..., :w.D - rd], pbits[..., :w.D - rd]), what
    got = wl.bf16_bits_to_f32(bits).astype(np.float64)
    exp = oracle.sparse_attn_rope_ref(w.q, w.kv_host(), w.sink, w.idxs, w.scale, freqs, rd)
    assert_close(got, exp, what)


@pytest.mark.parametrize("H,D,rd,S", [(8, 128, 32, 1), (8, 128, 32, 3), (16, 256, 8, 2),
                                      (64, 512, 64, 1), (64, 512, 64, 4), (4, 128, 128, 1)])
def test_rope_fused(H, D, rd, S):
    w = wl.make_random(250 + D + S, 2, 5, H, D, 300, 96)
    check_rope(w, rd, S, f"rope H={H} D={D} rd={rd} S={S}")


def test_rope_many_query_path():
    w = wl.make_random(260, 2, many_query_T(), 64, 512, 160, 75, p_unused=0.3)
    for S in (1, 2):
        check_rope(w, 64, S, f"rope many-query S={S}")


def test_rope_zero_is_plain():
    w = wl.make_random(261, 2, 3, 16, 256, 200, 64)
    for S in (1, 3):
        bits, pbits = run_rope(w, None, 0, S)
        assert np.array_equal(bits, pbits)


def test_rope_full_decode(ref):
    import oracle
    w = wl.make("decode")
    freqs = wl.make_freqs(w.seed, w.T, 64)
    bits, pbits = run_rope(w, freqs, 64, 0)
    assert np.array_equal(bits[..., :w.D - 64], pbits[..., :w.D - 64])
    got = wl.bf16_bits_to_f32(bits).astype(np.float64)
    exps = []
    for b in range(w.B):
        q1, kv1, i1 = w.query_slice(b, 0)
        exps.append(oracle.sparse_attn_rope_ref(q1, kv1, w.sink, i1, w.scale, freqs, 64)[0, 0])
    assert_close(got[:, 0], np.stack(exps), "rope decode every query")


# ------------------------------------------------- top-k selection (the lists' compressed segment)

@pytest.fixture(scope="module")
def topk_ref():
    import oracle
    return oracle.topk_ref


def test_topk_decode_shape_in_place(topk_ref):
    # 64 queries x 8192 compressed scores -> 512 positions + 128 (the window),
    # written straight into the compressed segment of [64, 1, 640] lists
    torch = torch_mod()
    from sparse_top_latent_amd import api
    rng = np.random.default_rng(40)
    sc = rng.standard_normal((64, 1, 8192), dtype=np.float32)
    lists = torch.full((64, 1, 640), 7, dtype=torch.int32, device="cuda")
    api.topk(torch.from_numpy(sc).cuda(), 512, 128, out=lists[..., 128:])
    torch.cuda.synchronize()
    got = lists.cpu().numpy()
    assert np.all(got[..., :128] == 7)                       # the window segment untouched
    assert np.array_equal(got[:, 0, 128:], topk_ref(sc[:, 0], None, 512, 128))


def test_topk_ties_and_special_values(topk_ref):
    torch = torch_mod()
    from sparse_top_latent_amd import api
    rng = np.random.default_rng(41)
    sc = rng.integers(-3, 4, (50, 3000)).astype(np.float32)   # heavy ties
    sc[rng.random(sc.shape) < 0.05] = np.nan
    sc[rng.random(sc.shape) < 0.05] = -0.0
    sc[rng.random(sc.shape) < 0.02] = np.inf
    sc[rng.random(sc.shape) < 0.02] = -np.inf
    got = api.topk(torch.from_numpy(sc).cuda(), 700, 5).cpu().numpy()
    assert np.array_equal(got, topk_ref(sc, None, 700, 5))


def test_topk_causal_visible_counts(topk_ref):
    # prefill shape: query t sees floor((t+1)/2) of 2048 compressed positions
    torch = torch_mod()
    from sparse_top_latent_amd import api
    rng = np.random.default_rng(42)
    T = 4096
    sc = rng.standard_normal((T, 2048), dtype=np.float32)
    lens = ((np.arange(T) + 1) // 2).astype(np.int32)
    got = api.topk(torch.from_numpy(sc).cuda(), 512, 4096,
                   lens=torch.from_numpy(lens).cuda()).cpu().numpy()
    assert np.array_equal(got, topk_ref(sc, lens, 512, 4096))


def test_topk_long_rows_and_edges(topk_ref):
    torch = torch_mod()
    from sparse_top_latent_amd import api
    rng = np.random.default_rng(43)
    sc = rng.standard_normal((8, 65536), dtype=np.float32)       # rows re-read from memory
    got = api.topk(torch.from_numpy(sc).cuda(), 512, 128).cpu().numpy()
    assert np.array_equal(got, topk_ref(sc, None, 512, 128))
    # every workgroup shape: odd row lengths (scalar loads), visible counts
    # cut mid-thread, and rows past the register limit with counts
    for Qk, Ck, kk in ((6, 12001, 512), (4, 16384, 2048), (7, 4093, 300), (3, 20000, 512)):
        sc = rng.standard_normal((Qk, Ck), dtype=np.float32)
        lens = rng.integers(0, Ck + 1, Qk).astype(np.int32)
        lens[0] = Ck
        got = api.topk(torch.from_numpy(sc).cuda(), kk, 0,
                       lens=torch.from_numpy(lens).cuda()).cpu().numpy()
        assert np.array_equal(got, topk_ref(sc, lens, kk, 0)), (Qk, Ck, kk)
    small = rng.standard_normal((5, 37), dtype=np.float32)
    for k in (0, 1, 36, 37, 60):
        g = api.topk(torch.from_numpy(small).cuda(), k, 0).cpu().numpy()
        assert np.array_equal(g, topk_ref(small, None, k, 0)), k


def test_topk_feeds_attention(ref, topk_ref):
    # end to end: scores -> compressed segment of the lists -> sparse_attn
    torch = torch_mod()
    from sparse_top_latent_amd import api
    rng = np.random.default_rng(44)
    B, W, C, H, D = 4, 128, 1024, 64, 512
    base = wl.make_random(240, B, 1, H, D, W + C, 256, p_unused=0.0)
    sc = rng.standard_normal((B, 1, C), dtype=np.float32)
    lists = np.full((B, 1, W + 256), -1, np.int32)
    lists[..., :W] = np.arange(W)
    lists_t = torch.from_numpy(lists).cuda()
    api.topk(torch.from_numpy(sc).cuda(), 256, W, out=lists_t[..., W:])
    exp_lists = lists.copy()
    exp_lists[:, 0, W:] = topk_ref(sc[:, 0], None, 256, W)
    torch.cuda.synchronize()
    assert np.array_equal(lists_t.cpu().numpy(), exp_lists)
    q, kv, sk, _ = to_dev(base)
    # dense random rows for every position (the base workload stores only its own rows)
    rows = torch.from_numpy(np.random.default_rng(45).standard_normal((B, W + C, D), dtype=np.float32))
    kv_bits = wl.to_bf16_bits(rows.numpy())
    kv_t = torch.from_numpy(kv_bits.view(np.int16)).cuda().view(torch.bfloat16)
    out = api.sparse_attn(q, kv_t, sk, lists_t, base.scale)
    torch.cuda.synchronize()
    got = wl.bf16_bits_to_f32(out.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
    exp = ref(base.q, kv_bits, base.sink, exp_lists, base.scale)
    assert_close(got, exp, "top-k lists into sparse_attn")


# --------------------------------------------------------- full-size workloads
# Same launch configuration as bench.py: num_splits=0 (planned by the library).

def sampled_check(ref, w, queries, got):
    """Oracle on the listed queries one by one; same bar as assert_close."""
    exps = []
    for (b, t) in queries:
        q1, kv1, i1 = w.query_slice(b, t)
        exps.append(ref(q1, kv1, w.sink, i1, w.scale)[0, 0])
    exp = np.stack(exps)
    sub = np.stack([got[b, t] for (b, t) in queries])
    assert_close(sub, exp, f"{w.name} sampled {len(queries)}")


@pytest.mark.parametrize("name", ["decode", "long", "window"])
def test_full_config_every_query(ref, name):
    w = wl.make(name)
    got = run_gpu(w, 0)
    exp = ref(w.q, w.kv_host(), w.sink, w.idxs, w.scale) if name == "window" else None
    if exp is not None:
        assert_close(got, exp, name)
    else:
        sampled_check(ref, w, [(b, 0) for b in range(w.B)], got)


def compact_rows(w):
    """Each sequence's stored rows as a compact kv [B, R, D] (R = the most rows
    any sequence stores) and its lists remapped onto them by position among the
    sorted stored rows.  Exact plumbing, no arithmetic: it keeps the 8.6 GB
    dense key-value tensor of the ragged batch out of host memory."""
    R = max(len(r) for r in w.rows)
    kv = np.full((w.B, R, w.D), wl.BF16_NAN, np.uint16)
    idx = np.full_like(w.idxs, -1)
    for b in range(w.B):
        kv[b, :len(w.rows[b])] = w.vals[b]
        m = w.idxs[b] >= 0
        idx[b][m] = np.searchsorted(w.rows[b], w.idxs[b][m])
    return kv, idx


def test_full_prefill_every_query(ref):
    """All 4096 prefill queries (the many-query kernel at its real launch
    shape, every unit and the spare workgroups of the last XCD turn) against
    the oracle, element by element."""
    w = wl.make("prefill")
    got = run_gpu(w, 0)
    exp = ref(w.q, w.kv_host(), w.sink, w.idxs, w.scale)
    assert_close(got, exp, "prefill, every query")


@pytest.mark.parametrize("S", [0, 2])
def test_full_ragged_every_query(ref, S):
    """All 256 ragged-batch queries against the oracle, in the planned launch
    (one split) and with two split slots per query, where each query's own
    valid count decides how many it uses."""
    w = wl.make("ragged")
    got = run_gpu(w, S)
    kvc, idc = compact_rows(w)
    exp = ref(w.q, kvc, w.sink, idc, w.scale)
    assert_close(got, exp, f"ragged S={S}, every query")


@pytest.mark.parametrize("S", [3, 4, 8])
def test_per_query_split_plan(ref, S):
    """Lists of very different valid counts in one launch: each query cuts its
    own valid entries into ceil(n S / K) ranges (spare split slots idle, the
    combine merges only the ranges used), including empty and one-entry lists."""
    w = wl.make_decode(B=10)
    lst = w.idxs.copy()
    for b, n in enumerate([0, 1, 31, 64, 100, 161, 320, 500, 639, 640]):
        keep = np.zeros(w.K, bool)
        keep[np.random.default_rng(b).choice(w.K, n, replace=False)] = True
        lst[b, 0][~keep] = -1
    check(ref, w, S, idxs=lst, what=f"per-query plan S={S}")


def test_full_decode_with_unused_entries_in_every_slice(ref):
    """The decode batch with unused (-1) and out-of-range (>= N) entries spread
    through every split's slice, in the launch configuration bench.py times:
    the rows a fully valid list would put in each split's first chunk are
    requested before the list is compacted and then corrected, so the result
    must equal the oracle on the cleaned lists (out-of-range entries skipped)."""
    w = wl.make("decode")
    rng = np.random.default_rng(5)
    lst = w.idxs.copy()
    lst[rng.random(lst.shape) < 0.15] = -1
    lst[rng.random(lst.shape) < 0.02] = w.N + 7
    got = run_gpu(w, 0, idxs=lst)
    clean = np.where(lst >= w.N, -1, lst).astype(np.int32)
    exps = []
    for b in range(w.B):
        q1, kv1, _ = w.query_slice(b, 0)
        exps.append(ref(q1, kv1, w.sink, clean[b:b + 1, 0:1], w.scale)[0, 0])
    assert_close(got[:, 0], np.stack(exps), "decode with unused and out-of-range entries")
