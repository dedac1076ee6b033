#!/usr/bin/env python3
"""Throughput of the sparse latent attention step on one MI355X.

Headline workload: the DeepSeek-V4.1 decode batch (B=64 sequences, one query
each, H=64 heads of width 512, K=640 list entries = 128 window rows + 512
distinct compressed rows out of 8192, scale 512^-0.5), synthetic and seeded.
The same JSON line also carries the other configurations (causal prefill of
4096 queries, long-context decode, the ragged batch and window-only lists)
under ``workloads``, each timed the same way.

A step is one pass of the whole path over the batch: index decode, gather,
QK^T, sink softmax, PV and (with splits) the log-sum-exp combine.  Inputs are
resident in HBM before timing; the timed steps cycle through ``--rotate``
copies of q/kv/idxs at distinct addresses so that the rows a step gathers are
not still sitting in the 256 MB Infinity Cache from the previous step (a
second, labelled figure runs with one copy).  The timed steps are launched
back to back on one stream while the GPU first runs a short sleep kernel, so
that the host has queued them all before the first one starts and host launch
cost is not part of the time; the same steps replayed from a captured HIP
graph are reported beside them (``graph_replay``: on ROCm a graph adds time
between its kernel nodes).

Prints one JSON line.  ``value`` = queries per second of the headline workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0         # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCE = os.path.join(ROOT, "sparse_top_latent_amd", "csrc", "sparse_attn.hip")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--rotate", type=int, default=8, help="input copies cycled by the steps")
    ap.add_argument("--workload", default="decode",
                    help="decode (the benchmark line) or another generator name")
    ap.add_argument("--splits", type=int, default=0, help="0 = planned by the library")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--two-source", action="store_true",
                    help="also time the step with the window and compressed rows in two "
                         "buffers (sparse_attn_fwd_2src) and the concatenation it avoids")
    ap.add_argument("--kv-format", default="bf16", choices=["bf16", "fp4"],
                    help="fp4: also time the step with the compressed rows packed as FP4 "
                         "records (E2M1 codes, one E4M3 scale per 16) beside bf16 window rows")
    ap.add_argument("--rope", action="store_true",
                    help="also time the step with the output's inverse rotary step fused "
                         "(sparse_attn_fwd_rope, rd=64) against sparse_attn + a torch rotation")
    ap.add_argument("--topk", action="store_true",
                    help="also time the top-k selection that fills the lists' compressed "
                         "segment (decode and causal prefill shapes) and decode top-k + attention")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run plain 256 MiB copies first (HBM counter calibration)")
    ap.add_argument("--no-workloads", action="store_true",
                    help="time only the headline workload (profiling runs)")
    ap.add_argument("--list-sweep", action="store_true",
                    help="also time decode batches (64 queries, 64 heads) with lists of "
                         "128..640 entries: the planned kernel against the deep-gather "
                         "kernel at its best of 2-4 splits")
    return ap.parse_args()


OTHER_WORKLOADS = ("prefill", "long", "ragged", "window")


def source_digest():
    import hashlib
    return hashlib.sha256(open(KERNEL_SOURCE, "rb").read()).hexdigest()[:16]


def _read_kv(path):
    """key: value lines of a committed counter summary, or None when it is
    missing or was taken on another kernel source."""
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256_16") != source_digest():
        return None
    return kv


def read_counters(workload):
    """HBM bytes per launch of the dominant kernel from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary of this workload."""
    kv = _read_kv(os.path.join(PROFILES, f"attn_fwd_{workload}_counters.txt"))
    try:
        return None if kv is None else float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def read_mfma_busy(workload):
    """MFMA busy share per SIMD of the dominant kernel from the committed
    rocprofv3 SQ counter summary of this workload: SQ_VALU_MFMA_BUSY_CYCLES /
    (4 SIMDs x SQ_BUSY_CU_CYCLES), with the clock those counters imply."""
    kv = _read_kv(os.path.join(PROFILES, f"attn_fwd_{workload}_sq_counters.txt"))
    try:
        if kv is None:
            return None
        return {"mfma_busy_per_simd": float(kv["mfma_busy_per_simd"]),
                "clock_ghz": float(kv["clock_ghz"]),
                "source": f"profiles/attn_fwd_{workload}_sq_counters.txt"}
    except (KeyError, ValueError):
        return None


def gate(torch, ms=20.0):
    """Keep the GPU busy for a moment so the host can queue the timed work."""
    torch.cuda._sleep(int(ms * 1e-3 * 2.1e9))


def gate_ms(calls):
    """A sleep long enough for the host to queue `calls` calls (each well under
    0.5 ms of host time, a few binding or torch launches)."""
    return max(20.0, 0.5 * calls)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from sparse_top_latent_amd import api, workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    cap_stream = torch.cuda.Stream()

    def measure(w, R, warm_cache):
        """Time one workload: ms per step (back-to-back launches cycling
        through R input copies; also replayed from a graph of R steps),
        optionally with one copy (warm cache), and the dominant kernel alone
        on the stream it runs on.  Returns the figures and the device inputs."""
        q0 = torch.from_numpy(w.q.view(np.int16)).to(dev).view(torch.bfloat16)
        kv0 = w.kv_device(dev)
        idx0 = torch.from_numpy(w.idxs).to(dev)
        sink = torch.from_numpy(w.sink).to(dev)
        qs = [q0] + [q0.clone() for _ in range(R - 1)]
        kvs = [kv0] + [kv0.clone() for _ in range(R - 1)]
        idxs = [idx0] + [idx0.clone() for _ in range(R - 1)]
        out = torch.empty_like(q0)
        S = args.splits if args.splits > 0 else api.plan_splits(q0, kv0, idx0)
        kernel = api.plan_kernel(q0, kv0, idx0, S)
        ws_bytes = api.workspace_bytes(q0, kv0, idx0, S)
        ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)

        def step(i):
            api.sparse_attn(qs[i], kvs[i], sink, idxs[i], w.scale, out=out, num_splits=S,
                            workspace=ws)

        # Warm up eagerly (also checks that the path runs), then capture
        # graphs: one holding R consecutive steps (one per input copy, as a
        # model's decode graph would chain them) and one graph per single step
        # for a remainder.
        for i in range(max(1, args.warmup)):
            step(i % R)
        torch.cuda.synchronize()

        def capture(copies):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap_stream):
                for i in copies:
                    step(i)
            return g

        g_rot = capture(range(R))
        g_one = [capture([i]) for i in range(R)]
        g_warm = capture([0] * R) if warm_cache else None
        for g in [g_rot] + g_one + ([g_warm] if g_warm is not None else []):
            g.replay()
        torch.cuda.synchronize()

        def timed(g_many):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            gate(torch)
            e0.record()
            for _ in range(args.steps // R):
                g_many.replay()
            for k in range(args.steps % R):
                g_one[k if g_many is g_rot else 0].replay()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / args.steps

        def timed_eager(rotate):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            gate(torch, gate_ms(args.steps))
            e0.record()
            for k in range(args.steps):
                step(k % R if rotate else 0)
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / args.steps

        ms_step = timed_eager(True)
        ms_step_graph = timed(g_rot)
        ms_step_warm = timed_eager(False) if warm_cache else None

        # the dominant kernel alone: back-to-back launches on the stream it
        # runs on (torch's current stream, where the binding launches)
        stream = torch.cuda.current_stream(dev)
        torch.cuda.synchronize()
        gate(torch)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for k in range(args.steps):
            i = k % R
            if S > 1:
                api.sparse_attn_partial(qs[i], kvs[i], idxs[i], w.scale, S, ws)
            else:
                api.sparse_attn(qs[i], kvs[i], sink, idxs[i], w.scale, out=out, num_splits=1)
        e1.record(stream)
        torch.cuda.synchronize()
        ms_main = e0.elapsed_time(e1) / args.steps

        Qn = w.queries
        valid = w.valid_entries()
        kv_bytes = w.distinct_rows() * w.D * 2
        q_bytes = Qn * w.H * w.D * 2
        idx_bytes = w.idxs.size * 4
        # algorithmic bytes of the dominant kernel: rows, q and lists in; with
        # one split also the bf16 output and the sink (else those belong to
        # the combine)
        main_bytes = (kv_bytes + q_bytes + idx_bytes + (q_bytes if S == 1 else 0)
                      + (w.H * 4 if S == 1 else 0))
        path_bytes = w.algorithmic_bytes()
        flops = w.algorithmic_flops()
        t_step = ms_step * 1e-3
        t_roof = max(path_bytes / (HBM_PEAK_GBPS * 1e9), flops / (MFMA_BF16_PEAK_TFLOPS * 1e12))
        t_main = ms_main * 1e-3
        if flops / (MFMA_BF16_PEAK_TFLOPS * 1e12) > path_bytes / (HBM_PEAK_GBPS * 1e9):
            roof = {"kernel": kernel, "bound": "mfma",
                    "achieved": round(flops / t_main / 1e12, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                    "unit": "TFLOP/s",
                    "frac": round(flops / t_main / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                    "algorithmic_flops_per_launch": flops}
        else:
            roof = {"kernel": kernel, "bound": "hbm",
                    "achieved": round(main_bytes / t_main / 1e9, 1), "peak": HBM_PEAK_GBPS,
                    "unit": "GB/s", "frac": round(main_bytes / t_main / 1e9 / HBM_PEAK_GBPS, 4),
                    "algorithmic_bytes_per_launch": main_bytes}
        roof["traffic"] = read_counters(w.name)
        roof["avg_launch_us"] = round(ms_main * 1e3, 3)
        roof["mfma_busy_counters"] = read_mfma_busy(w.name)
        fig = {
            "ms_per_step": round(ms_step, 5),
            "value": round(Qn / t_step, 1),
            "graph_replay": {"ms_per_step": round(ms_step_graph, 5),
                             "value": round(Qn / (ms_step_graph * 1e-3), 1)},
            "config": {"workload": f"deepseek-v4.1-{w.name}", "B": w.B, "T": w.T, "H": w.H,
                       "D": w.D, "K": w.K, "N": w.N, "valid_entries": valid, "splits": S,
                       "input_copies_rotated": R},
            "gathered_kv_GBps": round(valid * w.D * 2 / t_step / 1e9, 1),
            "path_roofline_frac": round(t_roof / t_step, 4),
            "mfma_util": round(flops / t_step / (MFMA_BF16_PEAK_TFLOPS * 1e12), 4),
            "roofline": roof,
        }
        if ms_step_warm is not None:
            fig["warm_cache"] = {
                "value": round(Qn / (ms_step_warm * 1e-3), 1),
                "ms_per_step": round(ms_step_warm, 5),
                "note": "same inputs every step: rows may be served from the Infinity Cache"}
        state = {"qs": qs, "kvs": kvs, "idxs": idxs, "sink": sink, "out": out, "ws": ws, "S": S,
                 "step": step}
        return fig, state

    w = wl.make(args.workload)
    R = max(1, args.rotate)
    fig, st = measure(w, R, warm_cache=True)
    qs, kvs, idxs, sink, out, ws, S, step = (st[k] for k in ("qs", "kvs", "idxs", "sink", "out",
                                                            "ws", "S", "step"))
    Qn = w.queries
    flops = w.algorithmic_flops()
    if args.copy_probe:
        a = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
    line = {
        "metric": "sparse-attn queries/sec + gathered-KV HBM GB/s (% roofline), H=64 D=512 K=640",
        "value": fig["value"],
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": fig["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": dict(fig["config"], parallelism="single-gpu"),
        "gathered_kv_GBps": fig["gathered_kv_GBps"],
        "path_roofline_frac": fig["path_roofline_frac"],
        "mfma_util": fig["mfma_util"],
        "warm_cache": fig["warm_cache"],
        "graph_replay": fig["graph_replay"],
        "roofline": fig["roofline"],
    }

    def time_calls(fn):
        """ms per call of fn(i), launched back to back over the R copies (as
        the headline step)."""
        for i in range(R):
            fn(i)
        torch.cuda.synchronize()
        n = max(R, args.steps)
        gate(torch, gate_ms(n))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for k in range(n):
            fn(k % R)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    if args.two_source:
        # the rows as the model holds them: window rows and compressed rows in
        # separate buffers; the one-buffer path needs them concatenated first
        W = w.window_rows
        wins = [k[:, :W].contiguous() for k in kvs]
        cmps = [k[:, W:].contiguous() for k in kvs]

        def step2(i):
            api.sparse_attn_2src(qs[i], wins[i], cmps[i], W, w.N, sink, idxs[i], w.scale,
                                 out=out, num_splits=S, workspace=ws)

        def cat(i):
            torch.cat([wins[i], cmps[i]], dim=1)

        ms2 = time_calls(step2)
        ms_cat = time_calls(cat)
        line["two_source"] = {
            "window_rows": W, "ms_per_step": round(ms2, 5), "value": round(Qn / (ms2 * 1e-3), 1),
            "concat_copy_ms": round(ms_cat, 5),
            "note": "rows read in place from the window and compressed buffers; "
                    "concat_copy_ms is the torch.cat the one-buffer call needs first"}

    if args.kv_format == "fp4":
        # window rows bf16, compressed rows as packed FP4 records (the pages'
        # cache format); synthetic records, the same index lists
        W = w.window_rows
        Rb = api.fp4_record_bytes(w.D)
        rec0 = torch.from_numpy(wl.make_fp4_records(w.seed, w.B, w.N - W, w.D, Rb)).to(dev)
        recs = [rec0] + [rec0.clone() for _ in range(R - 1)]
        wins4 = [k[:, :W].contiguous() for k in kvs]

        def step4(i):
            api.sparse_attn_2src_fp4(qs[i], wins4[i], recs[i], W, w.N, sink, idxs[i], w.scale,
                                     out=out, num_splits=S, workspace=ws)

        ms4 = time_calls(step4)
        # algorithmic bytes: distinct window rows x 2D + distinct compressed rows x record
        nwin = sum(int(np.count_nonzero(np.asarray(r) < W)) for r in w.rows)
        ncmp = sum(int(np.count_nonzero(np.asarray(r) >= W)) for r in w.rows)
        b4 = (nwin * w.D * 2 + ncmp * Rb + 2 * Qn * w.H * w.D * 2 + w.idxs.size * 4 + w.H * 4)
        t4 = max(b4 / (HBM_PEAK_GBPS * 1e9), flops / (MFMA_BF16_PEAK_TFLOPS * 1e12))
        line["kv_fp4"] = {
            "ms_per_step": round(ms4, 5), "value": round(Qn / (ms4 * 1e-3), 1),
            "record_bytes": Rb, "algorithmic_bytes": b4,
            "path_roofline_frac": round(t4 / (ms4 * 1e-3), 4),
            "note": "window rows bf16; compressed rows as FP4 records (E2M1 codes + one E4M3 "
                    "scale per 16 elements), expanded to bf16 in LDS"}


    if args.rope:
        # the output's last 64 dims rotated back (the step right after
        # sparse_attn in the pages' forward), fused into the output rounding,
        # against the unfused pair: sparse_attn, then a float32 complex
        # rotation of o[..., -64:] in torch
        rd = 64
        fr = torch.from_numpy(wl.make_freqs(w.seed, w.T, rd)).to(dev)
        fc = torch.view_as_complex(fr).conj()[None, :, None, :]

        def fused(i):
            api.sparse_attn_rope(qs[i], kvs[i], sink, idxs[i], w.scale, fr, rd, out=out,
                                 num_splits=S, workspace=ws)

        def unfused(i):
            step(i)
            x = out[..., -rd:].float().reshape(w.B, w.T, w.H, rd // 2, 2)
            y = torch.view_as_real(torch.view_as_complex(x) * fc)
            out[..., -rd:] = y.reshape(w.B, w.T, w.H, rd).to(torch.bfloat16)

        ms_f = time_calls(fused)
        ms_u = time_calls(unfused)
        line["rope"] = {"rd": rd, "ms_per_step": round(ms_f, 5),
                        "value": round(Qn / (ms_f * 1e-3), 1),
                        "unfused_ms_per_step": round(ms_u, 5),
                        "note": "inverse rotation of o[..., -64:] inside the output rounding "
                                "(combine or epilogue) against sparse_attn + torch rotation"}

    if args.topk:
        # the compressed segment of the lists from indexer scores: the decode
        # batch (64 queries x 8192 compressed positions -> 512, written after
        # the window entries) and the causal prefill shape (4096 queries, query
        # t sees (t+1)//2 of 2048 positions), then decode top-k + attention
        gen = torch.Generator(device=dev)
        gen.manual_seed(7)
        TOPK = 512
        res = {}
        for name, Qk, Ck, causal in (("decode", w.B * w.T, 8192, False),
                                      ("prefill", 4096, 2048, True)):
            scs = [torch.randn(Qk, Ck, generator=gen, device=dev) for _ in range(R)]
            lens = (torch.arange(1, Qk + 1, device=dev, dtype=torch.int32) // 2) if causal else None
            outk = torch.empty(Qk, TOPK, dtype=torch.int32, device=dev)
            ms_k = time_calls(lambda i: api.topk(scs[i], TOPK, 128, lens=lens, out=outk))
            nbytes = Qk * Ck * 4 + Qk * TOPK * 4 + (Qk * 4 if causal else 0)
            res[name] = {"queries": Qk, "candidates": Ck, "k": TOPK, "ms": round(ms_k, 5),
                         "GBps": round(nbytes / (ms_k * 1e-3) / 1e9, 1),
                         "hbm_frac": round(nbytes / (ms_k * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
        if w.T == 1 and w.K >= 128 + TOPK:
            scd = [torch.randn(w.B, 8192, generator=gen, device=dev) for _ in range(R)]
            lists = [x.clone() for x in idxs]

            def step_k(i):
                api.topk(scd[i], TOPK, 128, out=lists[i][:, 0, 128:128 + TOPK])
                api.sparse_attn(qs[i], kvs[i], sink, lists[i], w.scale, out=out, num_splits=S,
                                workspace=ws)

            # the rows picked here are random positions of kv, so the step
            # gathers the same number of rows as the benchmark step
            ms_kd = time_calls(step_k)
            res["decode_with_attention"] = {"ms_per_step": round(ms_kd, 5),
                                            "value": round(Qn / (ms_kd * 1e-3), 1)}
        line["topk"] = res

    if not args.no_workloads and args.workload == "decode":
        # the other configurations, each timed like the headline (a step =
        # the whole path over its batch); kernels and rooflines per workload
        res = {}
        for name in OTHER_WORKLOADS:
            wo = wl.make(name)
            fo, so = measure(wo, R, warm_cache=False)
            res[name] = {k: fo[k] for k in ("value", "ms_per_step", "graph_replay", "gathered_kv_GBps",
                                             "path_roofline_frac", "mfma_util", "roofline")}
            res[name]["unit"] = "queries/s"
            res[name]["config"] = fo["config"]
            del so, fo, wo
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
        line["workloads"] = res

    if args.list_sweep:
        # where the head-split kernel takes over: K-entry lists (all valid), and
        # 640-entry lists with about 160 or 320 valid entries
        sweep = []
        cases = [(K, 0.0) for K in (128, 192, 256, 320, 384, 448, 512, 640)]
        cases += [(640, 1 - 160 / 640), (640, 1 - 320 / 640)]
        keep = args.splits
        for K, pu in cases:
            ws_ = wl.make_random(11, 64, 1, 64, 512, 8320, K, p_unused=pu, scale=512 ** -0.5)
            args.splits = 0
            fp, sp = measure(ws_, R, warm_cache=False)
            best = None
            for S_ in (2, 3, 4):
                args.splits = S_
                fs, ss = measure(ws_, R, warm_cache=False)
                if best is None or fs["ms_per_step"] < best[1]:
                    best = (S_, fs["ms_per_step"])
                del ss
            sweep.append({"K": K, "valid_entries": fp["config"]["valid_entries"],
                          "planned": {"kernel": fp["roofline"]["kernel"],
                                      "splits": fp["config"]["splits"],
                                      "us_per_step": round(fp["ms_per_step"] * 1e3, 2)},
                          "deep_gather_best": {"splits": best[0],
                                               "us_per_step": round(best[1] * 1e3, 2)}})
            del sp
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
        args.splits = keep
        line["list_sweep"] = sweep

    if not args.no_cpu_baseline:
        import ctypes
        import oracle
        kvh = np.stack([w.kv_dense_host(b) for b in range(w.B)])

        def rate(fn, n_per_call, budget):
            done, t0 = 0, time.perf_counter()
            while True:
                fn()
                done += 1
                el = time.perf_counter() - t0
                if el >= budget or done >= 1000:
                    return done * n_per_call / el, done, el

        # all the host cores the process may use (OpenMP over queries)
        v_all, done, el = rate(lambda: oracle.sparse_attn_ref(w.q, kvh, w.sink, w.idxs, w.scale),
                               Qn, 10.0)
        threads = oracle.num_threads()
        # one thread on a fixed subset (the first 8 queries): the per-core rate
        gomp = ctypes.CDLL("libgomp.so.1")
        gomp.omp_set_num_threads(1)
        try:
            v_one, done1, el1 = rate(lambda: oracle.sparse_attn_ref(
                w.q[:8], kvh[:8], w.sink, w.idxs[:8], w.scale), 8, 3.0)
        finally:
            gomp.omp_set_num_threads(threads)
        cpu_model = "unknown"
        try:
            for ln in open("/proc/cpuinfo"):
                if ln.startswith("model name"):
                    cpu_model = ln.split(":", 1)[1].strip()
                    break
        except OSError:
            pass
        line["cpu_baseline"] = {
            "value": round(v_all, 2), "unit": "queries/s",
            "cores": threads, "kind": "oracle",
            "sample": f"the full {w.name} batch ({Qn} queries) computed {done} times "
                      f"by the fp64 oracle, {el:.1f} s wall",
            "cpu_model": cpu_model,
            "affinity_cores": len(os.sched_getaffinity(0)),
            "per_core": {"value": round(v_one, 2), "unit": "queries/s", "threads": 1,
                         "sample": f"queries 0..7 of the {w.name} batch, {done1} times, "
                                   f"{el1:.1f} s wall"}}
        if not args.no_workloads and args.workload == "decode":
            # prefill: a stratified subset (every 64th query t, 64 queries)
            wp = wl.make("prefill")
            ts = np.arange(0, wp.T, 64)
            kvp = wp.kv_host()
            v_p, donep, elp = rate(lambda: oracle.sparse_attn_ref(
                wp.q[:, ts], kvp, wp.sink, wp.idxs[:, ts], wp.scale), len(ts), 3.0)
            line["cpu_baseline"]["prefill"] = {
                "value": round(v_p, 2), "unit": "queries/s", "threads": threads,
                "sample": f"every 64th prefill query ({len(ts)} queries, t = 0, 64, ..., "
                          f"{ts[-1]}), {donep} times, {elp:.1f} s wall"}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
