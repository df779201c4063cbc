#!/usr/bin/env python3
"""Benchmark of the block-quantized decode mat-vec on one MI355X.

One step = one pass of the decode projections of the Q8_0 attention workload
(batch 1): quantize an 8192-wide fp32 activation to Q8, the 8192 -> 4096 output
projection, quantize a 4096-wide activation, and the paired 4096 -> 1024 +
4096 -> 512 low-rank projection in one launch.  The same step with the
quantization fused into the projections (qgemv_*_f32) is timed too
(config.fused_quantize_step_us).  Inputs are seeded synthetic
tensors resident in HBM before timing starts.  Weights rotate over copies that
together exceed 1 GiB, so no step reads weights left in the 256 MB Infinity
Cache or in L2 by an earlier step.  The steps are captured once in a HIP graph
and replayed, so host launch cost does not enter the timed region.

Prints ONE JSON line.  `value` is the achieved algorithmic HBM bandwidth of the
whole step (packed weight blocks + activations + outputs, GB/s); `roofline`
describes the dominant kernel (the 4096 x 8192 Q8_0 GEMV) timed live with HIP
events; `cpu_baseline` is the fp64 CPU oracle on a bounded sample of the same
step; `extra` holds the other workloads (latency, Q4_K, batched sweep, routed
MoE tokens/s, prefill) measured the same way.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-extra]
       python bench.py --summarize-rocprof DIR   (turn rocprofv3 csv output into a text summary)
       python bench.py --probe {gemv,gemv_batch,copy,prefill,prefill_ws,prefill_q8_0,fp8_16384x4096,fp4_16384x4096,
                                 moe_e256_t1,moe_fp8_e256_t1,moe_fp4_e384_t1,...} --steps K
                 (eager launches of one kernel, for rocprofv3 --pmc counter runs)
       python bench.py --summarize-pmc GEMV_FETCH GEMV_WRITE COPY_FETCH COPY_WRITE
                 (HBM bytes per launch of the GEMV from FETCH_SIZE / WRITE_SIZE runs,
                  scaled by the copy kernel's counters; writes profiles/qgemv_q8_0_4096x8192_hbm_traffic.json)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
MFMA_FP16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16, published
MFMA_INT8_PEAK_TOPS = 5000.0    # MI355X dense int8, published
ROTATE_BYTES = 1 << 30  # > 2x the 256 MB Infinity Cache
METRIC = "decode GEMV µs and achieved HBM GB/s (% of peak); routed-MoE tokens/s"


GEMV_SOURCES = ("csrc/gemv.hip", "csrc/gemv_device.h", "csrc/quantize_device.h", "csrc/common.h",
                "../include/qgemv.h")


def kernel_source_hash(files=GEMV_SOURCES) -> str:
    """Hash of the sources the GEMV kernel is compiled from; counter summaries record it, so
    counters taken on an older kernel are detected and not reported."""
    h = hashlib.sha256()
    pkg = os.path.join(ROOT, "routed_moe_matvec_amd")
    for name in files:
        with open(os.path.normpath(os.path.join(pkg, name)), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


# ----------------------------------------------------------------------------- timing helpers

TRIALS = 7  # timed replays per measurement; the median is reported, with the interquartile range


class Timer:
    """HIP-event timing of work enqueued on one stream."""

    def __init__(self, stream):
        import torch
        self.torch = torch
        self.stream = stream

    def run(self, fn):
        torch = self.torch
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        with torch.cuda.stream(self.stream):  # graph replays go to the current stream
            s.record(self.stream)
            fn()
            e.record(self.stream)
        torch.cuda.synchronize()
        return s.elapsed_time(e) * 1e-3  # seconds

    def trials(self, fn, per_trial: int, trials: int = TRIALS):
        """One untimed call of fn, then `trials` timed calls; seconds per unit of work
        (fn does per_trial units) of each trial."""
        self.run(fn)
        return [self.run(fn) / per_trial for _ in range(trials)]


def spread(samples):
    """Median and interquartile range (p25, p75) of a list of seconds, in microseconds."""
    q = np.percentile(np.asarray(samples, np.float64) * 1e6, [25, 50, 75])
    return {"median_us": round(float(q[1]), 3), "p25_us": round(float(q[0]), 3), "p75_us": round(float(q[2]), 3),
            "trials": len(samples)}


def capture(fn, n: int, stream):
    """HIP graph of n calls fn(0..n-1) on `stream`."""
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        fn(0)  # make sure every lazily created resource exists before capture
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=stream):
        for i in range(n):
            fn(i)
    torch.cuda.synchronize()
    return g


def rotation_count(bytes_per_copy: int) -> int:
    return max(2, -(-ROTATE_BYTES // bytes_per_copy))


# ----------------------------------------------------------------------------- workload

class DecodeStep:
    """The timed step: two quantizations and the out / paired Q8_0 projections."""

    def __init__(self, qg, torch):
        import synth
        w_out = synth.WORKLOADS["q8_0_out_4096x8192"]
        w_pair = synth.WORKLOADS["q8_0_pair_1024+512x4096"]
        g = synth.rng(w_out["seed"])
        self.N, self.K = w_out["N"], w_out["K"]
        self.N1, self.N2, self.K2 = w_pair["N1"], w_pair["N2"], w_pair["K"]
        self.W_host = synth.q8_0_weight(g, self.N, self.K)
        self.x_host = synth.activations(g, 1, self.K)
        self.W1_host = synth.q8_0_weight(g, self.N1, self.K2)
        self.W2_host = synth.q8_0_weight(g, self.N2, self.K2)
        self.x2_host = synth.activations(g, 1, self.K2)
        per_copy = self.W_host.nbytes + self.W1_host.nbytes + self.W2_host.nbytes
        self.R = rotation_count(per_copy)
        dev = "cuda"
        base = [torch.from_numpy(a).to(dev) for a in (self.W_host, self.W1_host, self.W2_host)]
        self.W = [base[0]] + [base[0].clone() for _ in range(self.R - 1)]
        self.W1 = [base[1]] + [base[1].clone() for _ in range(self.R - 1)]
        self.W2 = [base[2]] + [base[2].clone() for _ in range(self.R - 1)]
        self.x = torch.from_numpy(self.x_host).to(dev)
        self.x2 = torch.from_numpy(self.x2_host).to(dev)
        K, K2 = self.K, self.K2
        self.qx = torch.empty(1, K, dtype=torch.int8, device=dev)
        self.dx = torch.empty(1, K // 32, dtype=torch.float32, device=dev)
        self.sx = torch.empty(1, K // 32, dtype=torch.int32, device=dev)
        self.qx2 = torch.empty(1, K2, dtype=torch.int8, device=dev)
        self.dx2 = torch.empty(1, K2 // 32, dtype=torch.float32, device=dev)
        self.sx2 = torch.empty(1, K2 // 32, dtype=torch.int32, device=dev)
        self.y = torch.empty(1, self.N, dtype=torch.float32, device=dev)
        self.y1 = torch.empty(1, self.N1, dtype=torch.float32, device=dev)
        self.y2 = torch.empty(1, self.N2, dtype=torch.float32, device=dev)
        self.qg = qg
        self.weight_bytes = per_copy

    # algorithmic bytes (what the method must move), per kernel
    def bytes_quantize(self, K):
        return K * 4 + K + (K // 32) * 8

    def bytes_gemv(self, Wbytes, N, K):
        return Wbytes + K + (K // 32) * 4 + N * 4

    @property
    def out_gemv_bytes(self):
        return self.bytes_gemv(self.W_host.nbytes, self.N, self.K)

    @property
    def step_bytes(self):
        return (self.bytes_quantize(self.K) + self.out_gemv_bytes + self.bytes_quantize(self.K2)
                + self.W1_host.nbytes + self.W2_host.nbytes + self.K2 + (self.K2 // 32) * 4
                + (self.N1 + self.N2) * 4)

    def step(self, i):
        """quantize_act_q8 once per activation, then the projections that consume it."""
        qg, r = self.qg, i % self.R
        qg.quantize_act_q8(self.x, 1, self.K, self.qx, self.dx, self.sx)
        qg.qgemv_q8_0(self.W[r], self.N, self.K, self.qx, self.dx, 1, self.y)
        qg.quantize_act_q8(self.x2, 1, self.K2, self.qx2, self.dx2, self.sx2)
        qg.qgemv_paired(qg.FMT_Q8_0, self.W1[r], self.N1, self.W2[r], self.N2, self.K2, self.qx2, self.dx2,
                        self.sx2, 1, self.y1, self.y2)

    def step_fused(self, i):
        """The same step with the quantization done inside the consuming projections."""
        qg, r = self.qg, i % self.R
        qg.qgemv_q8_0_f32(self.W[r], self.N, self.K, self.x, 1, self.y, self.qx, self.dx, self.sx)
        qg.qgemv_paired_f32(qg.FMT_Q8_0, self.W1[r], self.N1, self.W2[r], self.N2, self.K2, self.x2, 1, self.y1,
                            self.y2, self.qx2, self.dx2, self.sx2)

    def out_gemv(self, i):
        self.qg.qgemv_q8_0(self.W[i % self.R], self.N, self.K, self.qx, self.dx, 1, self.y)


def host_threads() -> int:
    """Host cores this process may use (its CPU affinity, capped by OMP_NUM_THREADS when set)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and int(omp) > 0:
        n = min(n, int(omp))
    return max(1, n)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(step: DecodeStep, budget_s: float = 8.0) -> dict:
    """The CPU oracle, untuned, on the same step: quantize both activations and run the
    three products in fp64, as many whole steps as fit in ~budget_s, once on all the
    host cores this process may use (OpenMP over rows) and once on one thread."""
    import oracle

    def leg(threads):
        t0 = time.perf_counter()
        n = 0
        while True:
            qx, dx, _ = oracle.quantize_act_q8(step.x_host)
            oracle.gemv(oracle.FMT_Q8_0, step.W_host, step.N, step.K, qx, dx, nthreads=threads)
            qx2, dx2, _ = oracle.quantize_act_q8(step.x2_host)
            oracle.gemv(oracle.FMT_Q8_0, step.W1_host, step.N1, step.K2, qx2, dx2, nthreads=threads)
            oracle.gemv(oracle.FMT_Q8_0, step.W2_host, step.N2, step.K2, qx2, dx2, nthreads=threads)
            n += 1
            el = time.perf_counter() - t0
            if el >= budget_s:
                return n, el / n

    threads = host_threads()
    n_all, per_all = leg(threads)
    n_one, per_one = leg(1)
    return {"value": round(step.step_bytes / per_all / 1e9, 3), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "ms_per_step": round(per_all * 1e3, 3),
            "value_1thread": round(step.step_bytes / per_one / 1e9, 3), "ms_per_step_1thread": round(per_one * 1e3, 3),
            "cpu_model": cpu_model(),
            "sample": "%d whole steps on %d threads and %d on 1 thread of the same decode workload (quantize 8192 + "
                      "Q8_0 4096x8192 + quantize 4096 + Q8_0 1024x4096 and 512x4096), fp64 oracle, OpenMP over "
                      "rows" % (n_all, threads, n_one)}


def gpu_clocks() -> dict:
    """The GPU's current clocks as the driver reports them (read only; nothing is changed):
    the graphics clock of each XCD (min and max over them), memory and SoC clocks, and
    whether any clock is locked."""
    import subprocess
    try:
        p = subprocess.run(["amd-smi", "metric", "-g", "0", "-c", "--json"], capture_output=True, text=True,
                           timeout=20)
        clk = json.loads(p.stdout)["gpu_data"][0]["clock"]
    except (OSError, subprocess.TimeoutExpired, ValueError, KeyError, IndexError, TypeError):
        return {"tool": "amd-smi metric -c", "report": "not available"}

    def mhz(v):
        c = v.get("clk") if isinstance(v, dict) else None
        return c.get("value") if isinstance(c, dict) else None

    gfx = [mhz(v) for k, v in clk.items() if k.startswith("gfx_") and mhz(v) is not None]
    out = {"tool": "amd-smi metric -c", "gfx_mhz_min": min(gfx) if gfx else None,
           "gfx_mhz_max": max(gfx) if gfx else None, "xcds": len(gfx)}
    for key in ("mem_0", "socclk_0", "fclk_0"):
        if key in clk:
            out[key.split("_")[0] + "_mhz"] = mhz(clk[key])
    g0 = clk.get("gfx_0", {})
    out["gfx_max_mhz"] = (g0.get("max_clk") or {}).get("value") if isinstance(g0.get("max_clk"), dict) else None
    out["locked"] = sorted({str(v.get("clk_locked")) for v in clk.values() if isinstance(v, dict)})
    return out


def read_ceilings(qg, torch, stream, timer, same_bytes: int) -> dict:
    """Measured read rates of this part, by qg_stream_read (the library's streaming-read
    diagnostic): the rate over a 1 GiB buffer read in one launch, and the best time per
    launch for reading `same_bytes` once per launch, back to back in a graph, from
    rotating places in that buffer (so no launch reads bytes left in a cache)."""
    big = 1 << 30
    buf = torch.empty(big, dtype=torch.uint8, device="cuda")
    buf.fill_(0x5A)
    out = {}
    # (no output array: the read alone; the tests check what it reads)
    best_big = None
    for kib, waves in ((4, 4), (8, 4)):
        with torch.cuda.stream(stream):
            sp = spread(timer.trials(lambda: qg.qg_stream_read(buf, big, kib, waves, None, 0, stream=stream), 1))
        if best_big is None or sp["median_us"] < best_big["median_us"]:
            best_big = dict(sp, chunk_kib=kib, waves=waves)
    best_big["GB_s"] = round(big / (best_big["median_us"] * 1e-6) / 1e9, 1)
    out["read_1gib"] = best_big
    R = big // same_bytes
    best = None
    for kib, waves in ((2, 4), (4, 4), (8, 4), (4, 8), (8, 8)):
        n = max(R, 100)
        gr = capture(lambda i: qg.qg_stream_read(buf[(i % R) * same_bytes:], same_bytes, kib, waves, None, 0,
                                                 stream=stream), n, stream)
        sp = spread(timer.trials(gr.replay, n))
        if best is None or sp["median_us"] < best["median_us"]:
            best = dict(sp, chunk_kib=kib, waves=waves)
        del gr
    best["GB_s"] = round(same_bytes / (best["median_us"] * 1e-6) / 1e9, 1)
    best["bytes"] = same_bytes
    out["read_same_bytes"] = best
    del buf
    torch.cuda.empty_cache()
    return out


def load_traffic(kernel_key: str, src_hash: str):
    """Measured HBM bytes per launch from the committed counter summary, if it was taken
    on the current kernel sources; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    ent = data.get(kernel_key)
    if not ent or ent.get("source_hash") != src_hash:
        return None
    return ent.get("hbm_bytes_per_launch")


# ----------------------------------------------------------------------------- extra workloads

def extra_measurements(qg, torch, stream, timer) -> dict:
    import synth
    out = {}
    dev = "cuda"

    def quantized(K, M=1, seed=0):
        g = synth.rng(seed)
        x = torch.from_numpy(synth.activations(g, M, K)).to(dev)
        qx = torch.empty(M, K, dtype=torch.int8, device=dev)
        dx = torch.empty(M, K // 32, dtype=torch.float32, device=dev)
        sx = torch.empty(M, K // 32, dtype=torch.int32, device=dev)
        qg.quantize_act_q8(x, M, K, qx, dx, sx)
        return qx, dx, sx

    def gemv_rate(fmt, W_host, N, K, Ms, label, G=1):
        """G > 1: the grouped call, W_host holding G matrices of N rows on G input slices of K."""
        R = rotation_count(W_host.nbytes)
        base = torch.from_numpy(W_host).to(dev)
        copies = [base] + [base.clone() for _ in range(R - 1)]
        res = {}
        for M in Ms:
            qx, dx, sx = quantized(G * K, M)
            y = torch.empty(M, G * N, dtype=torch.float32, device=dev)
            if G > 1:
                fn = lambda i: qg.qgemv_grouped(fmt, copies[i % R], G, N, K, qx, dx, sx, M, y)
            elif fmt in (qg.FMT_FP8_E4M3_B128, qg.FMT_FP4_E2M1_MX):
                fn = lambda i: qg.qgemv_mx(fmt, copies[i % R], N, K, qx, dx, M, y)
            elif fmt == 0:
                fn = lambda i: qg.qgemv_q8_0(copies[i % R], N, K, qx, dx, M, y)
            else:
                fn = lambda i: qg.qgemv_q4k(copies[i % R], N, K, qx, dx, sx, M, y)
            n = max(R, 64)
            g = capture(fn, n, stream)
            sp = spread(timer.trials(g.replay, n))
            sec = sp["median_us"] * 1e-6
            byts = W_host.nbytes + G * (M * K + M * (K // 32) * (8 if fmt == 1 else 4) + M * N * 4)
            res["M%d" % M] = {"us": round(sec * 1e6, 3), "iqr_us": [sp["p25_us"], sp["p75_us"]],
                              "GB_s": round(byts / sec / 1e9, 1), "hbm_frac": round(byts / sec / 1e9 / HBM_PEAK_GBS, 4)}
            del g
        del copies, base
        torch.cuda.empty_cache()
        out[label] = res

    def moe_rate(key, n_sets):
        w = synth.WORKLOADS[key]
        E, D, F, T, topk = w["E"], w["D"], w["F"], w["T"], w["topk"]
        fmt = w.get("fmt", qg.FMT_Q4K)
        g = synth.rng(w["seed"])
        # two full expert pools, generated expert by expert straight to the device
        pools = []
        for _ in range(2):
            pool = [[], [], []]
            for e in range(E):
                for lst, (n, k) in zip(pool, ((F, D), (F, D), (D, F))):
                    lst.append(torch.from_numpy(synth.weight(fmt, g, n, k)).to(dev))
            pools.append([qg.pointer_table(lst, dev) for lst in pool] + [pool])
        draw = synth.moe_ids_zipf if w["ids"] == "zipf" else synth.moe_ids_uniform
        ids = [draw(g, T, E, topk) for _ in range(n_sets)]
        rws = [torch.from_numpy(synth.routing_weights(g, T, topk)).to(dev) for _ in range(n_sets)]
        xs = [torch.from_numpy(synth.activations(g, T, D)).to(dev) for _ in range(n_sets)]
        ids_d = [torch.from_numpy(i).to(dev) for i in ids]
        qx = torch.empty(T, D, dtype=torch.int8, device=dev)
        dx = torch.empty(T, D // 32, dtype=torch.float32, device=dev)
        sx = torch.empty(T, D // 32, dtype=torch.int32, device=dev)
        y = torch.empty(T, D, dtype=torch.float32, device=dev)
        nbytes = qg.moe_routed_workspace_bytes(T, topk, E, D, F)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        status = torch.empty(1, dtype=torch.int32, device=dev)

        def call(i):
            k = i % n_sets
            pool = pools[i % 2]
            qg.quantize_act_q8(xs[k], T, D, qx, dx, sx)
            qg.moe_routed_qgemv_fmt(fmt, qx, dx, sx, T, D, F, E, topk, ids_d[k], rws[k], pool[0], pool[1], pool[2],
                                    y, ws, nbytes, status)

        n = 2 * n_sets
        gr = capture(call, n, stream)
        sp = spread(timer.trials(gr.replay, n))
        sec = sp["median_us"] * 1e-6
        expert_bytes = 2 * qg.qg_matrix_bytes(fmt, F, D) + qg.qg_matrix_bytes(fmt, D, F)
        uniq = np.mean([len(np.unique(i)) for i in ids])
        byts = uniq * expert_bytes + T * D * 4 * 2 + T * topk * 8
        out["moe_" + key.split("_", 1)[1]] = {
            "tokens_per_s": round(T / sec, 1), "us_per_call": round(sec * 1e6, 3),
            "iqr_us": [sp["p25_us"], sp["p75_us"]], "mean_distinct_experts": float(uniq),
            "GB_s": round(byts / sec / 1e9, 1), "hbm_frac": round(byts / sec / 1e9 / HBM_PEAK_GBS, 4),
            "includes": ("quantize_act_q8 of the T tokens + moe_routed_qgemv (3 launches at T=1, the table built "
                         "in the gate/up launch; 5 for 2-8 tokens; 7 from 9 tokens: the popular experts' "
                         "matrix-core launches)"
                         if fmt == qg.FMT_Q4K else
                         "quantize_act_q8 of the T tokens + moe_routed_qgemv_fmt (at T=1 the table built in the "
                         "gate/up launch: 4 launches, 3 for FP4 experts whose down launch also forms h; 5 "
                         "otherwise)")}
        del gr, pools, ws
        torch.cuda.empty_cache()

    def prefill_rate():
        w = synth.WORKLOADS["q4k_prefill_512x8192x4096"]
        g = synth.rng(w["seed"])
        N, K, M = w["N"], w["K"], w["M"]
        W_host = synth.q4k_weight(g, N, K)
        R = rotation_count(W_host.nbytes)
        base = torch.from_numpy(W_host).to(dev)
        copies = [base] + [base.clone() for _ in range(R - 1)]
        xb = torch.from_numpy(synth.bf16_activations(g, M, K).view(np.int16)).to(dev)
        y = torch.empty(M, N, dtype=torch.float32, device=dev)
        nb = qg.qgemm_prefill_workspace_bytes(M, K)
        ws = torch.empty(nb, dtype=torch.uint8, device=dev)
        flops = 2.0 * M * N * K
        res = {}
        for name, fn in [
                ("qgemm_prefill", lambda i: qg.qgemm_prefill(qg.FMT_Q4K, copies[i % R], N, K, xb, M, y)),
                ("qgemm_prefill_ws", lambda i: qg.qgemm_prefill_ws(qg.FMT_Q4K, copies[i % R], N, K, xb, M, y, ws,
                                                                   nb))]:
            gr = capture(fn, R, stream)
            sp = spread(timer.trials(gr.replay, R))
            sec = sp["median_us"] * 1e-6
            res[name] = {"us": round(sec * 1e6, 3), "iqr_us": [sp["p25_us"], sp["p75_us"]],
                         "TFLOP_s": round(flops / sec / 1e12, 1),
                         "mfma_frac": round(flops / sec / 1e12 / MFMA_FP16_PEAK_TFLOPS, 4)}
            del gr
        res["includes"] = "qgemm_prefill_ws: the bf16 -> fp16 pre-pass and the GEMM"
        out["prefill_q4k_512x8192x4096"] = res
        del copies, base, ws
        torch.cuda.empty_cache()

    g = synth.rng(0)
    w = synth.WORKLOADS["q8_0_512x1024"]
    gemv_rate(0, synth.q8_0_weight(g, w["N"], w["K"]), w["N"], w["K"], [1], "q8_0_512x1024")
    # the fp32-activation comparator on the out-projection (no activation quantization)
    w = synth.WORKLOADS["q8_0_out_4096x8192"]
    gq = synth.rng(w["seed"])
    Wq = synth.q8_0_weight(gq, w["N"], w["K"])
    R = rotation_count(Wq.nbytes)
    base = torch.from_numpy(Wq).to(dev)
    copies = [base] + [base.clone() for _ in range(R - 1)]
    xq = torch.from_numpy(synth.activations(gq, 1, w["K"])).to(dev)
    yq = torch.empty(1, w["N"], dtype=torch.float32, device=dev)
    n = max(R, 64)
    gr = capture(lambda i: qg.qgemv_q8_0_quality(copies[i % R], w["N"], w["K"], xq, 1, yq), n, stream)
    sp = spread(timer.trials(gr.replay, n))
    sec = sp["median_us"] * 1e-6
    byts = Wq.nbytes + w["K"] * 4 + w["N"] * 4
    out["quality_q8_0_4096x8192"] = {"us": round(sec * 1e6, 3), "iqr_us": [sp["p25_us"], sp["p75_us"]],
                                     "GB_s": round(byts / sec / 1e9, 1),
                                     "hbm_frac": round(byts / sec / 1e9 / HBM_PEAK_GBS, 4),
                                     "includes": "qgemv_q8_0_quality: fp32 activation, no quantization"}
    del gr, copies, base
    torch.cuda.empty_cache()
    w = synth.WORKLOADS["q8_0_grouped_8x1024x4096"]
    gw = synth.rng(w["seed"])
    gemv_rate(0, np.concatenate([synth.q8_0_weight(gw, w["N"], w["K"]) for _ in range(w["G"])], axis=0), w["N"],
              w["K"], [1], "q8_0_grouped_8x1024x4096", G=w["G"])
    w = synth.WORKLOADS["q4k_8192x4096"]
    gemv_rate(1, synth.q4k_weight(synth.rng(w["seed"]), w["N"], w["K"]), w["N"], w["K"], [1, 8, 16, 32],
              "q4k_8192x4096")
    w = synth.WORKLOADS["q8_0_16384x4096"]
    gemv_rate(0, synth.q8_0_weight(synth.rng(w["seed"]), w["N"], w["K"]), w["N"], w["K"], list(w["Ms"]),
              "q8_0_16384x4096")
    for key in ("fp8_16384x4096", "fp4_16384x4096"):
        w = synth.WORKLOADS[key]
        gemv_rate(w["fmt"], synth.weight(w["fmt"], synth.rng(w["seed"]), w["N"], w["K"]), w["N"], w["K"], [1], key)
    prefill_rate()
    # the Q8_0 prefill product on int8 MFMA, with its activation quantization
    w = synth.WORKLOADS["q8_0_prefill_512x8192x4096"]
    gp = synth.rng(w["seed"])
    N, K, M = w["N"], w["K"], w["M"]
    W_host = synth.q8_0_weight(gp, N, K)
    R = rotation_count(W_host.nbytes)
    base = torch.from_numpy(W_host).to(dev)
    copies = [base] + [base.clone() for _ in range(R - 1)]
    xp = torch.from_numpy(synth.activations(gp, M, K)).to(dev)
    qx, dx, sx = (torch.empty(M, K, dtype=torch.int8, device=dev), torch.empty(M, K // 32, dtype=torch.float32,
                  device=dev), torch.empty(M, K // 32, dtype=torch.int32, device=dev))
    yp = torch.empty(M, N, dtype=torch.float32, device=dev)

    def q8_prefill(i):
        qg.quantize_act_q8(xp, M, K, qx, dx, sx)
        qg.qgemm_q8_0(copies[i % R], N, K, qx, dx, M, yp)
    gr = capture(q8_prefill, R, stream)
    sp = spread(timer.trials(gr.replay, R))
    sec = sp["median_us"] * 1e-6
    ops = 2.0 * M * N * K
    out["prefill_q8_0_512x8192x4096"] = {
        "us": round(sec * 1e6, 3), "iqr_us": [sp["p25_us"], sp["p75_us"]], "TOP_s": round(ops / sec / 1e12, 1),
        "mfma_frac": round(ops / sec / 1e12 / MFMA_INT8_PEAK_TOPS, 4),
        "includes": "quantize_act_q8 of the 512 tokens + qgemm_q8_0 (int8 MFMA; rows equal the decode call)"}
    del gr, copies, base
    torch.cuda.empty_cache()
    moe_rate("moe_e256_t1", 16)
    moe_rate("moe_e256_t8", 16)
    moe_rate("moe_e384_t64_zipf", 4)
    moe_rate("moe_fp8_e256_t1", 16)
    moe_rate("moe_fp4_e384_t1", 16)
    return out


# ----------------------------------------------------------------------------- rocprof summary

def summarize_rocprof(path: str) -> str:
    """Text summary of a rocprofv3 --kernel-trace --stats --output-format csv directory:
    per (kernel, grid size) the number of dispatches and their average / min / max duration."""
    import csv
    import glob
    import statistics
    lines = []
    for tr in sorted(glob.glob(os.path.join(path, "**", "*kernel_trace.csv"), recursive=True)):
        with open(tr) as f:
            rows = list(csv.DictReader(f))
        groups = {}
        for r in rows:
            key = (r.get("Kernel_Name", "?"), r.get("Grid_Size_X", r.get("Grid_Size", "?")))
            d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            groups.setdefault(key, []).append(d)
        lines.append("# %s: per kernel and grid size, durations in microseconds" % os.path.relpath(tr, path))
        lines.append("%-56s %9s %6s %10s %10s %10s %10s" % ("kernel", "grid_x", "calls", "avg_us", "median_us",
                                                            "min_us", "max_us"))
        for (name, grid), ds in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
            lines.append("%-56s %9s %6d %10.3f %10.3f %10.3f %10.3f" % (
                name[:56], grid, len(ds), sum(ds) / len(ds), statistics.median(ds), min(ds), max(ds)))
        # The busiest (kernel, grid) split by the kernel dispatched just before it:
        # one kernel replayed back to back and the same kernel inside a longer
        # sequence of launches run at different speeds.
        if groups:
            top = max(groups, key=lambda k: sum(groups[k]))
            rows.sort(key=lambda r: int(r["Start_Timestamp"]))
            after = {}
            for prev, r in zip([None] + rows[:-1], rows):
                if (r.get("Kernel_Name", "?"), r.get("Grid_Size_X", r.get("Grid_Size", "?"))) != top:
                    continue
                pk = "-" if prev is None else "%s grid_x %s" % (prev.get("Kernel_Name", "?")[:48],
                                                                 prev.get("Grid_Size_X", prev.get("Grid_Size", "?")))
                after.setdefault(pk, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
            lines.append("# %s grid_x %s by the dispatch before it" % (top[0][:56], top[1]))
            for pk, ds in sorted(after.items(), key=lambda kv: -len(kv[1])):
                lines.append("  after %-66s calls=%d avg_us=%.3f median_us=%.3f" % (
                    pk, len(ds), sum(ds) / len(ds), statistics.median(ds)))
    for s in sorted(glob.glob(os.path.join(path, "**", "*kernel_stats.csv"), recursive=True)):
        with open(s) as f:
            rows = list(csv.DictReader(f))
        lines.append("# %s: rocprofv3 --stats per kernel name" % os.path.relpath(s, path))
        for r in rows:
            lines.append("%-70s calls=%s avg_us=%.3f min_us=%.3f max_us=%.3f" % (
                r.get("Name", "?")[:70], r.get("Calls"), float(r.get("AverageNs", 0)) / 1e3,
                float(r.get("MinNs", 0)) / 1e3, float(r.get("MaxNs", 0)) / 1e3))
    return "\n".join(lines)



# ----------------------------------------------------------------------------- counter runs

TRAFFIC_FILE = os.path.join(ROOT, "profiles", "qgemv_q8_0_4096x8192_hbm_traffic.json")
COPY_PROBE_BYTES = 1 << 29  # 512 MiB read + 512 MiB written per copy launch


def run_probe(name: str, steps: int, warmup: int, qg, torch) -> None:
    """Eager launches (no graph, so counters attribute per dispatch) of one kernel,
    rotating weights like the timed runs."""
    import synth
    stream = torch.cuda.current_stream()
    if name == "gemv":
        step = DecodeStep(qg, torch)
        step.step(0)  # quantized activations for the projection
        fn = step.out_gemv
    elif name.startswith("gemv_batch"):
        # the batched Q8_0 sweep: 16384 x 4096, 32 tokens (gemv_batch) or the
        # number of tokens after the name (gemv_batch8: 8 tokens)
        w = synth.WORKLOADS["q8_0_16384x4096"]
        g = synth.rng(w["seed"])
        N, K = w["N"], w["K"]
        M = int(name[len("gemv_batch"):]) if name != "gemv_batch" else max(w["Ms"])
        W_host = synth.q8_0_weight(g, N, K)
        R = rotation_count(W_host.nbytes)
        base = torch.from_numpy(W_host).to("cuda")
        copies = [base] + [base.clone() for _ in range(R - 1)]
        x = torch.from_numpy(synth.activations(g, M, K)).to("cuda")
        qx = torch.empty(M, K, dtype=torch.int8, device="cuda")
        dx = torch.empty(M, K // 32, dtype=torch.float32, device="cuda")
        sx = torch.empty(M, K // 32, dtype=torch.int32, device="cuda")
        qg.quantize_act_q8(x, M, K, qx, dx, sx)
        y = torch.empty(M, N, dtype=torch.float32, device="cuda")

        def fn(i):
            qg.qgemv_q8_0(copies[i % R], N, K, qx, dx, M, y)
    elif name == "q4k":
        # the one-token Q4_K projection 4096 -> 8192
        w = synth.WORKLOADS["q4k_8192x4096"]
        g = synth.rng(w["seed"])
        N, K = w["N"], w["K"]
        W_host = synth.q4k_weight(g, N, K)
        R = rotation_count(W_host.nbytes)
        base = torch.from_numpy(W_host).to("cuda")
        copies = [base] + [base.clone() for _ in range(R - 1)]
        x = torch.from_numpy(synth.activations(g, 1, K)).to("cuda")
        qx = torch.empty(1, K, dtype=torch.int8, device="cuda")
        dx = torch.empty(1, K // 32, dtype=torch.float32, device="cuda")
        sx = torch.empty(1, K // 32, dtype=torch.int32, device="cuda")
        qg.quantize_act_q8(x, 1, K, qx, dx, sx)
        y = torch.empty(1, N, dtype=torch.float32, device="cuda")

        def fn(i):
            qg.qgemv_q4k(copies[i % R], N, K, qx, dx, sx, 1, y)
    elif name in ("fp8_16384x4096", "fp4_16384x4096"):
        w = synth.WORKLOADS[name]
        g = synth.rng(w["seed"])
        fmt, N, K = w["fmt"], w["N"], w["K"]
        W_host = synth.weight(fmt, g, N, K)
        R = rotation_count(W_host.nbytes)
        base = torch.from_numpy(W_host).to("cuda")
        copies = [base] + [base.clone() for _ in range(R - 1)]
        x = torch.from_numpy(synth.activations(g, 1, K)).to("cuda")
        qx = torch.empty(1, K, dtype=torch.int8, device="cuda")
        dx = torch.empty(1, K // 32, dtype=torch.float32, device="cuda")
        sx = torch.empty(1, K // 32, dtype=torch.int32, device="cuda")
        qg.quantize_act_q8(x, 1, K, qx, dx, sx)
        y = torch.empty(1, N, dtype=torch.float32, device="cuda")

        def fn(i):
            qg.qgemv_mx(fmt, copies[i % R], N, K, qx, dx, 1, y)
    elif name == "prefill_q8_0":
        w = synth.WORKLOADS["q8_0_prefill_512x8192x4096"]
        g = synth.rng(w["seed"])
        N, K, M = w["N"], w["K"], w["M"]
        W_host = synth.q8_0_weight(g, N, K)
        R = rotation_count(W_host.nbytes)
        base = torch.from_numpy(W_host).to("cuda")
        copies = [base] + [base.clone() for _ in range(R - 1)]
        x = torch.from_numpy(synth.activations(g, M, K)).to("cuda")
        qx = torch.empty(M, K, dtype=torch.int8, device="cuda")
        dx = torch.empty(M, K // 32, dtype=torch.float32, device="cuda")
        sx = torch.empty(M, K // 32, dtype=torch.int32, device="cuda")
        qg.quantize_act_q8(x, M, K, qx, dx, sx)
        y = torch.empty(M, N, dtype=torch.float32, device="cuda")

        def fn(i):
            qg.qgemm_q8_0(copies[i % R], N, K, qx, dx, M, y)
    elif name == "copy":
        src = torch.ones(COPY_PROBE_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)

        def fn(i):
            dst.copy_(src)
    elif name in ("prefill", "prefill_ws"):
        w = synth.WORKLOADS["q4k_prefill_512x8192x4096"]
        g = synth.rng(w["seed"])
        N, K, M = w["N"], w["K"], w["M"]
        W_host = synth.q4k_weight(g, N, K)
        R = rotation_count(W_host.nbytes)
        base = torch.from_numpy(W_host).to("cuda")
        copies = [base] + [base.clone() for _ in range(R - 1)]
        xb = torch.from_numpy(synth.bf16_activations(g, M, K).view(np.int16)).to("cuda")
        y = torch.empty(M, N, dtype=torch.float32, device="cuda")
        nb = qg.qgemm_prefill_workspace_bytes(M, K)
        ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
        if name == "prefill":
            def fn(i):
                qg.qgemm_prefill(qg.FMT_Q4K, copies[i % R], N, K, xb, M, y)
        else:
            def fn(i):
                qg.qgemm_prefill_ws(qg.FMT_Q4K, copies[i % R], N, K, xb, M, y, ws, nb)
    elif name.startswith("moe_"):
        w = synth.WORKLOADS[name]
        E, D, F, T, topk = w["E"], w["D"], w["F"], w["T"], w["topk"]
        fmt = w.get("fmt", qg.FMT_Q4K)
        g = synth.rng(w["seed"])
        pools = []
        for _ in range(2):
            pool = [[], [], []]
            for e in range(E):
                for lst, (n, k) in zip(pool, ((F, D), (F, D), (D, F))):
                    lst.append(torch.from_numpy(synth.weight(fmt, g, n, k)).to("cuda"))
            pools.append([qg.pointer_table(lst, "cuda") for lst in pool] + [pool])
        draw = synth.moe_ids_zipf if w["ids"] == "zipf" else synth.moe_ids_uniform
        ids_d = torch.from_numpy(draw(g, T, E, topk)).to("cuda")
        rw = torch.from_numpy(synth.routing_weights(g, T, topk)).to("cuda")
        x = torch.from_numpy(synth.activations(g, T, D)).to("cuda")
        qx = torch.empty(T, D, dtype=torch.int8, device="cuda")
        dx = torch.empty(T, D // 32, dtype=torch.float32, device="cuda")
        sx = torch.empty(T, D // 32, dtype=torch.int32, device="cuda")
        y = torch.empty(T, D, dtype=torch.float32, device="cuda")
        nb = qg.moe_routed_workspace_bytes(T, topk, E, D, F)
        ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
        status = torch.empty(1, dtype=torch.int32, device="cuda")

        def fn(i):
            pool = pools[i % 2]
            qg.quantize_act_q8(x, T, D, qx, dx, sx)
            qg.moe_routed_qgemv_fmt(fmt, qx, dx, sx, T, D, F, E, topk, ids_d, rw, pool[0], pool[1], pool[2], y, ws,
                                    nb, status)
    else:
        raise SystemExit("unknown probe %r" % name)
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        fn(i)
    torch.cuda.synchronize()
    print("probe %s: %d launches, %.3f us each (host clock, eager)" % (
        name, steps, (time.perf_counter() - t0) / steps * 1e6), flush=True)
    del stream


def pmc_values(path: str) -> dict:
    """{(kernel name, counter): mean value per dispatch} from a rocprofv3 --pmc csv directory."""
    import csv
    import glob
    acc = {}
    for f in sorted(glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True)):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                key = (r.get("Kernel_Name", "?"), r.get("Counter_Name", "?"))
                acc.setdefault(key, []).append(float(r.get("Counter_Value", "nan")))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def pick(vals: dict, counter: str, needle: str):
    hits = [(k, v) for k, v in vals.items() if k[1] == counter and needle in k[0]]
    if not hits:
        raise SystemExit("no %s value for a kernel matching %r" % (counter, needle))
    return max(hits, key=lambda kv: kv[1])


def summarize_pmc(gf: str, gw: str, cf: str, cw: str) -> str:
    """HBM traffic per GEMV launch: FETCH_SIZE / WRITE_SIZE (KiB per dispatch), each scaled by
    the factor that makes the same counter read exactly the copy kernel's known bytes."""
    (gk, g_fetch) = pick(pmc_values(gf), "FETCH_SIZE", "qgemv_kernel")
    (_, g_write) = pick(pmc_values(gw), "WRITE_SIZE", "qgemv_kernel")
    (ck, c_fetch) = pick(pmc_values(cf), "FETCH_SIZE", "")
    (_, c_write) = pick(pmc_values(cw), "WRITE_SIZE", "")
    known_kib = COPY_PROBE_BYTES / 1024.0
    f_read, f_write = known_kib / c_fetch, known_kib / c_write
    hbm = (g_fetch * f_read + g_write * f_write) * 1024.0
    ent = {
        "kernel": gk[0][:120], "source_hash": kernel_source_hash(),
        "fetch_kib_per_dispatch": round(g_fetch, 1), "write_kib_per_dispatch": round(g_write, 1),
        "copy_kernel": ck[0][:120], "copy_bytes": COPY_PROBE_BYTES,
        "copy_fetch_kib": round(c_fetch, 1), "copy_write_kib": round(c_write, 1),
        "read_scale": round(f_read, 4), "write_scale": round(f_write, 4),
        "hbm_bytes_per_launch": int(round(hbm)),
    }
    pmc = "rocprofv3 --output-format csv --pmc %s -d %s -o run -- python3 -u bench.py --probe %s --steps %d --warmup %d"
    ent["commands"] = [
        pmc % ("FETCH_SIZE", gf, "gemv", 50, 5), pmc % ("WRITE_SIZE", gw, "gemv", 50, 5),
        pmc % ("FETCH_SIZE", cf, "copy", 5, 1), pmc % ("WRITE_SIZE", cw, "copy", 5, 1),
        "python3 bench.py --summarize-pmc %s %s %s %s" % (gf, gw, cf, cw)]
    ent["note"] = ("FETCH_SIZE / WRITE_SIZE are KiB per dispatch; each is multiplied by the factor that makes "
                   "the same counter equal the known bytes of a %d-byte device copy" % COPY_PROBE_BYTES)
    path = TRAFFIC_FILE
    try:
        with open(path) as f:
            data = json.load(f)
    except (OSError, ValueError):
        data = {}
    data["qgemv_q8_0_4096x8192"] = ent
    with open(path, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
        f.write("\n")
    return json.dumps(ent, indent=1)

SQ_PASSES = (
    "SQ_WAVES SQ_BUSY_CYCLES SQ_WAVE_CYCLES SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_WAIT_INST_LDS SQ_INSTS_SALU",
    "SQ_LDS_BANK_CONFLICT SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS SQ_ACTIVE_INST_ANY "
    "SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CU_CYCLES",
)


def summarize_sq(d1: str, d2: str, kernel: str, probe: str, steps: int) -> str:
    """SQ counter summary of one kernel from two rocprofv3 --pmc passes (SQ_PASSES) of
    `bench.py --probe PROBE`: mean per dispatch of the dispatches whose kernel name starts
    with `kernel`, and the ratios used to read them."""
    vals = {}
    for d in (d1, d2):
        for (name, counter), v in pmc_values(d).items():
            if name.startswith(kernel):
                vals.setdefault(counter, []).append(v)
    v = {c: sum(x) / len(x) for c, x in vals.items()}
    lines = ["# rocprofv3 SQ counters of %s (probe %s)" % (kernel, probe)]
    for i, counters in enumerate(SQ_PASSES):
        lines.append("# pass %d: rocprofv3 --output-format csv --pmc %s -d %s -o run -- python3 -u bench.py "
                     "--probe %s --steps %d --warmup 2" % (i + 1, counters, (d1, d2)[i], probe, steps))
    lines.append("# summary: python3 bench.py --summarize-sq %s %s '%s' %s %d" % (d1, d2, kernel, probe, steps))
    lines.append("%-28s %16s" % ("counter", "per dispatch"))
    for c in sorted(v):
        lines.append("%-28s %16.1f" % (c, v[c]))
    w = v.get("SQ_WAVES", 0.0)
    if w:
        lines.append("# per wave: VALU %.0f, MFMA %.0f, LDS %.0f, SALU %.0f instructions" % (
            v.get("SQ_INSTS_VALU", 0) / w, v.get("SQ_INSTS_MFMA", 0) / w, v.get("SQ_INSTS_LDS", 0) / w,
            v.get("SQ_INSTS_SALU", 0) / w))
    if v.get("SQ_WAVE_CYCLES") and v.get("SQ_BUSY_CU_CYCLES"):
        lines.append("# SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES = %.2f (share of wave time waiting on a dependency); "
                     "SQ_ACTIVE_INST_VALU / SQ_BUSY_CU_CYCLES = %.2f; SQ_VALU_MFMA_BUSY_CYCLES / SQ_BUSY_CU_CYCLES "
                     "= %.2f" % (v["SQ_WAIT_INST_ANY"] / v["SQ_WAVE_CYCLES"],
                                 v["SQ_ACTIVE_INST_VALU"] / v["SQ_BUSY_CU_CYCLES"],
                                 v["SQ_VALU_MFMA_BUSY_CYCLES"] / v["SQ_BUSY_CU_CYCLES"]))
    return "\n".join(lines)


# ----------------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--summarize-rocprof", default=None)
    ap.add_argument("--probe", default=None)
    ap.add_argument("--summarize-pmc", nargs=4, default=None)
    ap.add_argument("--summarize-sq", nargs=5, default=None, metavar=("PASS1", "PASS2", "KERNEL", "PROBE", "STEPS"))
    args = ap.parse_args()

    if args.summarize_rocprof:
        print(summarize_rocprof(args.summarize_rocprof))
        return 0
    if args.summarize_pmc:
        print(summarize_pmc(*args.summarize_pmc))
        return 0
    if args.summarize_sq:
        d1, d2, kern, probe, steps = args.summarize_sq
        print(summarize_sq(d1, d2, kern, probe, int(steps)))
        return 0
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (the decode mat-vec would "
              "shard by output rows with no exchange, the routed experts by expert). Run with --gpus 1.",
              file=sys.stderr)
        return 2

    import torch
    import routed_moe_matvec_amd as qg

    if args.probe:
        run_probe(args.probe, args.steps, args.warmup, qg, torch)
        return 0
    torch.cuda.init()
    stream = torch.cuda.Stream()
    timer = Timer(stream)
    step = DecodeStep(qg, torch)

    clocks_before = gpu_clocks()
    # warmup: W eager steps, then the graph of K steps replayed once untimed;
    # then TRIALS timed replays of the K steps (the median is reported)
    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            step.step(i)
    torch.cuda.synchronize()
    g_steps = capture(step.step, args.steps, stream)
    step_t = timer.trials(g_steps.replay, args.steps)
    step_sp = spread(step_t)
    ms_per_step = step_sp["median_us"] * 1e-3
    value = step.step_bytes / (ms_per_step * 1e-3) / 1e9

    # dominant kernel: the 4096 x 8192 Q8_0 GEMV, timed alone over a rotation of weights
    n_k = max(step.R, 100)
    g_k = capture(step.out_gemv, n_k, stream)
    k_sp = spread(timer.trials(g_k.replay, n_k))
    ksec = k_sp["median_us"] * 1e-6
    achieved = step.out_gemv_bytes / ksec / 1e9
    src_hash = kernel_source_hash()
    traffic = load_traffic("qgemv_q8_0_4096x8192", src_hash)
    ceil = read_ceilings(qg, torch, stream, timer, step.W_host.nbytes)
    floor_us = ceil["read_same_bytes"]["median_us"]

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {
            "workload": "Q8_0 attention projections, batch 1: quantize + out 8192->4096 + quantize + paired "
                        "4096->1024 & 4096->512 (one launch)",
            "tokens_per_step": 1,
            "algorithmic_bytes_per_step": step.step_bytes,
            "weight_rotation_copies": step.R,
            "us_per_step": round(ms_per_step * 1e3, 3),
            "step_spread": step_sp,
            "hbm_frac_of_peak": round(value / HBM_PEAK_GBS, 4),
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "qgemv_q8_0 N=4096 K=8192 M=1",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "avg_launch_us": round(ksec * 1e6, 3),
            "launch_spread": k_sp,
            "algorithmic_bytes_per_launch": step.out_gemv_bytes,
            "read_ceiling_gbs": ceil["read_1gib"]["GB_s"],
            "frac_of_read_ceiling": round(achieved / ceil["read_1gib"]["GB_s"], 4),
            "read_floor_same_bytes_us": floor_us,
            "frac_of_read_floor": round(floor_us / (ksec * 1e6), 4),
            "read_probe": ceil,
            "source_hash": src_hash,
        },
    }
    g_f = capture(step.step_fused, args.steps, stream)
    fsp = spread(timer.trials(g_f.replay, args.steps))
    del g_steps, g_k, g_f
    result["config"]["fused_quantize_step_us"] = fsp["median_us"]
    if not args.no_extra:
        result["extra"] = extra_measurements(qg, torch, stream, timer)
    result["clocks"] = {"before": clocks_before, "after": gpu_clocks()}
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(step)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
