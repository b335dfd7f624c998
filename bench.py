"""Benchmark of the W8A8 INT8 linear layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--secondary decode,group128,group128_act,w8a16,rmsnorm_quant,
                                 m_sweep | none]
                    [--calibrate-copy]

A step is one pass of the W8A8 hot path over the prefill workload
(X bf16 [8192, 5120] after the smoothing fold, W int8 [15360, 5120] with
per-channel scales): per-token quantization of X (row absmax -> scale ->
codes) followed by the INT8 x INT8 -> INT32 GEMM with the per-token x
per-channel epilogue to bf16, both through the library's one-call entry
point.  Inputs (synthetic, seeded) are resident in HBM before timing; the
weight quantization and the fold are offline preparation, outside the timed
region.  Prints one JSON line:
  value    = 2*M*N*K*steps / elapsed  (TOPS, whole quant+GEMM step)
  roofline = the GEMM kernel alone, timed with events on the launch stream,
             against the INT8 dense MFMA peak (5.0 POP/s)
  cpu_baseline = the CPU oracle on a bounded sample of the same workload
  secondary    = decode (M=1, M=8) GB/s of the one-call layer with the weight
             copies rotated past the 256 MB last-level cache, and the other
             workloads
--calibrate-copy adds a plain device-to-device copy of 512 MiB (torch's copy
kernel), so that a hardware-counter run of this script also measures the
bytes the counters report for a transfer of known size.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402
import w8a8_int8_gemm_token_amd as q8  # noqa: E402

METRIC = "W8A8 quant+GEMM TOPS at M=8192,K=5120,N=15360; % INT8 MFMA peak; M=8 GB/s"
PEAK_INT8_TOPS = 5000.0   # MI355X dense INT8 MFMA, published
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense BF16 MFMA, published
PEAK_FP8_TFLOPS = 5000.0   # MI355X dense FP8 MFMA, published
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E, published


# HBM bytes of the prefill GEMM from hardware counters (rocprofv3 --pmc
# FETCH_SIZE, then WRITE_SIZE, KiB per dispatch, mean over the dispatches of
# gemm_big_kernel<EPI_CHANNEL> in a short bench run), scaled by what the same
# counters read for a plain 512 MiB device copy.  Valid only for the kernel
# sources they were taken on: if those files change, the figure is withdrawn
# (null).
GEMM_COUNTERS = {
    "sources_sha256": {
        "gemm_big.hpp": "86785bac67fcdcaaf077878f83390f6fc1805d1d3c6b704b21311aa69f3681a1",
        "gemm_i8.hpp": "cd18b8b57aa890022611210e3ae06f99127a3762c9173ed154adcd2b6d701081",
        "q8_device.hpp": "93921317d9ee2061ee8f6a130188921aef7ffc81f9e84a6867f9e2ea825e1a33",
    },
    "fetch_kib": 367721.7, "write_kib": 261641.9,
    "copy_kib": 524288.0, "copy_fetch_kib": 262155.5, "copy_write_kib": 524288.0,
}


def gemm_traffic():
    """(read bytes, write bytes) per GEMM launch, or None if stale."""
    csrc = os.path.join(ROOT, "w8a8_int8_gemm_token_amd", "csrc")
    for name, digest in GEMM_COUNTERS["sources_sha256"].items():
        with open(os.path.join(csrc, name), "rb") as f:
            if hashlib.sha256(f.read()).hexdigest() != digest:
                return None
    c = GEMM_COUNTERS
    rd = c["fetch_kib"] * 1024 * c["copy_kib"] / c["copy_fetch_kib"]
    wr = c["write_kib"] * 1024 * c["copy_kib"] / c["copy_write_kib"]
    return rd, wr


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _events_once(fn, iters: int) -> float:
    s = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(iters):
        fn()
    e1.record(s)
    e1.synchronize()
    return e0.elapsed_time(e1) / iters


def events_time(fn, iters: int, settle_ms: float = 60.0) -> float:
    """Average ms per call of fn() over iters calls, HIP events on the
    current stream (the stream the library launches on).  fn first runs for
    about settle_ms of GPU time, untimed, so that the clocks the board
    settles at under this load are the ones measured."""
    t1 = _events_once(fn, 1)
    for _ in range(int(min(5000, max(1, settle_ms / max(t1, 1e-3))))):
        fn()
    s = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(iters):
        fn()
    e1.record(s)
    e1.synchronize()
    return e0.elapsed_time(e1) / iters


def prefill_setup(dev):
    wl = synth.WORKLOADS["prefill"]
    x = synth.activations(wl, 0).to(dev)
    w = synth.weights(wl, 0).to(dev)
    xo, wo, _ = q8.q8_smooth_fold(x, w)
    del x, w
    wq, sc = q8.q8_quant_weight(wo)
    del wo
    torch.cuda.synchronize()
    return wl, xo, wq, sc


def cpu_baseline(target_s: float = 15.0):
    """The oracle (as it stands) on a bounded sample of the prefill workload:
    quantize a block of token rows and run the scaled INT8 GEMM for them
    against all 15360 channels.  Scaled to TOPS like the GPU figure."""
    import oracle
    wl = synth.WORKLOADS["prefill"]
    x = synth.bf16_bits(synth.activations(wl, 0))
    w = synth.weights(wl, 0).numpy()
    s = oracle.smooth_scales(x)
    xo = oracle.smooth_fold_x(x, s)
    wq, sc = oracle.quant_weight(oracle.smooth_fold_w(w, s))
    del w

    def run(rows):
        t0 = time.perf_counter()
        xq, st = oracle.quant_per_token(np.ascontiguousarray(xo[:rows]))
        oracle.scaled_mm(xq, wq, st, sc)
        return time.perf_counter() - t0

    rows = 16
    t = run(rows)
    while t < 1.0 and rows < wl.M:  # grow until the per-row cost is steady
        rows = min(wl.M, rows * 4)
        t = run(rows)
    rows = int(max(16, min(wl.M, rows * target_s / t)))
    t = run(rows)
    ops = 2.0 * rows * wl.N * wl.K
    threads = oracle.threads()
    return {"value": ops / t / 1e12, "unit": "TOPS", "cores": threads, "kind": "oracle",
            "sample": f"{rows} of {wl.M} token rows x all {wl.N} channels, K={wl.K} "
                      f"(quant + INT32 GEMM + epilogue), {t:.1f} s"}


def decode_gbs(dev, reps=20):
    """Fused quant+GEMM at M in {1, 8}: algorithmic bytes / kernel time.
    The calls cycle through enough weight copies that one cycle exceeds 2x
    the 256 MB last-level cache, and are captured in a HIP graph so that the
    events time the kernels back to back rather than the host's launch
    rate."""
    wl = synth.WORKLOADS["decode"]
    w = synth.weights(wl, 0).to(dev)
    wq, sc = q8.q8_quant_weight(w)
    del w
    ncopy = 24  # 24 x 26.2 MB = 629 MB
    wqs = [wq.clone() for _ in range(ncopy)]
    out = {}
    for M in (1, 8):
        x = synth.activations(wl, 0, M=M).to(dev)
        y = torch.empty((M, wl.N), dtype=torch.bfloat16, device=dev)
        xq = torch.empty((M, wl.K), dtype=torch.int8, device=dev)
        st = torch.empty((M,), dtype=torch.float32, device=dev)

        def cycle():
            for i in range(ncopy):
                q8.q8_quant_scaled_mm(x, wqs[i], sc, out=y, xq_out=xq, scale_tok_out=st)

        cycle()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            cycle()
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        ms = events_time(g.replay, reps) / ncopy
        nbytes = wl.N * wl.K + 4 * wl.N + 2 * M * wl.K + 2 * M * wl.N + 4 * M + M * wl.K
        out[f"M{M}"] = {"us": ms * 1e3, "GB/s": nbytes / (ms * 1e-3) / 1e9,
                        "frac_hbm": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                        "bytes": nbytes, "timing": "HIP graph of 24 calls, events"}
    return out


def group_tops(dev, iters=20):
    wl = synth.WORKLOADS["group128"]
    x = synth.activations(wl, 0).to(dev)
    w = synth.weights(wl, 0).to(dev)
    wq, sg = q8.q8_quant_weight(w, group=128)
    xq, st = q8.q8_quant_per_token(x)
    y = torch.empty((wl.M, wl.N), dtype=torch.bfloat16, device=dev)
    f = lambda: q8.q8_scaled_mm_group128(xq, wq, st, sg, out=y)  # noqa: E731
    for _ in range(3):
        f()
    ms = events_time(f, iters)
    t = 2.0 * wl.M * wl.N * wl.K / (ms * 1e-3) / 1e12
    return {"us": ms * 1e3, "TOPS": t, "frac_int8_peak": t / PEAK_INT8_TOPS}


def w8a16_tflops(dev, iters=20):
    wl = synth.WORKLOADS["w8a16"]
    x = synth.activations(wl, 0).to(dev)
    w = synth.weights(wl, 0).to(dev)
    wq, sc = q8.q8_quant_weight(w)
    del w
    y = torch.empty((wl.M, wl.N), dtype=torch.bfloat16, device=dev)
    f = lambda: q8.w8a16_mm(x, wq, sc, out=y)  # noqa: E731
    for _ in range(5):
        f()
    ms = events_time(f, iters)
    t = 2.0 * wl.M * wl.N * wl.K / (ms * 1e-3) / 1e12
    return {"us": ms * 1e3, "TFLOPS": t, "frac_bf16_peak": t / PEAK_BF16_TFLOPS}


def copy_calibration(dev, nbytes=512 << 20, reps=3):
    """A plain copy of known size, for scaling the HBM byte counters."""
    a = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    b = torch.empty_like(a)
    ms = events_time(lambda: b.copy_(a), reps)
    return {"bytes_read": nbytes, "bytes_written": nbytes, "us": ms * 1e3,
            "GB/s": 2 * nbytes / (ms * 1e-3) / 1e9}


def quant_after(quant, before, iters: int) -> float:
    """Median time (ms) of quant() measured with events on the launch stream
    when each call follows a call of before() (whose traffic evicts quant's
    input from the caches, as in the step)."""
    s = torch.cuda.current_stream()
    for _ in range(3):
        before()
        quant()
    s.synchronize()
    ev = []
    for _ in range(iters):
        before()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        quant()
        e1.record(s)
        ev.append((e0, e1))
    s.synchronize()
    ts = sorted(a.elapsed_time(b) for a, b in ev)
    return ts[len(ts) // 2]


def rmsnorm_quant_gbs(dev, iters=20):
    """Residual add + RMSNorm + per-token quant at the prefill shape: bytes
    = x read + residual read and write + codes + scales (+ gamma), over the
    kernel time (events)."""
    wl = synth.WORKLOADS["prefill"]
    x = synth.activations(wl, 0).to(dev)
    res = synth.activations(wl, 1).to(dev)
    gam = torch.ones((wl.K,), dtype=torch.bfloat16, device=dev)
    xq = torch.empty((wl.M, wl.K), dtype=torch.int8, device=dev)
    st = torch.empty((wl.M,), dtype=torch.float32, device=dev)
    f = lambda: q8.q8_rmsnorm_quant(x, gam, 1e-6, residual=res, out=xq, scale_out=st)  # noqa: E731
    for _ in range(3):
        f()
    ms = events_time(f, iters)
    nbytes = 2 * wl.M * wl.K * 3 + wl.M * wl.K + 4 * wl.M + 2 * wl.K
    return {"us": ms * 1e3, "GB/s": nbytes / (ms * 1e-3) / 1e9,
            "frac_hbm": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, "bytes": nbytes,
            "shape": [wl.M, wl.K]}


def group_act_tops(dev, iters=20):
    """Per-token-per-group activation quant + the GEMM with both block
    scales, at the group-128 workload shape."""
    wl = synth.WORKLOADS["group128"]
    x = synth.activations(wl, 0).to(dev)
    w = synth.weights(wl, 0).to(dev)
    wq, sw = q8.q8_quant_weight(w, group=128)
    del w
    xq, sx = q8.q8_quant_per_group128(x)
    y = torch.empty((wl.M, wl.N), dtype=torch.bfloat16, device=dev)
    g = lambda: q8.q8_scaled_mm_group128_act(xq, wq, sx, sw, out=y)  # noqa: E731
    qf = lambda: q8.q8_quant_per_group128(x, out=xq, scale_out=sx)  # noqa: E731
    for _ in range(3):
        qf()
        g()
    gms = events_time(g, iters)
    qms = events_time(qf, iters)
    t = 2.0 * wl.M * wl.N * wl.K / (gms * 1e-3) / 1e12
    qbytes = 3 * wl.M * wl.K + 4 * wl.M * (wl.K // 128)
    return {"gemm_us": gms * 1e3, "TOPS": t, "frac_int8_peak": t / PEAK_INT8_TOPS,
            "quant_us": qms * 1e3, "quant_GB/s": qbytes / (qms * 1e-3) / 1e9}


def fp8_block_tflops(dev, iters=20):
    """FP8 block W8A8 at the prefill shape: per-token-per-group E4M3
    activation quant + the [128,128] block-scaled FP8 GEMM.  GEMM, quant and
    the whole step are timed separately with events."""
    wl = synth.WORKLOADS["fp8_block"]
    x = synth.activations(wl, 0).to(dev)
    w = synth.weights(wl, 0).to(dev)
    xo, wo, _ = q8.q8_smooth_fold(x, w)
    del x, w
    wq, sw = q8.q8_quant_weight_fp8_block128(wo)
    del wo
    xq, sx = q8.q8_quant_fp8_per_group128(xo)
    y = torch.empty((wl.M, wl.N), dtype=torch.bfloat16, device=dev)
    g = lambda: q8.q8_fp8_block_scaled_mm(xq, wq, sx, sw, out=y)  # noqa: E731
    qf = lambda: q8.q8_quant_fp8_per_group128(xo, out=xq, scale_out=sx)  # noqa: E731

    def step():
        qf()
        g()
    for _ in range(5):
        step()
    gms = events_time(g, iters)
    qms = events_time(qf, iters)
    sms = events_time(step, iters)
    flops = 2.0 * wl.M * wl.N * wl.K
    t = flops / (gms * 1e-3) / 1e12
    qbytes = 3 * wl.M * wl.K + 4 * wl.M * (wl.K // 128)
    return {"gemm_us": gms * 1e3, "TFLOPS": t, "frac_fp8_peak": t / PEAK_FP8_TFLOPS,
            "quant_us": qms * 1e3, "quant_GB/s": qbytes / (qms * 1e-3) / 1e9,
            "step_us": sms * 1e3, "step_TFLOPS": flops / (sms * 1e-3) / 1e12,
            "shape": [wl.M, wl.N, wl.K]}


def f16_layer(dev, iters=20):
    """The fp16 variant of the one-call layer (fp16 in, fp16 out): the
    prefill shape timed with events, and M=8 decode per call in a HIP graph
    over weight copies (as the bf16 decode line); then the weight-only GEMM
    with fp16 activations at the W8A16 shape (fp16 MFMA peak = bf16's)."""
    wl = synth.WORKLOADS["prefill"]
    x = synth.activations(wl, 0).to(dev).half()
    w = synth.weights(wl, 0).to(dev)
    wq, sc = q8.q8_quant_weight(w)
    del w
    y = torch.empty((wl.M, wl.N), dtype=torch.float16, device=dev)
    xq = torch.empty((wl.M, wl.K), dtype=torch.int8, device=dev)
    st = torch.empty((wl.M,), dtype=torch.float32, device=dev)
    f = lambda: q8.q8_quant_scaled_mm_f16(x, wq, sc, out=y, xq_out=xq, scale_tok_out=st)  # noqa: E731
    for _ in range(5):
        f()
    ms = events_time(f, iters)
    ops = 2.0 * wl.M * wl.N * wl.K
    out = {"prefill": {"us": ms * 1e3, "TOPS": ops / (ms * 1e-3) / 1e12}}
    del y, xq, st, wq, sc, x
    dw = synth.WORKLOADS["decode"]
    w = synth.weights(dw, 0).to(dev)
    wq, sc = q8.q8_quant_weight(w)
    del w
    ncopy = 24
    wqs = [wq.clone() for _ in range(ncopy)]
    M = 8
    x = synth.activations(dw, 0, M=M).to(dev).half()
    y = torch.empty((M, dw.N), dtype=torch.float16, device=dev)
    xq = torch.empty((M, dw.K), dtype=torch.int8, device=dev)
    st = torch.empty((M,), dtype=torch.float32, device=dev)

    def cycle():
        for i in range(ncopy):
            q8.q8_quant_scaled_mm_f16(x, wqs[i], sc, out=y, xq_out=xq, scale_tok_out=st)
    cycle()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cycle()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    ms = events_time(g.replay, 20) / ncopy
    nbytes = dw.N * dw.K + 4 * dw.N + 2 * M * dw.K + 2 * M * dw.N + 4 * M + M * dw.K
    out["decode_M8"] = {"us": ms * 1e3, "GB/s": nbytes / (ms * 1e-3) / 1e9,
                        "timing": "HIP graph of 24 calls, events"}
    del wqs, wq, sc, x, y, xq, st
    # the weight-only GEMM with fp16 activations at the W8A16 workload shape
    ww = synth.WORKLOADS["w8a16"]
    x = synth.activations(ww, 0).to(dev).half()
    w = synth.weights(ww, 0).to(dev)
    wq, sc = q8.q8_quant_weight(w)
    del w
    y = torch.empty((ww.M, ww.N), dtype=torch.float16, device=dev)
    f = lambda: q8.w8a16_mm_f16(x, wq, sc, out=y)  # noqa: E731
    for _ in range(5):
        f()
    ms = events_time(f, iters)
    t = 2.0 * ww.M * ww.N * ww.K / (ms * 1e-3) / 1e12
    out["w8a16_prefill"] = {"us": ms * 1e3, "TFLOPS": t, "frac_fp16_peak": t / PEAK_BF16_TFLOPS,
                            "shape": [ww.M, ww.N, ww.K]}
    return out


# The model's Linear shapes (hidden 5120, intermediate 17408): W8A8 modules
# (q/k/v-like 15360 x 5120, gate/up 17408 x 5120, o-like 5120 x 5120) and
# the W8A16 down projection (5120 x 17408).
SWEEP_SHAPES = (("qkv", "w8a8", 15360, 5120), ("gate_up", "w8a8", 17408, 5120),
                ("o_proj", "w8a8", 5120, 5120), ("down_proj", "w8a16", 5120, 17408))
SWEEP_M = (1, 2, 4, 8, 16, 32, 64, 96, 128, 256)


def m_sweep(dev, reps=10):
    """Per-call time of each model shape at small token counts (decode,
    speculative verify, small batches): calls cycle through enough weight
    copies to exceed 2x the 256 MB last-level cache, captured in a HIP graph.
    GB/s counts the weights, scales, activations and outputs once."""
    out = {}
    for name, kind, N, K in SWEEP_SHAPES:
        w = synth.weights(synth.WORKLOADS["decode"], 0, N=N, K=K).to(dev)
        wq, sc = q8.q8_quant_weight(w)
        del w
        ncopy = max(2, -(-600_000_000 // (N * K)))
        wqs = [wq] + [wq.clone() for _ in range(ncopy - 1)]
        row = {}
        for M in SWEEP_M:
            x = synth.activations(synth.WORKLOADS["decode"], 0, M=M, K=K).to(dev)
            y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            if kind == "w8a8":
                xq = torch.empty((M, K), dtype=torch.int8, device=dev)
                st = torch.empty((M,), dtype=torch.float32, device=dev)

                def call(wi):
                    q8.q8_quant_scaled_mm(x, wi, sc, out=y, xq_out=xq, scale_tok_out=st)
                nbytes = N * K + 4 * N + 2 * M * K + M * K + 4 * M + 2 * M * N
            else:
                def call(wi):
                    q8.w8a16_mm(x, wi, sc, out=y)
                nbytes = N * K + 4 * N + 2 * M * K + 2 * M * N

            def cycle():
                for wi in wqs:
                    call(wi)
            cycle()
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                cycle()
            g.replay()
            torch.cuda.synchronize()
            ms = events_time(g.replay, reps) / ncopy
            row[f"M{M}"] = {"us": round(ms * 1e3, 2), "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1)}
            del g
        out[f"{name} {kind} N={N} K={K}"] = row
        del wqs, wq
        torch.cuda.empty_cache()
    return out


SECONDARY = {"decode": lambda dev: decode_gbs(dev), "group128": lambda dev: group_tops(dev),
             "m_sweep": lambda dev: m_sweep(dev),
             "group128_act": lambda dev: group_act_tops(dev),
             "w8a16": lambda dev: w8a16_tflops(dev), "rmsnorm_quant": lambda dev: rmsnorm_quant_gbs(dev),
             "fp8_block": lambda dev: fp8_block_tflops(dev), "f16": lambda dev: f16_layer(dev)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--secondary",
                    default="decode,group128,group128_act,w8a16,rmsnorm_quant,fp8_block,f16,m_sweep",
                    help="comma list of secondary workloads, or 'none'")
    ap.add_argument("--calibrate-copy", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    q8.load()

    log("setup: prefill workload")
    wl, xo, wq, sc = prefill_setup(dev)
    M, N, K = wl.M, wl.N, wl.K
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    xq = torch.empty((M, K), dtype=torch.int8, device=dev)
    st = torch.empty((M,), dtype=torch.float32, device=dev)

    def step():
        q8.q8_quant_scaled_mm(xo, wq, sc, out=y, xq_out=xq, scale_tok_out=st)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ops = 2.0 * M * N * K
    value = ops * args.steps / elapsed / 1e12

    # dominant kernel (the INT8 GEMM) alone, events on the launch stream
    gemm = lambda: q8.q8_scaled_mm(xq, wq, st, sc, out=y)  # noqa: E731
    gemm_ms = events_time(gemm, args.steps)
    quant = lambda: q8.q8_quant_per_token(xo, out=xq, scale_out=st)  # noqa: E731
    quant_ms = events_time(quant, args.steps)
    achieved = ops / (gemm_ms * 1e-3) / 1e12
    quant_bytes = M * K * 2 + M * K + 4 * M
    traffic = gemm_traffic()
    algo_bytes = M * K + N * K + 4 * M + 4 * N + 2 * M * N
    roofline = {"bound": "mfma", "achieved": achieved, "peak": PEAK_INT8_TOPS,
                "unit": "TFLOP/s", "frac": achieved / PEAK_INT8_TOPS,
                "traffic": None if traffic is None else sum(traffic),
                "traffic_read_write": traffic, "algorithmic_bytes": algo_bytes,
                "kernel": "gemm_big_kernel (per-channel epilogue, 256 x 384 tiles)",
                "kernel_us": gemm_ms * 1e3}
    quant_step_ms = quant_after(quant, gemm, args.steps)
    secondary = {"quant_kernel": {"us": quant_ms * 1e3,
                                  "GB/s": quant_bytes / (quant_ms * 1e-3) / 1e9,
                                  "timing": "back to back, X left in the last-level cache",
                                  "in_step_us": quant_step_ms * 1e3,
                                  "in_step_GB/s": quant_bytes / (quant_step_ms * 1e-3) / 1e9,
                                  "in_step_timing": "each call right after a GEMM, as in the step: X read from HBM"}}
    names = [] if args.no_secondary or args.secondary == "none" else args.secondary.split(",")
    for name in names:
        if name not in SECONDARY:
            print(f"unknown secondary workload {name!r}", file=sys.stderr)
            sys.exit(2)
        log(f"secondary: {name}")
        secondary[name] = SECONDARY[name](dev)
    if args.calibrate_copy:
        log("copy calibration")
        secondary["copy_calibration"] = copy_calibration(dev)
    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        cpu = cpu_baseline()
    rec = {
        "metric": METRIC, "value": value, "unit": "TOPS", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": elapsed / args.steps * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "i8", "data": "synthetic",
        "config": {"workload": "prefill W8A8 linear: per-token quant + INT8 GEMM, "
                               "M=8192 K=5120 N=15360, bf16 out", "M": M, "K": K, "N": N},
        "frac_int8_peak": value / PEAK_INT8_TOPS,
        "roofline": roofline, "cpu_baseline": cpu, "secondary": secondary,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
