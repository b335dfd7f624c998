"""Benchmark of the W8A8 INT8 linear layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--secondary decode,tiny,group128,group128_act,w8a16,
                                 rmsnorm_quant,fp8_block,f16,m_sweep,codes_sweep,
                                 vendor | none]
                    [--calibrate-copy]

A step is one pass of the W8A8 hot path over the prefill workload
(X bf16 [8192, 5120] after the smoothing fold, W int8 [15360, 5120] with
per-channel scales): per-token quantization of X (row absmax -> scale ->
codes) followed by the INT8 x INT8 -> INT32 GEMM with the per-token x
per-channel epilogue to bf16 -- the two kernels the one-call entry point
q8_quant_scaled_mm launches at this size, called here as q8_quant_per_token
then q8_scaled_mm so that HIP events can mark the GEMM inside every timed
step.  Inputs (synthetic, seeded) are resident in HBM before timing; the
weight quantization and the fold are offline preparation, outside the timed
region.  Before the W warm-up steps the GEMM runs alone for about 60 ms
(the "gemm_alone" figure), which also brings the board from idle to the
clock it holds under this load.  Prints one JSON line:
  value    = 2*M*N*K*steps / elapsed  (TOPS, whole quant+GEMM step, host
             clock around the K timed steps)
  roofline = the GEMM kernel: its mean duration over the K timed steps from
             the events around it (on the stream it is launched on), against
             the INT8 dense MFMA peak (5.0 POP/s), with the ceiling an MFMA-only
             loop of the GEMM's instruction on changing operands reaches on
             the same board, and the
             same kernel at the same shape on all-zero and on small and
             full-range uniform codes (the clock the board holds depends on
             the operand values)
  cpu_baseline = the CPU oracle on a bounded sample of the same workload,
             and on each of the other four workloads (per_config)
  secondary    = decode (M=1, M=8) per call in a HIP graph with the weight
             copies rotated past the 256 MB last-level cache, against 8 TB/s
             and against a plain read of the same bytes in the same protocol;
             the tiny workload's latency; the measured ceilings; the
             other workloads (p10/p50/p90 of per-call event times); and the
             vendor BLAS (hipBLASLt through torch) on plain GEMMs of the
             same shapes, for context
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
# gemm_big16_kernel<EPI_CHANNEL> in a short bench run), scaled by what the same
# counters read for a plain 512 MiB device copy.  Valid only for the kernel
# sources they were taken on: if those files change, the figure is withdrawn
# (null).
GEMM_COUNTERS = {
    "sources_sha256": {
        "gemm_big.hpp": "4b40e4a66dba685d115c6e7bec3da3edea697ca0b44b19007a54a00db6822588",
        "gemm_i8.hpp": "cda32a4092af89f146b4cf1525ebbcdd0e8e91839f7c3688837cde37d5078a24",
        "q8_device.hpp": "ccd2b93eca43b76b27e87299ed951a8a59342afdb931f850f87bdacbbe91dfc2",
    },
    "fetch_kib": 363672.6, "write_kib": 245837.2,
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


def call_stats(fn, iters: int, settle_ms: float = 60.0) -> dict:
    """Per-call times of fn() (ms), each call between its own pair of HIP
    events on the current stream, after about settle_ms of untimed calls:
    mean, p10, p50, p90."""
    t1 = _events_once(fn, 1)
    for _ in range(int(min(5000, max(1, settle_ms / max(t1, 1e-3))))):
        fn()
    s = torch.cuda.current_stream()
    ev = []
    for _ in range(iters):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        fn()
        e1.record(s)
        ev.append((e0, e1))
    s.synchronize()
    t = np.array([a.elapsed_time(b) for a, b in ev])
    return {"mean": float(t.mean()), "p10": float(np.percentile(t, 10)),
            "p50": float(np.percentile(t, 50)), "p90": float(np.percentile(t, 90))}


def gemm_operand_values(dev, M: int, N: int, K: int, sc, st, y, iters: int) -> dict:
    """The prefill GEMM kernel on the same shape with other operand values:
    all-zero codes, and codes drawn uniformly from [-4, 4] and from
    [-127, 127] (seeded).  The instructions, addresses and traffic are the
    same in every case; what changes is the switching in the matrix cores,
    so the board holds another clock.  Per-call times like gemm_alone."""
    g = torch.Generator(device=dev)
    out = {}
    for name, lim in (("zero", 0), ("uniform_pm4", 4), ("uniform_pm127", 127)):
        g.manual_seed(7)
        xq = torch.randint(-lim, lim + 1, (M, K), dtype=torch.int8, device=dev, generator=g)
        wq = torch.randint(-lim, lim + 1, (N, K), dtype=torch.int8, device=dev, generator=g)
        st_ = call_stats(lambda: q8.q8_scaled_mm(xq, wq, st, sc, out=y), iters)
        out[name] = dict(_us(st_), TOPS=2.0 * M * N * K / (st_["p50"] * 1e-3) / 1e12)
        del xq, wq
    torch.cuda.empty_cache()
    return out


def _us(st: dict) -> dict:
    return {k: round(v * 1e3, 3) for k, v in st.items()}


_ceil = None


def ceil_lib():
    """The benchmark's measurement kernels (libq8_ceilings.so)."""
    global _ceil
    if _ceil is None:
        import ctypes
        path = os.path.join(ROOT, "w8a8_int8_gemm_token_amd", "libq8_ceilings.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} not built (python -m w8a8_int8_gemm_token_amd.build)")
        lib = ctypes.CDLL(path)
        P, I, C = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        lib.q8c_mfma_i8_loop.argtypes = [C, C, C, P, P]
        lib.q8c_mfma_i8_loop.restype = C
        lib.q8c_mfma_i8_loop16.argtypes = [C, C, C, P, P]
        lib.q8c_mfma_i8_loop16.restype = C
        lib.q8c_stream_read.argtypes = [P, I, C, P, P]
        lib.q8c_stream_read.restype = C
        _ceil = lib
    return _ceil


def _stream_ptr():
    import ctypes
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def mfma_ceiling(dev, random: bool, iters: int = 16384, reps: int = 10, form: str = "32x32x32") -> dict:
    """int8 MFMA rate of a loop of v_mfma_i32_32x32x32_i8 (four chains per
    wave) or v_mfma_i32_16x16x64_i8 (eight chains) from registers (no
    memory traffic): 768 workgroups of 4 waves (3 waves per SIMD, all
    resident); operands changing every MFMA (random) or all zero."""
    import ctypes
    lib = ceil_lib()
    blocks = 768
    out = torch.empty(blocks * 256, dtype=torch.int32, device=dev)
    fn = lib.q8c_mfma_i8_loop if form == "32x32x32" else lib.q8c_mfma_i8_loop16

    def f():
        rc = fn(blocks, iters, int(random), ctypes.c_void_p(out.data_ptr()), _stream_ptr())
        if rc != 0:
            raise RuntimeError(f"MFMA loop failed ({rc})")
    ms = events_time(f, reps)
    # per wave: 4 chains of 32x32x32 (65536 ops each) or 8 of 16x16x64 (32768)
    ops = blocks * 4 * iters * (4 * 65536.0 if form == "32x32x32" else 8 * 32768.0)
    return {"TOPS": ops / (ms * 1e-3) / 1e12, "ms": ms, "operands": "random" if random else "zero",
            "form": form}


def read_ceiling_graph(dev, nbytes: int, ncopy: int = 24, reps: int = 20) -> dict:
    """A plain read of nbytes per call, cycling through ncopy buffers (past
    the 256 MB last-level cache), captured in a HIP graph and timed per call
    with events: the decode line's protocol with the layer replaced by a
    bare read.  The fastest of a few grid sizes is kept."""
    import ctypes
    lib = ceil_lib()
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(i % 251) for i in range(ncopy)]
    best = None
    for blocks in (512, 1024, 2048, 4096):
        out = torch.empty(blocks * 256, dtype=torch.int32, device=dev)

        def cycle():
            for b in bufs:
                rc = lib.q8c_stream_read(ctypes.c_void_p(b.data_ptr()), nbytes, blocks,
                                         ctypes.c_void_p(out.data_ptr()), _stream_ptr())
                if rc != 0:
                    raise RuntimeError(f"q8c_stream_read failed ({rc})")
        cycle()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            cycle()
        g.replay()
        torch.cuda.synchronize()
        ms = events_time(g.replay, reps) / ncopy
        if best is None or ms < best[0]:
            best = (ms, blocks)
        del g
    ms, blocks = best
    return {"us": ms * 1e3, "GB/s": nbytes / (ms * 1e-3) / 1e9, "bytes": nbytes, "blocks": blocks,
            "timing": f"HIP graph of {ncopy} calls on distinct buffers, events"}


def read_ceiling_big(dev, nbytes: int = 512 << 20, reps: int = 10) -> dict:
    """A plain read of one 512 MiB buffer (twice the last-level cache),
    events per call."""
    import ctypes
    lib = ceil_lib()
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(3)
    blocks = 4096
    out = torch.empty(blocks * 256, dtype=torch.int32, device=dev)

    def f():
        rc = lib.q8c_stream_read(ctypes.c_void_p(buf.data_ptr()), nbytes, blocks,
                                 ctypes.c_void_p(out.data_ptr()), _stream_ptr())
        if rc != 0:
            raise RuntimeError(f"q8c_stream_read failed ({rc})")
    ms = events_time(f, reps)
    return {"us": ms * 1e3, "GB/s": nbytes / (ms * 1e-3) / 1e9, "bytes": nbytes}


_CEILINGS = {}


def ceilings(dev) -> dict:
    """The board's measured ceilings: int8 MFMA on changing and on zero
    operands, and plain reads (the decode protocol's 26,398,752 bytes per
    call over 24 buffers, and one 512 MiB buffer)."""
    if not _CEILINGS:
        _CEILINGS["mfma_int8_random"] = mfma_ceiling(dev, True)
        _CEILINGS["mfma_int8_zero"] = mfma_ceiling(dev, False)
        _CEILINGS["mfma_int8_16x16x64_random"] = mfma_ceiling(dev, True, form="16x16x64")
        _CEILINGS["mfma_int8_16x16x64_zero"] = mfma_ceiling(dev, False, form="16x16x64")
        _CEILINGS["read_decode_bytes_graph"] = read_ceiling_graph(dev, 26_398_752)
        _CEILINGS["read_512MiB"] = read_ceiling_big(dev)
        torch.cuda.empty_cache()
    return dict(_CEILINGS)


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


def cpu_model() -> str | None:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _timed(fn) -> float:
    t0 = time.perf_counter()
    fn()
    return time.perf_counter() - t0


def _rows_for(run, total_rows: int, target_s: float) -> tuple[int, float]:
    """Grow a row block until its time is steady, then size it to about
    target_s of oracle work; returns (rows, seconds of the sized run)."""
    rows = 16
    t = run(rows)
    while t < 0.5 and rows < total_rows:
        rows = min(total_rows, rows * 4)
        t = run(rows)
    rows = int(max(16, min(total_rows, rows * target_s / t)))
    return rows, run(rows)


def cpu_baseline(target_s: float = 10.0):
    """The oracle (as it stands) on the host cores: on a bounded sample of
    the prefill workload (a block of token rows quantized and multiplied
    against all 15360 channels, sized to about target_s), and on the other
    four workloads (tiny and decode whole, median of 5; W8A16 and group-128
    on a row block of about 5 s).  Scaled to the unit of the GPU figures."""
    import oracle
    wl = synth.WORKLOADS["prefill"]
    x = synth.bf16_bits(synth.activations(wl, 0))
    w = synth.weights(wl, 0).numpy()
    s = oracle.smooth_scales(x)
    xo = oracle.smooth_fold_x(x, s)
    wq, sc = oracle.quant_weight(oracle.smooth_fold_w(w, s))
    del w, x

    def run(rows):
        def f():
            xq, st = oracle.quant_per_token(np.ascontiguousarray(xo[:rows]))
            oracle.scaled_mm(xq, wq, st, sc)
        return _timed(f)

    rows, t = _rows_for(run, wl.M, target_s)
    ops = 2.0 * rows * wl.N * wl.K
    threads = oracle.threads()
    rec = {"value": ops / t / 1e12, "unit": "TOPS", "cores": threads, "kind": "oracle",
           "sample": f"{rows} of {wl.M} token rows x all {wl.N} channels, K={wl.K} "
                     f"(quant + INT32 GEMM + epilogue), {t:.1f} s",
           "cpu_model": cpu_model()}
    del xo, wq, sc
    per = {}
    for name in ("tiny", "decode"):
        wk = synth.WORKLOADS[name]
        xb = synth.bf16_bits(synth.activations(wk, 0))
        wq_, sc_ = oracle.quant_weight(synth.weights(wk, 0).numpy())

        def f():
            xq_, st_ = oracle.quant_per_token(xb)
            oracle.scaled_mm(xq_, wq_, st_, sc_)
        t = float(np.median([_timed(f) for _ in range(5)]))
        nbytes = wk.N * wk.K + 4 * wk.N + 3 * wk.M * wk.K + 4 * wk.M + 2 * wk.M * wk.N
        per[name] = {"us": t * 1e6, "TOPS": 2.0 * wk.M * wk.N * wk.K / t / 1e12,
                     "GB/s": nbytes / t / 1e9, "sample": f"whole workload {wk.M}x{wk.N}x{wk.K}, median of 5"}
    wk = synth.WORKLOADS["w8a16"]
    xb = synth.bf16_bits(synth.activations(wk, 0))
    wq_, sc_ = oracle.quant_weight(synth.weights(wk, 0).numpy())
    rows, t = _rows_for(lambda r: _timed(lambda: oracle.w8a16_ref(np.ascontiguousarray(xb[:r]), wq_, sc_)),
                        wk.M, 5.0)
    per["w8a16"] = {"TFLOPS": 2.0 * rows * wk.N * wk.K / t / 1e12,
                    "sample": f"{rows} of {wk.M} rows x all {wk.N} channels, K={wk.K} (fp64 reference), {t:.1f} s"}
    del xb, wq_
    wk = synth.WORKLOADS["group128"]
    xb = synth.bf16_bits(synth.activations(wk, 0))
    wq_, sg_ = oracle.quant_weight(synth.weights(wk, 0).numpy(), group=128)

    def run_g(r):
        def f():
            xq_, st_ = oracle.quant_per_token(np.ascontiguousarray(xb[:r]))
            oracle.scaled_mm_group128(xq_, wq_, st_, sg_)
        return _timed(f)
    rows, t = _rows_for(run_g, wk.M, 5.0)
    per["group128"] = {"TOPS": 2.0 * rows * wk.N * wk.K / t / 1e12,
                       "sample": f"{rows} of {wk.M} rows x all {wk.N} channels, K={wk.K} "
                                 f"(quant + group-128 GEMM), {t:.1f} s"}
    rec["per_config"] = per
    return rec


def decode_gbs(dev, reps=20):
    """Fused quant+GEMM at M in {1, 8}: algorithmic bytes / kernel time,
    against 8 TB/s and against a plain read of the same bytes per call in
    the same protocol (the measured ceiling).
    The calls cycle through enough weight copies that one cycle exceeds 2x
    the 256 MB last-level cache, and are captured in a HIP graph so that the
    events time the kernels back to back rather than the host's launch
    rate."""
    ceil = ceilings(dev)["read_decode_bytes_graph"]
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
        st = call_stats(g.replay, reps)
        ms = st["mean"] / ncopy
        nbytes = wl.N * wl.K + 4 * wl.N + 2 * M * wl.K + 2 * M * wl.N + 4 * M + M * wl.K
        gbs = nbytes / (ms * 1e-3) / 1e9
        out[f"M{M}"] = {"us": ms * 1e3, "GB/s": gbs, "frac_hbm": gbs / PEAK_HBM_GBS,
                        "frac_read_ceiling": gbs / ceil["GB/s"],
                        "per_call_us_p10_p50_p90": [round(st[k] / ncopy * 1e3, 3) for k in ("p10", "p50", "p90")],
                        "bytes": nbytes, "timing": "HIP graph of 24 calls, events"}
        del g
    out["read_ceiling"] = {"us": ceil["us"], "GB/s": ceil["GB/s"], "bytes": ceil["bytes"],
                           "timing": ceil["timing"]}
    return out


def tiny_latency(dev, ncopy: int = 64, reps: int = 20):
    """The tiny workload (X [16,256], W [128,256]) through the one-call
    layer: per call inside a HIP graph of 64 calls (the kernels back to back),
    and per call launched from the host (events around each call)."""
    wl = synth.WORKLOADS["tiny"]
    x = synth.activations(wl, 0).to(dev)
    w = synth.weights(wl, 0).to(dev)
    wq, sc = q8.q8_quant_weight(w)
    y = torch.empty((wl.M, wl.N), dtype=torch.bfloat16, device=dev)
    xq = torch.empty((wl.M, wl.K), dtype=torch.int8, device=dev)
    st = torch.empty((wl.M,), dtype=torch.float32, device=dev)

    def call():
        q8.q8_quant_scaled_mm(x, wq, sc, out=y, xq_out=xq, scale_tok_out=st)

    def cycle():
        for _ in range(ncopy):
            call()
    cycle()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cycle()
    g.replay()
    torch.cuda.synchronize()
    gs = call_stats(g.replay, reps)
    es = call_stats(call, 200)
    return {"graph_us_per_call": gs["mean"] / ncopy * 1e3,
            "graph_us_per_call_p10_p50_p90": [round(gs[k] / ncopy * 1e3, 3) for k in ("p10", "p50", "p90")],
            "eager_us": _us(es), "shape": [wl.M, wl.N, wl.K],
            "timing": "HIP graph of 64 calls (per call), and per eager call between events"}


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
    st = call_stats(f, iters)
    ms = st["mean"]
    t = 2.0 * wl.M * wl.N * wl.K / (ms * 1e-3) / 1e12
    return {"us": ms * 1e3, "TOPS": t, "frac_int8_peak": t / PEAK_INT8_TOPS, "stats_us": _us(st)}


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
    st = call_stats(f, iters)
    ms = st["mean"]
    t = 2.0 * wl.M * wl.N * wl.K / (ms * 1e-3) / 1e12
    return {"us": ms * 1e3, "TFLOPS": t, "frac_bf16_peak": t / PEAK_BF16_TFLOPS, "stats_us": _us(st)}


def copy_calibration(dev, nbytes=512 << 20, reps=3):
    """A plain copy of known size, for scaling the HBM byte counters."""
    a = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    b = torch.empty_like(a)
    ms = events_time(lambda: b.copy_(a), reps)
    return {"bytes_read": nbytes, "bytes_written": nbytes, "us": ms * 1e3,
            "GB/s": 2 * nbytes / (ms * 1e-3) / 1e9}


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
    st = call_stats(f, iters)
    ms = st["mean"]
    nbytes = 2 * wl.M * wl.K * 3 + wl.M * wl.K + 4 * wl.M + 2 * wl.K
    return {"us": ms * 1e3, "GB/s": nbytes / (ms * 1e-3) / 1e9, "stats_us": _us(st),
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
    gst = call_stats(g, iters)
    gms = gst["mean"]
    qms = events_time(qf, iters)
    t = 2.0 * wl.M * wl.N * wl.K / (gms * 1e-3) / 1e12
    qbytes = 3 * wl.M * wl.K + 4 * wl.M * (wl.K // 128)
    return {"gemm_us": gms * 1e3, "TOPS": t, "frac_int8_peak": t / PEAK_INT8_TOPS, "gemm_stats_us": _us(gst),
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
    gst = call_stats(g, iters)
    gms = gst["mean"]
    qms = events_time(qf, iters)
    sms = events_time(step, iters)
    flops = 2.0 * wl.M * wl.N * wl.K
    t = flops / (gms * 1e-3) / 1e12
    qbytes = 3 * wl.M * wl.K + 4 * wl.M * (wl.K // 128)
    return {"gemm_us": gms * 1e3, "TFLOPS": t, "frac_fp8_peak": t / PEAK_FP8_TFLOPS, "gemm_stats_us": _us(gst),
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
    # the per-token quantizer alone, fp16 and bf16 rows side by side, at the
    # prefill width (10 chunks of 8 values per lane) and at K = 4096 (8)
    quant = {}
    for Kq in (wl.K, 4096):
        xh = x[:, :Kq].contiguous()
        xb = xh.to(torch.bfloat16)
        xq_ = torch.empty((wl.M, Kq), dtype=torch.int8, device=dev)
        for name, xx, fn in (("f16", xh, q8.q8_quant_per_token_f16), ("bf16", xb, q8.q8_quant_per_token)):
            qms = call_stats(lambda: fn(xx, out=xq_, scale_out=st), iters)["mean"]
            nb = 3 * wl.M * Kq + 4 * wl.M
            quant[f"{name}_K{Kq}"] = {"us": qms * 1e3, "GB/s": nb / (qms * 1e-3) / 1e9}
        del xh, xb, xq_
    out["quant_per_token"] = dict(quant, timing="back to back, rows left in the last-level cache")
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
SWEEP_M = (1, 2, 4, 8, 16, 32, 64, 96, 128, 192, 256, 384, 512)


def rotating_graph_us(fn, wqs, reps):
    """Per-call time of fn(w) over the weight copies wqs, one cycle captured
    in a HIP graph and replayed (launch gaps included)."""
    def cycle():
        for wi in wqs:
            fn(wi)
    cycle()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cycle()
    g.replay()
    torch.cuda.synchronize()
    us = events_time(g.replay, reps) / len(wqs) * 1e3
    del g
    return us


def m_sweep(dev, reps=10):
    """Per-call time of each model shape at 1-512 tokens (decode,
    speculative verify, small batches, chunks): calls cycle through enough
    weight copies to exceed 2x the 256 MB last-level cache, captured in a
    HIP graph.  Where the library splits K over a workspace, the _ws entry
    point is timed as well (ws_us).  GB/s counts the weights, scales,
    activations and outputs once."""
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
            wsb = q8.q8_workspace_bytes(M, N, K)
            ws = torch.empty((max(wsb, 1),), dtype=torch.uint8, device=dev)
            if kind == "w8a8":
                xq = torch.empty((M, K), dtype=torch.int8, device=dev)
                st = torch.empty((M,), dtype=torch.float32, device=dev)

                def call(wi):
                    q8.q8_quant_scaled_mm(x, wi, sc, out=y, xq_out=xq, scale_tok_out=st)

                def call_ws(wi):
                    q8.q8_quant_scaled_mm_ws(x, wi, sc, out=y, xq_out=xq, scale_tok_out=st, workspace=ws)
                nbytes = N * K + 4 * N + 2 * M * K + M * K + 4 * M + 2 * M * N
            else:
                def call(wi):
                    q8.w8a16_mm(x, wi, sc, out=y)

                def call_ws(wi):
                    q8.w8a16_mm_ws(x, wi, sc, out=y, workspace=ws)
                nbytes = N * K + 4 * N + 2 * M * K + 2 * M * N

            us = rotating_graph_us(call, wqs, reps)
            row[f"M{M}"] = {"us": round(us, 2), "GB/s": round(nbytes / (us * 1e-6) / 1e9, 1)}
            if wsb:  # K split over a workspace (the _ws entry point)
                us = rotating_graph_us(call_ws, wqs, reps)
                row[f"M{M}"].update({"ws_us": round(us, 2), "ws_GB/s": round(nbytes / (us * 1e-6) / 1e9, 1),
                                     "ws_bytes": wsb})
            del ws
        out[f"{name} {kind} N={N} K={K}"] = row
        del wqs, wq
        torch.cuda.empty_cache()
    return out


CODES_SHAPES = (("qkv", 15360, 5120), ("gate_up", 17408, 5120), ("o_proj", 5120, 5120),
                ("4096x4096", 4096, 4096), ("2048x8192", 2048, 8192))


def codes_sweep(dev, reps=10):
    """q8_scaled_mm on int8 codes that are already at hand (as after the
    fused RMSNorm + quantizer), per call at 1, 8 and 16 tokens, in the
    m_sweep protocol (rotating weight copies past the last-level cache, one
    cycle in a HIP graph): the model's W8A8 shapes and two narrower layers,
    where the decode-structured kernel on codes runs (N <= 4096)."""
    out = {}
    for name, N, K in CODES_SHAPES:
        w = synth.weights(synth.WORKLOADS["decode"], 0, N=N, K=K).to(dev)
        wq, sc = q8.q8_quant_weight(w)
        del w
        ncopy = max(2, -(-600_000_000 // (N * K)))
        wqs = [wq] + [wq.clone() for _ in range(ncopy - 1)]
        row = {}
        for M in (1, 8, 16):
            x = synth.activations(synth.WORKLOADS["decode"], 0, M=M, K=K).to(dev)
            xq, st = q8.q8_quant_per_token(x)
            y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            us = rotating_graph_us(lambda wi: q8.q8_scaled_mm(xq, wi, st, sc, out=y), wqs, reps)
            nbytes = N * K + 4 * N + M * K + 4 * M + 2 * M * N
            row[f"M{M}"] = {"us": round(us, 2), "GB/s": round(nbytes / (us * 1e-6) / 1e9, 1)}
        out[f"{name} N={N} K={K}"] = row
        del wqs, wq
        torch.cuda.empty_cache()
    return out


def vendor_gemms(dev, iters=20) -> dict:
    """The vendor BLAS (hipBLASLt, through torch's _int_mm, matmul and
    _scaled_mm) on this board at the workloads' shapes, timed like the
    layer's own lines (events per call after a settling run): plain INT8 x
    INT8 -> INT32 at the prefill and group-128 shapes (no scales, no
    quantizer), a plain bf16 GEMM at the W8A16 shape (no dequantization),
    and FP8 E4M3 with one scale per row and column at the FP8 block shape
    (no per-block fold).  Each does less than the layer's kernel at that
    shape; they are context, not the layer."""
    out = {"library": "hipBLASLt via torch (" + torch.__version__ + ")"}

    def run(name, f, flops):
        try:
            f()
            torch.cuda.synchronize()
            st = call_stats(f, iters)
            out[name] = {"us": round(st["p50"] * 1e3, 1), "TOPS": round(flops / (st["p50"] * 1e-3) / 1e12, 1),
                         "stats_us": _us(st)}
        except Exception as e:  # an op this torch build lacks
            out[name] = {"error": f"{type(e).__name__}: {str(e)[:120]}"}
    g = torch.Generator(device=dev).manual_seed(0)
    for name, key in (("int8_prefill", "prefill"), ("int8_group128_shape", "group128")):
        wl = synth.WORKLOADS[key]
        a = torch.randint(-127, 128, (wl.M, wl.K), dtype=torch.int8, device=dev, generator=g)
        b = torch.randint(-127, 128, (wl.N, wl.K), dtype=torch.int8, device=dev, generator=g)
        run(name, lambda: torch._int_mm(a, b.t()), 2.0 * wl.M * wl.N * wl.K)
        del a, b
    wl = synth.WORKLOADS["w8a16"]
    a = torch.randn((wl.M, wl.K), dtype=torch.bfloat16, device=dev, generator=g)
    b = torch.randn((wl.N, wl.K), dtype=torch.bfloat16, device=dev, generator=g)
    run("bf16_w8a16_shape", lambda: a @ b.t(), 2.0 * wl.M * wl.N * wl.K)
    del a, b
    wl = synth.WORKLOADS["fp8_block"]
    a = torch.randn((wl.M, wl.K), device=dev, generator=g).to(torch.float8_e4m3fn)
    b = torch.randn((wl.N, wl.K), device=dev, generator=g).to(torch.float8_e4m3fn)
    sa = torch.ones((wl.M, 1), device=dev)
    sb = torch.ones((1, wl.N), device=dev)
    run("fp8_rowwise_fp8_block_shape",
        lambda: torch._scaled_mm(a, b.t(), scale_a=sa, scale_b=sb, out_dtype=torch.bfloat16),
        2.0 * wl.M * wl.N * wl.K)
    del a, b
    torch.cuda.empty_cache()
    return out


SECONDARY = {"decode": lambda dev: decode_gbs(dev), "group128": lambda dev: group_tops(dev),
             "tiny": lambda dev: tiny_latency(dev),
             "m_sweep": lambda dev: m_sweep(dev), "codes_sweep": lambda dev: codes_sweep(dev),
             "group128_act": lambda dev: group_act_tops(dev),
             "w8a16": lambda dev: w8a16_tflops(dev), "rmsnorm_quant": lambda dev: rmsnorm_quant_gbs(dev),
             "fp8_block": lambda dev: fp8_block_tflops(dev), "f16": lambda dev: f16_layer(dev),
             "vendor": lambda dev: vendor_gemms(dev)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--secondary",
                    default="decode,tiny,group128,group128_act,w8a16,rmsnorm_quant,fp8_block,f16,m_sweep,"
                            "codes_sweep,vendor",
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
    quant = lambda: q8.q8_quant_per_token(xo, out=xq, scale_out=st)  # noqa: E731
    gemm = lambda: q8.q8_scaled_mm(xq, wq, st, sc, out=y)  # noqa: E731
    ops = 2.0 * M * N * K

    # the GEMM alone, events on the launch stream, after about 60 ms of
    # untimed calls: the board leaves its idle clock here, before the steps
    log("gemm alone")
    quant()
    gemm_alone = call_stats(gemm, args.steps)

    # events in the timed steps: one before the first step, then one after
    # each quantizer and one after each GEMM (the end of a step is the start
    # of the next), on the stream the library launches on
    s = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * args.steps + 1)]

    def step(i=None):
        quant()
        if i is not None:
            ev[2 * i + 1].record(s)
        gemm()
        if i is not None:
            ev[2 * i + 2].record(s)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    t0 = time.perf_counter()
    ev[0].record(s)
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    value = ops * args.steps / elapsed / 1e12
    quant_in = np.array([ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(args.steps)])
    gemm_in = np.array([ev[2 * i + 1].elapsed_time(ev[2 * i + 2]) for i in range(args.steps)])
    gemm_ms = float(gemm_in.mean())

    achieved = ops / (gemm_ms * 1e-3) / 1e12
    quant_bytes = M * K * 2 + M * K + 4 * M
    traffic = gemm_traffic()
    algo_bytes = M * K + N * K + 4 * M + 4 * N + 2 * M * N
    log("ceilings")
    ceil = ceilings(dev)
    mfma_ceil = ceil["mfma_int8_16x16x64_random"]["TOPS"]
    log("gemm on other operand values")
    operand_values = gemm_operand_values(dev, M, N, K, sc, st, y, args.steps)
    roofline = {"bound": "mfma", "achieved": achieved, "peak": PEAK_INT8_TOPS,
                "unit": "TFLOP/s", "frac": achieved / PEAK_INT8_TOPS,
                "traffic": None if traffic is None else sum(traffic),
                "traffic_read_write": traffic, "algorithmic_bytes": algo_bytes,
                "kernel": "gemm_big16_kernel (per-channel epilogue, 256 x 384 tiles, 16x16x64 int8 MFMA, one persistent workgroup per CU)",
                "kernel_us": gemm_ms * 1e3,
                "kernel_us_p10_p50_p90": [round(float(np.percentile(gemm_in, q)) * 1e3, 2) for q in (10, 50, 90)],
                "timing": "events around the GEMM inside each of the timed steps",
                "measured_ceiling": mfma_ceil, "frac_measured_ceiling": achieved / mfma_ceil,
                "measured_ceiling_kind": "int8 MFMA-only loop of the GEMM's instruction (16x16x64), "
                                         "operands changing every MFMA",
                "frac_256cu_2p4ghz_5033": achieved / 5033.2,
                "same_kernel_other_operand_values_us": operand_values}
    quant_step_ms = float(quant_in.mean())
    secondary = {"quant_kernel": {"in_step_us": quant_step_ms * 1e3,
                                  "in_step_GB/s": quant_bytes / (quant_step_ms * 1e-3) / 1e9,
                                  "in_step_timing": "events around the quantizer inside each timed step "
                                                    "(X read from HBM after the previous GEMM)"},
                 "gemm_alone": dict(_us(gemm_alone), TOPS=ops / (gemm_alone["mean"] * 1e-3) / 1e12,
                                    timing="events around each call, back to back, before the steps"),
                 "ceilings": ceil}
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
