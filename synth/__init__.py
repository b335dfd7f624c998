"""Seeded synthetic inputs for the W8A8 / W8A16 linear-layer workloads.

This module draws random numbers and nothing else: no scale, code, fold or
product of the method is computed here.  It is the only code shared by the
CPU oracle side and the HIP side of the tests and the benchmark.

Every tensor comes from numpy's PCG64 generator seeded by
``SeedSequence([seed, workload_id, tensor_tag])``; normals are
``standard_normal(dtype=float32)`` times sigma (one fp32 multiply), and the
activation matrix is then rounded to bf16 with torch's round-to-nearest-even
cast (bf16 is the activation dtype on the pages).

Workloads (shapes from the model facts on the pages: hidden 5120 is K of the
q/k/v/gate/up projections; 8192-token batched prefill chunks; decode batches of
at most 8 sequences):

  tiny      X [16,256]  ~N(0,1), channels 3 and 77 scaled x20;
            W [128,256] ~N(0,0.02)
  decode    X [8,5120]  ~N(0,1), 1% of channels (52) scaled x30;
            W [5120,5120] ~N(0,0.02)
  prefill   X [8192,5120] as decode; W [15360,5120] ~N(0,0.02);
            a smoothing fold is applied to X and W before quantization
  w8a16     X [8192,13824]: the first 1% of rows (82) ~N(0,1) x50, the rest
            ~N(0,1); W [5120,13824] ~N(0,0.015)
  group128  X [4096,5120] as decode; W [5120,5120] ~N(0,0.02), quantized
            with one scale per (channel, 128-wide K group)

The outlier channels are ceil(0.01*K) distinct columns drawn without
replacement by the same generator.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    wid: int
    M: int
    K: int
    N: int
    outlier: str          # "fixed2" | "cols" | "rows"
    outlier_gain: float
    w_sigma: float
    smooth: bool = False  # apply the smoothing fold (prefill)
    group: int | None = None  # 128 for group-scaled weights
    w8a16: bool = False


WORKLOADS = {
    "tiny": Workload("tiny", 1, 16, 256, 128, "fixed2", 20.0, 0.02),
    "decode": Workload("decode", 2, 8, 5120, 5120, "cols", 30.0, 0.02),
    "prefill": Workload("prefill", 3, 8192, 5120, 15360, "cols", 30.0, 0.02,
                        smooth=True),
    "w8a16": Workload("w8a16", 4, 8192, 13824, 5120, "rows", 50.0, 0.015,
                      w8a16=True),
    "group128": Workload("group128", 5, 4096, 5120, 5120, "cols", 30.0, 0.02,
                         group=128),
    # FP8 block W8A8 at the prefill shape; the smoothing fold stands in for
    # the FP8 page's smoothing pre-pass
    "fp8_block": Workload("fp8_block", 6, 8192, 5120, 15360, "cols", 30.0, 0.02,
                          smooth=True),
}

_TAG_X, _TAG_W, _TAG_OUT = 1, 2, 3


def _rng(seed: int, wid: int, tag: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(
        [int(seed), int(wid), int(tag)])))


def to_bf16(a_f32: np.ndarray) -> torch.Tensor:
    """fp32 numpy -> bf16 torch CPU tensor (torch's RNE cast)."""
    return torch.from_numpy(np.ascontiguousarray(a_f32, np.float32)).to(
        torch.bfloat16)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """bf16 torch tensor -> uint16 numpy array of its bit patterns."""
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def bits_to_bf16(b: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(b, np.uint16).view(
        np.int16)).view(torch.bfloat16)


def activations(w: Workload, seed: int = 0, M: int | None = None,
                K: int | None = None) -> torch.Tensor:
    """X bf16 [M,K] for workload w (M, K override the shape)."""
    M = w.M if M is None else M
    K = w.K if K is None else K
    g = _rng(seed, w.wid, _TAG_X)
    x = g.standard_normal((M, K), dtype=np.float32)
    og = np.float32(w.outlier_gain)
    if w.outlier == "fixed2":
        for c in (3, 77):
            if c < K:
                x[:, c] *= og
    elif w.outlier == "cols":
        gc = _rng(seed, w.wid, _TAG_OUT)
        cols = np.sort(gc.choice(K, size=math.ceil(0.01 * K), replace=False))
        x[:, cols] *= og
    elif w.outlier == "rows":
        x[: math.ceil(0.01 * M), :] *= og
    return to_bf16(x)


def weights(w: Workload, seed: int = 0, N: int | None = None,
            K: int | None = None) -> torch.Tensor:
    """W fp32 [N,K] ~ N(0, sigma) for workload w (not yet quantized)."""
    N = w.N if N is None else N
    K = w.K if K is None else K
    g = _rng(seed, w.wid, _TAG_W)
    a = g.standard_normal((N, K), dtype=np.float32)
    a *= np.float32(w.w_sigma)
    return torch.from_numpy(a)


def custom(M: int, K: int, N: int, seed: int, outlier_cols: int = 0,
           gain: float = 30.0, sigma: float = 0.02, wid: int = 99):
    """Generic X bf16 [M,K] and W fp32 [N,K] for edge-shape tests."""
    g = _rng(seed, wid, _TAG_X)
    x = g.standard_normal((M, K), dtype=np.float32)
    if outlier_cols:
        cols = _rng(seed, wid, _TAG_OUT).choice(K, size=min(K, outlier_cols),
                                                replace=False)
        x[:, cols] *= np.float32(gain)
    gw = _rng(seed, wid, _TAG_W)
    w = gw.standard_normal((N, K), dtype=np.float32) * np.float32(sigma)
    return to_bf16(x), torch.from_numpy(w)


def int8_uniform(shape, seed: int, lo: int = -128, hi: int = 127,
                 tag: int = 7) -> np.ndarray:
    """Uniform int8 codes in [lo, hi] (raw GEMM operands for INT32 tests)."""
    g = _rng(seed, 100, tag)
    return g.integers(lo, hi + 1, size=shape, dtype=np.int16).astype(np.int8)


def uniform_f32(shape, seed: int, lo: float, hi: float, tag: int = 8):
    g = _rng(seed, 101, tag)
    return g.uniform(lo, hi, size=shape).astype(np.float32)
