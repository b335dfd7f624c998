"""CPU oracle for the W8A8 INT8 linear layer -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It shares no code with the HIP library
(``w8a8_int8_gemm_token_amd``) and never imports it.

The arithmetic lives in ``q8_oracle.c`` (plain C loops, IEEE fp32, no fused
multiply-add except where ``fmaf`` is written).  This module only compiles it
with gcc, loads it with ctypes and marshals numpy arrays.  Each function names
the definition it follows; the C file carries the full citations and the
readings taken where the pages are silent.

Parity pins: every function here is pinned by ``tests/test_oracle_pins.py``
against exact rational arithmetic, library routines, closed forms and
invariants (none of them re-uses this module's arithmetic).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "q8_oracle.c")
_LIB = os.path.join(_HERE, "libq8_oracle.so")
_CFLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC"]

_lib = None


def build(force: bool = False) -> str:
    """Compile q8_oracle.c into libq8_oracle.so with gcc (no GPU involved)."""
    if force or not os.path.exists(_LIB) or \
            os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *_CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int64
        F = ctypes.c_float
        sig = {
            "q8o_env_ok": ([], ctypes.c_int),
            "q8o_threads": ([], ctypes.c_int),
            "q8o_f32_to_bf16": ([F], ctypes.c_uint16),
            "q8o_bf16_to_f32": ([ctypes.c_uint16], F),
            "q8o_quant_per_token": ([P, I, I, P, P], None),
            "q8o_quant_per_token_f16": ([P, I, I, P, P], None),
            "q8o_w8a16_ref_f16": ([P, P, P, I, I, I, P, P], None),
            "q8o_f16_to_f32": ([ctypes.c_uint16], F),
            "q8o_f32_to_f16": ([F], ctypes.c_uint16),
            "q8o_scaled_mm_f16": ([P, P, P, P, I, I, I, P], ctypes.c_int),
            "q8o_quant_per_group128_f16": ([P, I, I, P, P], ctypes.c_int),
            "q8o_scaled_mm_group128_act_f16": ([P, P, P, P, I, I, I, P], ctypes.c_int),
            "q8o_e4m3_value": ([ctypes.c_uint8], ctypes.c_double),
            "q8o_e4m3_rne": ([F], ctypes.c_uint8),
            "q8o_quant_fp8_per_group128": ([P, I, I, P, P], ctypes.c_int),
            "q8o_quant_weight_fp8_block128": ([P, I, I, P, P], ctypes.c_int),
            "q8o_fp8_block_mm": ([P, P, P, P, I, I, I, P, P], ctypes.c_int),
            "q8o_quant_weight": ([P, I, I, I, P, P], ctypes.c_int),
            "q8o_mm_i32": ([P, P, I, I, I, P], ctypes.c_int),
            "q8o_epilogue_channel": ([P, P, P, I, I, P], None),
            "q8o_scaled_mm": ([P, P, P, P, I, I, I, P], ctypes.c_int),
            "q8o_scaled_mm_group128": ([P, P, P, P, I, I, I, P], ctypes.c_int),
            "q8o_w8a16_ref": ([P, P, P, I, I, I, P, P], None),
            "q8o_smooth_scales": ([P, I, I, F, P], ctypes.c_int),
            "q8o_smooth_fold_x": ([P, P, I, I, P], None),
            "q8o_smooth_fold_w": ([P, P, I, I, P], None),
            "q8o_rmsnorm_quant": ([P, P, P, F, I, I, P, P, P, P], ctypes.c_int),
            "q8o_rmsnorm_quant_at_ss": ([P, P, F, I, I, P, P, P, P], ctypes.c_int),
            "q8o_sum_squares_bf16": ([P, I, I, P], None),
            "q8o_quant_per_group128": ([P, I, I, P, P], ctypes.c_int),
            "q8o_scaled_mm_group128_act": ([P, P, P, P, I, I, I, P], ctypes.c_int),
        }
        for name, (args, res) in sig.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = res
        if not lib.q8o_env_ok():
            raise RuntimeError("oracle: FPU not in round-to-nearest-even mode")
        _lib = lib
    return _lib


def _c(a: np.ndarray, dtype) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.dtype(dtype):
        raise TypeError(f"oracle: expected {np.dtype(dtype)}, got {a.dtype}")
    return a


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def threads() -> int:
    """Threads the oracle's parallel loops run on."""
    return int(_load().q8o_threads())


def f32_to_bf16(v: float) -> int:
    """bf16 bits of fp32 value v, round to nearest even."""
    return int(_load().q8o_f32_to_bf16(ctypes.c_float(v)))


def bf16_to_f32(bits: int) -> float:
    return float(_load().q8o_bf16_to_f32(ctypes.c_uint16(bits)))


def quant_per_token(x_bf16: np.ndarray):
    """Per-token quant.  x_bf16: uint16 [M,K] (bf16 bits) -> (xq int8 [M,K], s fp32 [M])."""
    x = _c(x_bf16, np.uint16)
    M, K = x.shape
    xq = np.empty((M, K), np.int8)
    s = np.empty((M,), np.float32)
    _load().q8o_quant_per_token(_p(x), M, K, _p(xq), _p(s))
    return xq, s


def quant_weight(w_f32: np.ndarray, group: int | None = None):
    """Weight quant.  w: fp32 [N,K] -> (wq int8 [N,K], s fp32 [N] or [N,K/group])."""
    w = _c(w_f32, np.float32)
    N, K = w.shape
    g = K if group is None else group
    wq = np.empty((N, K), np.int8)
    s = np.empty((N, K // g), np.float32)
    if _load().q8o_quant_weight(_p(w), N, K, g, _p(wq), _p(s)) != 0:
        raise ValueError("oracle: group must divide K")
    return wq, (s[:, 0].copy() if group is None else s)


def mm_i32(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """INT8 GEMM.  a int8 [M,K], b int8 [N,K] -> exact int32 [M,N]."""
    a = _c(a, np.int8)
    b = _c(b, np.int8)
    M, K = a.shape
    N, K2 = b.shape
    assert K == K2
    out = np.empty((M, N), np.int32)
    if _load().q8o_mm_i32(_p(a), _p(b), M, N, K, _p(out)) != 0:
        raise OverflowError("oracle: int32 accumulator overflow")
    return out


def epilogue_channel(acc: np.ndarray, s_tok: np.ndarray, s_ch: np.ndarray):
    """Per-channel epilogue.  int32 [M,N] -> bf16 bits uint16 [M,N]."""
    acc = _c(acc, np.int32)
    s_tok = _c(s_tok, np.float32)
    s_ch = _c(s_ch, np.float32)
    M, N = acc.shape
    y = np.empty((M, N), np.uint16)
    _load().q8o_epilogue_channel(_p(acc), _p(s_tok), _p(s_ch), M, N, _p(y))
    return y


def scaled_mm(a, b, s_tok, s_ch) -> np.ndarray:
    """GEMM + per-channel epilogue.  -> bf16 bits uint16 [M,N]."""
    a = _c(a, np.int8)
    b = _c(b, np.int8)
    s_tok = _c(s_tok, np.float32)
    s_ch = _c(s_ch, np.float32)
    M, K = a.shape
    N = b.shape[0]
    y = np.empty((M, N), np.uint16)
    if _load().q8o_scaled_mm(_p(a), _p(b), _p(s_tok), _p(s_ch), M, N, K,
                             _p(y)) != 0:
        raise OverflowError("oracle: int32 accumulator overflow")
    return y


def scaled_mm_group128(a, b, s_tok, s_grp) -> np.ndarray:
    """GEMM with group-128 weights.  s_grp fp32 [N, K/128] -> bf16 bits uint16 [M,N]."""
    a = _c(a, np.int8)
    b = _c(b, np.int8)
    s_tok = _c(s_tok, np.float32)
    s_grp = _c(s_grp, np.float32)
    M, K = a.shape
    N = b.shape[0]
    assert s_grp.shape == (N, K // 128)
    y = np.empty((M, N), np.uint16)
    if _load().q8o_scaled_mm_group128(_p(a), _p(b), _p(s_tok), _p(s_grp),
                                      M, N, K, _p(y)) != 0:
        raise ValueError("oracle: K must be a multiple of 128")
    return y


def w8a16_ref(x_bf16, wq, s_ch, with_mag: bool = False):
    """W8A16 reference.  -> fp64 y_ref [M,N] (and fp64 magnitude sums)."""
    x = _c(x_bf16, np.uint16)
    wq = _c(wq, np.int8)
    s_ch = _c(s_ch, np.float32)
    M, K = x.shape
    N = wq.shape[0]
    y = np.empty((M, N), np.float64)
    mag = np.empty((M, N), np.float64) if with_mag else None
    _load().q8o_w8a16_ref(_p(x), _p(wq), _p(s_ch), M, N, K, _p(y),
                          _p(mag) if with_mag else None)
    return (y, mag) if with_mag else y


def smooth_scales(x_bf16, cap: float = 16.0) -> np.ndarray:
    """s_j = min(cap, sqrtf(max_m |x[m,j]|)) -> fp32 [K]."""
    x = _c(x_bf16, np.uint16)
    M, K = x.shape
    s = np.empty((K,), np.float32)
    if _load().q8o_smooth_scales(_p(x), M, K, cap, _p(s)) != 0:
        raise ValueError("oracle: a smoothing scale is 0 (all-zero column)")
    return s


def smooth_fold_x(x_bf16, s) -> np.ndarray:
    x = _c(x_bf16, np.uint16)
    s = _c(s, np.float32)
    M, K = x.shape
    out = np.empty((M, K), np.uint16)
    _load().q8o_smooth_fold_x(_p(x), _p(s), M, K, _p(out))
    return out


def smooth_fold_w(w_f32, s) -> np.ndarray:
    w = _c(w_f32, np.float32)
    s = _c(s, np.float32)
    N, K = w.shape
    out = np.empty((N, K), np.float32)
    _load().q8o_smooth_fold_w(_p(w), _p(s), N, K, _p(out))
    return out


def rmsnorm_quant(x_bf16, gamma_bf16, eps: float, res_bf16=None, return_ss: bool = False):
    """Residual add (optional) + RMSNorm + per-token INT8 quant.
    Returns (xq int8 [M,K], scale fp32 [M], y bf16 bits [M,K], res_out bf16
    bits [M,K] or None), and with return_ss the fp32 sums of squares [M]
    (the exact sum of each row's squares, rounded once) as a fifth item."""
    x = _c(x_bf16, np.uint16)
    g = _c(gamma_bf16, np.uint16)
    M, K = x.shape
    if g.shape != (K,):
        raise ValueError("gamma must have K entries")
    res = None if res_bf16 is None else np.array(res_bf16, dtype=np.uint16, copy=True, order="C")
    xq = np.empty((M, K), np.int8)
    s = np.empty((M,), np.float32)
    y = np.empty((M, K), np.uint16)
    ss = np.empty((M,), np.float32)
    rc = _load().q8o_rmsnorm_quant(_p(x), None if res is None else _p(res), _p(g), float(eps),
                                   M, K, _p(xq), _p(s), _p(y), _p(ss))
    if rc != 0:
        raise ValueError(f"oracle rmsnorm_quant failed ({rc}): K must be a multiple of 8")
    return (xq, s, y, res, ss) if return_ss else (xq, s, y, res)


def sum_squares_bf16(h_bf16) -> np.ndarray:
    """Per row of bf16 bits [M,K]: the exact sum of the squares, rounded once
    to fp32 (round to nearest even)."""
    h = _c(h_bf16, np.uint16)
    M, K = h.shape
    ss = np.empty((M,), np.float32)
    _load().q8o_sum_squares_bf16(_p(h), M, K, _p(ss))
    return ss


def rmsnorm_quant_at_ss(h_bf16, gamma_bf16, eps: float, ss):
    """The normalization + quantization of rows h (bf16 bits [M,K], after the
    residual add) for given fp32 sums of squares ss [M]:
    returns (xq int8 [M,K], scale fp32 [M], y bf16 bits [M,K])."""
    h = _c(h_bf16, np.uint16)
    g = _c(gamma_bf16, np.uint16)
    ssa = _c(np.asarray(ss, dtype=np.float32), np.float32)
    M, K = h.shape
    if g.shape != (K,) or ssa.shape != (M,):
        raise ValueError("gamma must have K entries and ss M entries")
    xq = np.empty((M, K), np.int8)
    s = np.empty((M,), np.float32)
    y = np.empty((M, K), np.uint16)
    if _load().q8o_rmsnorm_quant_at_ss(_p(h), _p(g), float(eps), M, K, _p(ssa), _p(xq), _p(s), _p(y)) != 0:
        raise MemoryError("oracle rmsnorm_quant_at_ss: allocation failed")
    return xq, s, y


def quant_per_group128(x_bf16):
    """Per-token-per-128-group quant: -> (xq int8 [M,K], s_x fp32 [M,K/128])."""
    x = _c(x_bf16, np.uint16)
    M, K = x.shape
    xq = np.empty((M, K), np.int8)
    s = np.empty((M, K // 128), np.float32)
    if _load().q8o_quant_per_group128(_p(x), M, K, _p(xq), _p(s)) != 0:
        raise ValueError("oracle: K must be a multiple of 128")
    return xq, s


def scaled_mm_group128_act(a, b, s_x, s_w) -> np.ndarray:
    """GEMM with per-(token, block) and per-(channel, block) scales:
    s_x fp32 [M, K/128], s_w fp32 [N, K/128] -> bf16 bits uint16 [M,N]."""
    a = _c(a, np.int8)
    b = _c(b, np.int8)
    s_x = _c(s_x, np.float32)
    s_w = _c(s_w, np.float32)
    M, K = a.shape
    N = b.shape[0]
    assert s_x.shape == (M, K // 128) and s_w.shape == (N, K // 128)
    y = np.empty((M, N), np.uint16)
    if _load().q8o_scaled_mm_group128_act(_p(a), _p(b), _p(s_x), _p(s_w), M, N, K, _p(y)) != 0:
        raise ValueError("oracle: K must be a multiple of 128")
    return y


def e4m3_value(code: int) -> float:
    """Value of one E4M3 byte (OCP FP8, bias 7, max 448; NaN for 0x7F/0xFF)."""
    return _load().q8o_e4m3_value(int(code) & 0xFF)


def e4m3_rne(v: float) -> int:
    """E4M3 byte nearest to the fp32 value v (ties to even, saturating at 448)."""
    return int(_load().q8o_e4m3_rne(float(np.float32(v))))


def quant_fp8_per_group128(x_bf16):
    """Per-token-per-128-group FP8 quant: -> (xq E4M3 bytes uint8 [M,K],
    s_x fp32 [M,K/128])."""
    x = _c(x_bf16, np.uint16)
    M, K = x.shape
    xq = np.empty((M, K), np.uint8)
    s = np.empty((M, K // 128), np.float32)
    if _load().q8o_quant_fp8_per_group128(_p(x), M, K, _p(xq), _p(s)) != 0:
        raise ValueError("oracle: K must be a multiple of 128")
    return xq, s


def quant_weight_fp8_block128(w_f32):
    """FP8 [128,128] block weights: -> (wq E4M3 bytes uint8 [N,K],
    s_w fp32 [N/128, K/128])."""
    w = _c(w_f32, np.float32)
    N, K = w.shape
    wq = np.empty((N, K), np.uint8)
    s = np.empty((N // 128, K // 128), np.float32)
    if _load().q8o_quant_weight_fp8_block128(_p(w), N, K, _p(wq), _p(s)) != 0:
        raise ValueError("oracle: N and K must be multiples of 128")
    return wq, s


def fp8_block_mm(a, b, s_x, s_w, with_mag: bool = False):
    """FP8 block-scaled GEMM in fp64: a [M,K], b [N,K] E4M3 bytes, s_x
    [M,K/128], s_w [N/128,K/128] -> y float64 [M,N] (and the magnitude sum
    used for error bounds when with_mag)."""
    a = _c(a, np.uint8)
    b = _c(b, np.uint8)
    s_x = _c(s_x, np.float32)
    s_w = _c(s_w, np.float32)
    M, K = a.shape
    N = b.shape[0]
    assert b.shape[1] == K and s_x.shape == (M, K // 128) and s_w.shape == (N // 128, K // 128)
    y = np.empty((M, N), np.float64)
    mag = np.empty((M, N), np.float64) if with_mag else None
    rc = _load().q8o_fp8_block_mm(_p(a), _p(b), _p(s_x), _p(s_w), M, N, K, _p(y),
                                  None if mag is None else _p(mag))
    if rc == -1:
        raise ValueError("oracle: N and K must be multiples of 128")
    if rc == -2:
        raise ValueError("oracle: NaN E4M3 code in an operand")
    return (y, mag) if with_mag else y


# ---------------------------------------------------------------- fp16 --

def f16_to_f32(bits: int) -> float:
    """fp16 bits -> fp32 value (exact)."""
    return _load().q8o_f16_to_f32(int(bits) & 0xFFFF)


def f32_to_f16(v: float) -> int:
    """fp32 -> fp16 bits, round to nearest even (overflow to infinity)."""
    return int(_load().q8o_f32_to_f16(float(np.float32(v))))


def quant_per_token_f16(x_f16: np.ndarray):
    """Per-token quant of fp16 activations.  x: uint16 [M,K] fp16 bits ->
    (xq int8 [M,K], s fp32 [M])."""
    x = _c(x_f16, np.uint16)
    M, K = x.shape
    xq = np.empty((M, K), np.int8)
    s = np.empty((M,), np.float32)
    _load().q8o_quant_per_token_f16(_p(x), M, K, _p(xq), _p(s))
    return xq, s


def scaled_mm_f16(a, b, s_tok, s_ch) -> np.ndarray:
    """GEMM + per-channel epilogue, fp16 out -> fp16 bits uint16 [M,N]."""
    a = _c(a, np.int8)
    b = _c(b, np.int8)
    s_tok = _c(s_tok, np.float32)
    s_ch = _c(s_ch, np.float32)
    M, K = a.shape
    N = b.shape[0]
    y = np.empty((M, N), np.uint16)
    if _load().q8o_scaled_mm_f16(_p(a), _p(b), _p(s_tok), _p(s_ch), M, N, K, _p(y)) != 0:
        raise OverflowError("oracle: int32 accumulator overflow")
    return y


def quant_per_group128_f16(x_f16):
    """Per-token-per-128-group quant of fp16 activations -> (xq int8 [M,K],
    s_x fp32 [M,K/128])."""
    x = _c(x_f16, np.uint16)
    M, K = x.shape
    xq = np.empty((M, K), np.int8)
    s = np.empty((M, K // 128), np.float32)
    if _load().q8o_quant_per_group128_f16(_p(x), M, K, _p(xq), _p(s)) != 0:
        raise ValueError("oracle: K must be a multiple of 128")
    return xq, s


def scaled_mm_group128_act_f16(a, b, s_x, s_w) -> np.ndarray:
    """GEMM with per-(token, block) and per-(channel, block) scales, fp16
    out -> fp16 bits uint16 [M,N]."""
    a = _c(a, np.int8)
    b = _c(b, np.int8)
    s_x = _c(s_x, np.float32)
    s_w = _c(s_w, np.float32)
    M, K = a.shape
    N = b.shape[0]
    assert s_x.shape == (M, K // 128) and s_w.shape == (N, K // 128)
    y = np.empty((M, N), np.uint16)
    if _load().q8o_scaled_mm_group128_act_f16(_p(a), _p(b), _p(s_x), _p(s_w), M, N, K, _p(y)) != 0:
        raise ValueError("oracle: K must be a multiple of 128")
    return y


def w8a16_ref_f16(x_f16, wq, s_ch, with_mag: bool = False):
    """W8A16 reference with fp16 activations -> fp64 y_ref [M,N] (and fp64
    magnitude sums)."""
    x = _c(x_f16, np.uint16)
    wq = _c(wq, np.int8)
    s_ch = _c(s_ch, np.float32)
    M, K = x.shape
    N = wq.shape[0]
    y = np.empty((M, N), np.float64)
    mag = np.empty((M, N), np.float64) if with_mag else None
    _load().q8o_w8a16_ref_f16(_p(x), _p(wq), _p(s_ch), M, N, K, _p(y),
                              _p(mag) if with_mag else None)
    return (y, mag) if with_mag else y
