"""Pins for the FP8 block W8A8 part of the CPU oracle.

The method ("Qwen3.8-27B -- FP8 block + AWQ", "Recipe"): FP8 weights with one
scale per [128, 128] block, activations quantized at run time with one scale
per token and 128-wide K group; E4M3 scaled by amax/448 (the same page's
"KV cache" section).  Checks here are independent of the oracle's code: the
format's special points (``tests/golden/e4m3_spec_points.txt``), torch's own
float8_e4m3fn conversion, exact rational rounding (``tests/exact.py``),
power-of-two scales that make every quotient exact, invariants, and an fp64
matmul of the dequantized operands.  A plausible mistake (the FNUZ bias,
ties away from zero, a divisor of 127 or 447, a transposed scale grid, a
dropped block) fails at least one of them.
"""
from __future__ import annotations

import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.exact import e4m3, fp32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _torch_e4m3_bytes(v_f32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(v_f32, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _torch_e4m3_values(codes_u8: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(codes_u8, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _f32(bits_u16: np.ndarray) -> np.ndarray:
    return (bits_u16.astype(np.uint32) << 16).view(np.float32)


def test_e4m3_spec_points_golden():
    with open(os.path.join(GOLDEN, "e4m3_spec_points.txt")) as f:
        rows = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    assert len(rows) >= 10
    for code, val in rows:
        c = int(code, 16)
        got = oracle.e4m3_value(c)
        if val == "nan":
            assert np.isnan(got), code
        else:
            assert got == float(val) and np.signbit(got) == val.startswith("-"), code
            assert oracle.e4m3_rne(float(val)) == c, code


def test_e4m3_value_table_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = _torch_e4m3_values(codes)
    got = np.array([oracle.e4m3_value(int(c)) for c in codes])
    nan = np.isnan(ref)
    assert (np.isnan(got) == nan).all() and nan.sum() == 2
    np.testing.assert_array_equal(got[~nan], ref[~nan])
    assert (np.signbit(got[~nan]) == np.signbit(ref[~nan])).all()


def _probe_values() -> np.ndarray:
    """Log-uniform magnitudes over the whole E4M3 range and below, every
    midpoint between neighbouring codes (exact ties), and the fp32 values
    just either side of each midpoint, in both signs."""
    g = np.random.default_rng(7)
    mags = np.exp2(g.uniform(-14.0, np.log2(448.0), 20000)).astype(np.float32)
    vals = np.array([oracle.e4m3_value(c) for c in range(0x7F)])
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)  # exact in fp32
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(0))
    top = np.array([448.0, 455.0, 463.99997, 464.0], np.float32)
    v = np.concatenate([mags, mids, up, dn, vals.astype(np.float32), top,
                        np.array([0.0, 2.0 ** -149, 2.0 ** -10, 2.0 ** -11], np.float32)])
    return np.concatenate([v, -v]).astype(np.float32)


def test_e4m3_rne_matches_torch_cast():
    v = _probe_values()
    got = np.array([oracle.e4m3_rne(float(x)) for x in v], np.uint8)
    np.testing.assert_array_equal(got, _torch_e4m3_bytes(v))


def test_e4m3_rne_matches_exact_rational_rounding():
    v = _probe_values()[::7]
    for x in v:
        want = e4m3(Fraction(float(x)))
        got = oracle.e4m3_value(oracle.e4m3_rne(float(x)))
        assert Fraction(got) == want, x


def test_e4m3_rne_saturates_and_keeps_sign():
    for x in (448.0, 464.0, 465.0, 480.0, 1e6, 3.0e38, float("inf")):
        assert oracle.e4m3_rne(x) == 0x7E
        assert oracle.e4m3_rne(-x) == 0xFE
    assert oracle.e4m3_rne(-0.0) == 0x80 and oracle.e4m3_rne(-1e-30) == 0x80
    assert oracle.e4m3_rne(float("nan")) == 0x7F


def _blocky_activations(M, K, seed):
    """bf16 rows whose 128-blocks differ in magnitude by powers of ten, with
    an all-zero block and a block of negative zeros."""
    g = np.random.default_rng(seed)
    x = g.standard_normal((M, K)).astype(np.float32)
    x *= (10.0 ** g.integers(-3, 3, (M, K // 128, 1))).repeat(128, axis=2).reshape(M, K).astype(np.float32)
    x[0, 128:256] = 0.0
    x[min(1, M - 1), 0:128] = -0.0
    return synth.bf16_bits(torch.from_numpy(x).to(torch.bfloat16))


def test_fp8_group_quant_matches_torch_pipeline():
    M, K = 6, 768
    xb = _blocky_activations(M, K, 11)
    xq, s = oracle.quant_fp8_per_group128(xb)
    xf = torch.from_numpy(_f32(xb)).reshape(M, K // 128, 128)
    amax = xf.abs().amax(dim=2)
    s_ref = amax / torch.tensor(448.0)  # torch's IEEE fp32 division
    np.testing.assert_array_equal(s, s_ref.numpy())
    q = xf / torch.where(s_ref == 0, torch.ones_like(s_ref), s_ref)[..., None]
    codes = q.to(torch.float8_e4m3fn).view(torch.uint8)
    codes[s_ref == 0] = 0
    np.testing.assert_array_equal(xq, codes.reshape(M, K).numpy())


def test_fp8_group_quant_invariants():
    M, K = 8, 1024
    xb = synth.bf16_bits(synth.activations(synth.WORKLOADS["decode"], 0)[:M, :K].contiguous())
    xq, s = oracle.quant_fp8_per_group128(xb)
    val = _torch_e4m3_values(xq).reshape(M, K // 128, 128)
    assert not np.isnan(val).any()
    x = _f32(xb).astype(np.float64).reshape(M, K // 128, 128)
    am = np.abs(x).argmax(axis=2)
    assert (np.abs(np.take_along_axis(val, am[..., None], 2)) == 448.0).all()
    # round trip: |x - q*s| <= half the E4M3 spacing at q, times s (plus the
    # quotient's own rounding)
    q = x / s[..., None].astype(np.float64)
    e = np.floor(np.log2(np.maximum(np.abs(q), 2.0 ** -6)))
    half = np.exp2(e - 4)
    assert (np.abs(q - val) <= half * (1 + 2 ** -20) + np.abs(q) * 2 ** -23).all()


def test_fp8_group_quant_power_of_two_scales_are_exact():
    """Blocks whose absmax is 448 * 2^j have scale exactly 2^j, every
    quotient is exact, and the codes are those of the exactly scaled
    values."""
    M, K = 4, 512
    g = np.random.default_rng(5)
    x = g.uniform(-1.0, 1.0, (M, K)).astype(np.float32)
    js = g.integers(-6, 4, (M, K // 128))
    for m in range(M):
        for b in range(K // 128):
            blk = x[m, 128 * b:128 * b + 128] * np.float32(448.0 * 2.0 ** js[m, b])
            blk[g.integers(0, 128)] = np.float32(448.0 * 2.0 ** js[m, b]) * (1 if g.random() < 0.5 else -1)
            x[m, 128 * b:128 * b + 128] = blk
    xb = synth.bf16_bits(torch.from_numpy(x).to(torch.bfloat16))
    xq, s = oracle.quant_fp8_per_group128(xb)
    np.testing.assert_array_equal(s, np.exp2(js).astype(np.float32))
    xf = _f32(xb).reshape(M, K // 128, 128)
    exact = (xf / np.exp2(js)[..., None]).astype(np.float32)  # exact: power-of-two scaling
    for v, c in zip(exact.ravel()[::5], xq.reshape(M, K // 128, 128).ravel()[::5]):
        assert Fraction(oracle.e4m3_value(int(c))) == e4m3(Fraction(float(v)))


def _bf16_values(lo_bits: int, hi_bits: int) -> np.ndarray:
    b = torch.arange(lo_bits, hi_bits, dtype=torch.int32).to(torch.int16)
    return b.view(torch.bfloat16).float().numpy()


def test_fp8_group_quant_divides_rather_than_multiplying_by_reciprocal():
    """Rows built from bf16 values whose quotient x/s and product x*fl(1/s)
    round to different E4M3 codes: the codes must be those of the division."""
    xs = _bf16_values(0x3C00, 0x4380)  # 2^-7 .. 255
    pairs = []
    for a in _bf16_values(0x4300, 0x4400):  # block absmax in [128, 512)
        s = np.float32(np.float32(a) / np.float32(448.0))
        xx = xs[xs <= a]
        div = _torch_e4m3_bytes((xx / s).astype(np.float32))
        rec = _torch_e4m3_bytes((xx * np.float32(np.float32(1.0) / s)).astype(np.float32))
        for i in np.nonzero(div != rec)[0][:4]:
            pairs.append((a, xx[i], div[i], rec[i]))
    assert len(pairs) >= 50
    M = len(pairs)
    x = np.zeros((M, 128), np.float32)
    for r, (a, v, _, _) in enumerate(pairs):
        x[r, 0], x[r, 1], x[r, 2] = a, v, -v
    xq, s = oracle.quant_fp8_per_group128(synth.bf16_bits(torch.from_numpy(x).to(torch.bfloat16)))
    for r, (a, v, cd, cr) in enumerate(pairs):
        assert s[r, 0] == np.float32(np.float32(a) / np.float32(448.0))
        assert xq[r, 1] == cd and xq[r, 2] == (cd | 0x80) and cd != cr, (a, v)


def test_fp8_weight_block_quant_matches_torch_pipeline():
    N, K = 384, 256  # N != K: a transposed block grid fails
    g = np.random.default_rng(21)
    w = (g.standard_normal((N, K)) * 0.02).astype(np.float32)
    w *= (10.0 ** g.integers(-2, 2, (N // 128, 1, K // 128, 1))).repeat(128, 1).repeat(128, 3).reshape(N, K).astype(np.float32)
    # block maxima on every edge and corner of a block
    for i, (r, c) in enumerate([(127, 127), (0, 127), (127, 0), (0, 0), (64, 127), (127, 64)]):
        nb, kb = i % (N // 128), (i // (N // 128)) % (K // 128)
        blk = w[128 * nb:128 * nb + 128, 128 * kb:128 * kb + 128]
        blk[r, c] = np.float32(4.0) * np.abs(blk).max() * (1 if i % 2 else -1)
    wq, s = oracle.quant_weight_fp8_block128(w)
    assert s.shape == (N // 128, K // 128)
    wt = torch.from_numpy(w).reshape(N // 128, 128, K // 128, 128)
    amax = wt.abs().amax(dim=(1, 3))
    s_ref = amax / torch.tensor(448.0)
    np.testing.assert_array_equal(s, s_ref.numpy())
    codes = (wt / s_ref[:, None, :, None]).to(torch.float8_e4m3fn).view(torch.uint8)
    np.testing.assert_array_equal(wq, codes.reshape(N, K).numpy())


def _fp8_operands(M, N, K, seed):
    xb = _blocky_activations(M, K, seed)
    xq, sx = oracle.quant_fp8_per_group128(xb)
    g = np.random.default_rng(seed + 1)
    w = (g.standard_normal((N, K)) * 0.02).astype(np.float32)
    w *= (2.0 ** g.integers(-3, 3, (N // 128, 1, K // 128, 1))).repeat(128, 1).repeat(128, 3).reshape(N, K).astype(np.float32)
    wq, sw = oracle.quant_weight_fp8_block128(w)
    return xq, sx, wq, sw


def test_fp8_block_mm_matches_dequantized_fp64_matmul():
    M, N, K = 5, 384, 640
    xq, sx, wq, sw = _fp8_operands(M, N, K, 40)
    y, mag = oracle.fp8_block_mm(xq, wq, sx, sw, with_mag=True)
    xd = torch.from_numpy(_torch_e4m3_values(xq) * np.repeat(sx.astype(np.float64), 128, axis=1))
    wd = torch.from_numpy(_torch_e4m3_values(wq) * np.repeat(np.repeat(sw.astype(np.float64), 128, axis=0), 128, axis=1))
    ref = (xd @ wd.T).numpy()
    assert (np.abs(y - ref) <= 1e-13 * mag + 1e-300).all()
    absref = (xd.abs() @ wd.abs().T).numpy()
    np.testing.assert_allclose(mag, absref, rtol=1e-13)


def test_fp8_block_mm_exact_rational_tiny():
    M, N, K = 2, 128, 256
    xq, sx, wq, sw = _fp8_operands(M, N, K, 50)
    y = oracle.fp8_block_mm(xq, wq, sx, sw)
    for m in range(M):
        for n in (0, 1, 77, 127):
            acc = Fraction(0)
            for gi in range(K // 128):
                p = sum(Fraction(oracle.e4m3_value(int(xq[m, k]))) * Fraction(oracle.e4m3_value(int(wq[n, k])))
                        for k in range(128 * gi, 128 * gi + 128))
                acc += Fraction(float(sx[m, gi])) * Fraction(float(sw[n // 128, gi])) * p
            assert abs(Fraction(float(y[m, n])) - acc) <= abs(acc) * Fraction(1, 2 ** 50), (m, n)


def test_fp8_oracle_rejects_bad_shapes_and_nan_codes():
    with pytest.raises(ValueError):
        oracle.quant_fp8_per_group128(np.zeros((2, 100), np.uint16))
    with pytest.raises(ValueError):
        oracle.quant_weight_fp8_block128(np.zeros((100, 128), np.float32))
    a = np.zeros((1, 128), np.uint8)
    b = np.zeros((128, 128), np.uint8)
    b[3, 4] = 0x7F
    with pytest.raises(ValueError):
        oracle.fp8_block_mm(a, b, np.ones((1, 1), np.float32), np.ones((1, 1), np.float32))
