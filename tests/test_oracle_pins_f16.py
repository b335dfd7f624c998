"""Pins for the fp16 variant of the CPU oracle (fp16 activations in, fp16
outputs; "Qwen3.8-27B-GPTQ-INT8-W8A8-GS128", "Serving (vLLM, gfx908 fork)":
--dtype half is the model's native dtype, GEMM inputs quantized to INT8).

The fp16 conversions are checked against numpy's and torch's float16 casts
and exact rational rounding (``tests/exact.py``); the quantizers against
the bf16 quantizer on values both formats represent exactly and against
exact rationals; the epilogues against exact rational chains rounded to
fp16.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import torch

import oracle
import synth
from tests.exact import f16, fp32


def _f16_probe_values() -> np.ndarray:
    g = np.random.default_rng(9)
    mags = np.exp2(g.uniform(-26.0, 17.0, 20000)).astype(np.float32)
    fin = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    mids = ((fin[:-1] + fin[1:]) / 2)[::37].astype(np.float32)  # exact ties (fp32)
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(0))
    edge = np.array([65504.0, 65519.996, 65520.0, 70000.0, 2.0 ** -24, 2.0 ** -25,
                     3 * 2.0 ** -26, 2.0 ** -14, 0.0], np.float32)
    v = np.concatenate([mags, mids, up, dn, edge])
    return np.concatenate([v, -v]).astype(np.float32)


def test_f16_decode_all_patterns_match_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float32)
    got = np.array([oracle.f16_to_f32(int(b)) for b in bits[::1]], np.float32)
    nan = np.isnan(ref)
    assert (np.isnan(got) == nan).all()
    np.testing.assert_array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_f16_encode_matches_numpy_and_torch():
    v = _f16_probe_values()
    got = np.array([oracle.f32_to_f16(float(x)) for x in v], np.uint16)
    with np.errstate(over="ignore"):  # the probe includes values that overflow to infinity
        ref = v.astype(np.float16).view(np.uint16)
    np.testing.assert_array_equal(got, ref)
    np.testing.assert_array_equal(got, torch.from_numpy(v).half().view(torch.int16).numpy().view(np.uint16))


def test_f16_encode_matches_exact_rational_rounding():
    for x in _f16_probe_values()[::11]:
        want = f16(Fraction(float(x)))
        b = oracle.f32_to_f16(float(x))
        got = oracle.f16_to_f32(b)
        if abs(want) > 65504:
            assert np.isinf(got) and (got > 0) == (want > 0)
        else:
            assert Fraction(got) == want, x


def _both_formats(M, K, seed):
    """Values with at most 8 significant bits in [2^-14, 2^15): exactly
    representable as bf16 and as fp16."""
    g = np.random.default_rng(seed)
    mant = g.integers(128, 256, (M, K))
    ex = g.integers(-14 - 7, 8, (M, K))
    v = (mant * np.exp2(ex) * np.where(g.random((M, K)) < 0.5, -1, 1)).astype(np.float32)
    v[0, :5] = 0.0
    return v


def test_f16_quant_equals_bf16_quant_on_common_values():
    v = _both_formats(6, 512, 3)
    xb = synth.bf16_bits(torch.from_numpy(v).to(torch.bfloat16))
    xh = v.astype(np.float16).view(np.uint16)
    assert (torch.from_numpy(v).to(torch.bfloat16).float().numpy() == v).all()
    assert (v.astype(np.float16).astype(np.float32) == v).all()
    q1, s1 = oracle.quant_per_token(xb)
    q2, s2 = oracle.quant_per_token_f16(xh)
    np.testing.assert_array_equal(q1, q2)
    np.testing.assert_array_equal(s1, s2)
    g1, t1 = oracle.quant_per_group128(xb)
    g2, t2 = oracle.quant_per_group128_f16(xh)
    np.testing.assert_array_equal(g1, g2)
    np.testing.assert_array_equal(t1, t2)


def test_f16_quant_exact_rational():
    g = np.random.default_rng(4)
    x = (g.standard_normal((3, 96)) * 40).astype(np.float16)
    q, s = oracle.quant_per_token_f16(x.view(np.uint16))
    for m in range(3):
        row = [Fraction(float(v)) for v in x[m]]
        a = max(abs(r) for r in row)
        sc = fp32(a / 127)
        assert Fraction(float(s[m])) == sc
        for k, r in enumerate(row):
            t = fp32(r / sc)
            fl = t.numerator // t.denominator
            d = t - fl
            n = fl + 1 if d > Fraction(1, 2) or (d == Fraction(1, 2) and fl % 2) else fl
            assert q[m, k] == max(-127, min(127, n)), (m, k)


def test_f16_epilogues_exact_rational_chain():
    M, N, K = 3, 5, 256
    a = synth.int8_uniform((M, K), seed=61)
    b = synth.int8_uniform((N, K), seed=62)
    s_tok = synth.uniform_f32((M,), 63, 1e-3, 0.5)
    s_ch = synth.uniform_f32((N,), 64, 1e-4, 1e-2)
    y = oracle.scaled_mm_f16(a, b, s_tok, s_ch)
    for m in range(M):
        for n in range(N):
            acc = int(np.dot(a[m].astype(np.int64), b[n].astype(np.int64)))
            v = fp32(fp32(fp32(Fraction(acc)) * Fraction(float(s_tok[m]))) * Fraction(float(s_ch[n])))
            assert Fraction(oracle.f16_to_f32(int(y[m, n]))) == f16(v), (m, n)
    s_x = synth.uniform_f32((M, K // 128), 65, 1e-3, 0.5)
    s_w = synth.uniform_f32((N, K // 128), 66, 1e-5, 1e-3)
    y = oracle.scaled_mm_group128_act_f16(a, b, s_x, s_w)
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for gi in range(K // 128):
                p = int(np.dot(a[m, 128 * gi:128 * gi + 128].astype(np.int64),
                               b[n, 128 * gi:128 * gi + 128].astype(np.int64)))
                sc = fp32(Fraction(float(s_x[m, gi])) * Fraction(float(s_w[n, gi])))
                acc = fp32(Fraction(p) * sc + acc)
            assert Fraction(oracle.f16_to_f32(int(y[m, n]))) == f16(acc), (m, n)


def test_f16_and_bf16_epilogues_round_the_same_fp32_value():
    """Both output formats round one fp32 value: each is the nearest of its
    format to a common fp32 v (checked through the bf16 output's own
    rounding bracket)."""
    M, N, K = 4, 64, 384
    a = synth.int8_uniform((M, K), seed=71)
    b = synth.int8_uniform((N, K), seed=72)
    s_tok = synth.uniform_f32((M,), 73, 1e-3, 0.1)
    s_ch = synth.uniform_f32((N,), 74, 1e-4, 1e-3)
    yb = oracle.scaled_mm(a, b, s_tok, s_ch)
    yh = oracle.scaled_mm_f16(a, b, s_tok, s_ch)
    vb = (yb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    vh = yh.view(np.float16).astype(np.float64)
    assert np.all(np.abs(vb - vh) <= np.abs(vh) * (2.0 ** -8 + 2.0 ** -11) + 1e-30)


def test_w8a16_ref_f16_matches_torch_fp64():
    """The fp16-activation W8A16 reference against torch's fp64 matmul of
    the decoded operands (numpy's fp16 decode), channel scale applied after."""
    M, N, K = 5, 96, 384
    g = np.random.default_rng(12)
    x = (g.standard_normal((M, K)) * 3).astype(np.float16)
    wq = synth.int8_uniform((N, K), seed=13, lo=-127)
    s_ch = synth.uniform_f32((N,), 14, 1e-4, 1e-2)
    y, mag = oracle.w8a16_ref_f16(x.view(np.uint16), wq, s_ch, with_mag=True)
    xt = torch.from_numpy(x.astype(np.float64))
    wt = torch.from_numpy(wq.astype(np.float64))
    ref = (xt @ wt.T).numpy() * s_ch.astype(np.float64)[None, :]
    assert np.all(np.abs(y - ref) <= 1e-12 * mag + 1e-300)
    np.testing.assert_allclose(mag, (xt.abs() @ wt.abs().T).numpy() * s_ch.astype(np.float64)[None, :], rtol=1e-12)
