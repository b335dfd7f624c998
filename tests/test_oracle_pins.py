"""Pins for the CPU oracle: checks against what the pages and mathematics fix.

None of these tests re-types the oracle's formula.  They use exact rational
arithmetic (``tests/exact.py``), library routines (numpy integer matmul,
torch's bf16 cast, torch fp64 matmul), closed forms, constructed special cases
with known answers (``tests/golden/``) and invariants.  A plausible mistake in
the oracle (a dropped term, a wrong sign, a transposed operand, a multiply by a
reciprocal instead of a divide, round-half-up instead of half-even, a swapped
scale) fails at least one of them.

Definitions pinned (page title, section):
  per-token dynamic INT8 activations, per-channel symmetric INT8 weights --
    "Qwen3.8-27B -- SmoothQuant + activation-aware GPTQ, W8A8 INT8 (v3)",
    "Recipe"; "Qwen3.8-27B-INT8-W8A8", "Quantization";
  group size 128, symmetric, natural K order --
    "Qwen3.8-27B-GPTQ-INT8-W8A8-GS128", "Quantization details";
  the smoothing fold preserves the function, weight ratio is separable --
    "Qwen3.8-27B -- FP8 block + AWQ", "Recipe".
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.exact import bf16, bf16_bits_of, bf16_bits_value, fp32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bits(values) -> np.ndarray:
    return synth.bf16_bits(torch.tensor(values, dtype=torch.float32).to(
        torch.bfloat16))


def _f32(bits_u16: np.ndarray) -> np.ndarray:
    return (bits_u16.astype(np.uint32) << 16).view(np.float32)


# ------------------------------------------------------------- bf16 RNE --

def test_bf16_rounding_matches_torch_cast():
    rng = np.random.default_rng(1234)
    vals = list(rng.standard_normal(3000).astype(np.float32) *
                np.float32(1000.0))
    # exact ties: bit patterns whose low 16 bits are 0x8000, odd and even
    for hi in (0x3F80, 0x3F81, 0x4120, 0x4121, 0xBF80, 0xBF81, 0x0001):
        vals.append(np.uint32((hi << 16) | 0x8000).view(np.float32))
        vals.append(np.uint32((hi << 16) | 0x7FFF).view(np.float32))
        vals.append(np.uint32((hi << 16) | 0x8001).view(np.float32))
    vals += [np.float32(0.0), np.float32(-0.0), np.float32(3.4e38),
             np.float32(1e-40), np.float32(-1e-40)]
    arr = np.array(vals, np.float32)
    ref = synth.bf16_bits(torch.from_numpy(arr).to(torch.bfloat16))
    got = np.array([oracle.f32_to_bf16(float(v)) for v in arr], np.uint16)
    np.testing.assert_array_equal(got, ref)


# --------------------------------------------- per-token quantization ---

def _golden_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            rows.append([p.split() for p in line.split("|")])
    return rows


def test_quant_golden_ties():
    for (scale,), xs, qs in _golden_rows("quant_rne_ties.txt"):
        x = _bits([float(v) for v in xs])
        assert np.array_equal(_f32(x), np.array([float(v) for v in xs],
                                                np.float32)), "not bf16-exact"
        xq, s = oracle.quant_per_token(x[None, :])
        assert s[0] == np.float32(float(scale))
        np.testing.assert_array_equal(xq[0], np.array([int(q) for q in qs]))


def test_quant_exact_rational_tiny():
    """Every code of the tiny workload from exact rationals, one rounding each."""
    x = synth.bf16_bits(synth.activations(synth.WORKLOADS["tiny"], seed=0))
    xq, s = oracle.quant_per_token(x)
    M, K = x.shape
    for m in range(M):
        vals = [bf16_bits_value(int(b)) for b in x[m]]
        a = max(abs(v) for v in vals)
        s_ref = fp32(a / 127)
        assert Fraction(float(s[m])) == s_ref
        for k in range(K):
            t = fp32(vals[k] / s_ref)
            q = round(t)  # Python rounds half to even
            q = max(-127, min(127, q))
            assert xq[m, k] == q, (m, k)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_quant_fp64_route_and_invariants(seed):
    """fl32(x/s) == fl32(fl64(x)/fl64(s)) (double rounding is innocuous for
    division when 53 >= 2*24+2), then numpy's half-even rint."""
    xb = synth.bf16_bits(synth.activations(synth.WORKLOADS["decode"], seed))
    xb = np.concatenate([xb, np.zeros((1, xb.shape[1]), np.uint16)])
    xq, s = oracle.quant_per_token(xb)
    x = _f32(xb).astype(np.float64)
    a = np.abs(x).max(axis=1)
    s_ref = (a / 127.0).astype(np.float32)
    np.testing.assert_array_equal(s, s_ref)
    sd = s_ref.astype(np.float64)[:, None]
    with np.errstate(invalid="ignore", divide="ignore"):
        t = np.where(sd > 0, (x / sd), 0.0).astype(np.float32)
    q_ref = np.clip(np.rint(t), -127, 127).astype(np.int8)
    np.testing.assert_array_equal(xq, q_ref)
    # invariants: range, the absmax element maps to +-127, round-trip bound
    assert np.abs(xq.astype(np.int32)).max() <= 127
    for m in range(xb.shape[0] - 1):
        j = int(np.argmax(np.abs(x[m])))
        assert abs(int(xq[m, j])) == 127
    rt = np.abs(x - xq.astype(np.float64) * sd)
    assert np.all(rt <= sd * (0.5 + 2.0 ** -16))
    assert s[-1] == 0 and not xq[-1].any()


def test_quant_divides_rather_than_multiplying_by_reciprocal():
    """Rows built from the bf16 values where rne(fl32(x/s)) and
    rne(fl32(x*fl32(1/s))) disagree: the oracle must take the division."""
    allbf = (np.arange(0, 0x7F80, dtype=np.uint32) << 16).view(np.float32)
    rng = np.random.default_rng(0)
    rows = []
    for _ in range(300):
        a = allbf[rng.integers(0x3F00, 0x4400)]
        s = np.float32(np.float64(a) / 127.0)
        xs = allbf[allbf <= a]
        qd = np.rint((xs.astype(np.float64) / np.float64(s)).astype(np.float32))
        qr = np.rint((xs * (np.float32(1.0) / s)).astype(np.float32))
        idx = np.nonzero(qd != qr)[0]
        if len(idx):
            row = np.concatenate([[a], xs[idx], -xs[idx]]).astype(np.float32)
            rows.append((row, np.concatenate([[127], qd[idx], -qd[idx]])))
    assert len(rows) >= 10
    for row, expect in rows:
        xq, s = oracle.quant_per_token(_bits(row.tolist())[None, :])
        np.testing.assert_array_equal(xq[0], expect.astype(np.int8))


def test_weight_quant_per_channel_and_group128():
    w = synth.weights(synth.WORKLOADS["tiny"], seed=3).numpy()
    w[5, :] = 0.0
    wq, s = oracle.quant_weight(w)
    a = np.abs(w.astype(np.float64)).max(axis=1)
    np.testing.assert_array_equal(s, (a / 127.0).astype(np.float32))
    sd = s.astype(np.float64)[:, None]
    with np.errstate(invalid="ignore", divide="ignore"):
        t = np.where(sd > 0, w / sd, 0.0).astype(np.float32)
    np.testing.assert_array_equal(wq, np.clip(np.rint(t), -127, 127))
    assert s[5] == 0 and not wq[5].any()
    # group 128: contiguous blocks [128g, 128g+128), scale = block absmax/127
    wq2, s2 = oracle.quant_weight(w, group=128)
    N, K = w.shape
    blocks = np.abs(w.astype(np.float64)).reshape(N, K // 128, 128).max(axis=2)
    np.testing.assert_array_equal(s2, (blocks / 127.0).astype(np.float32))
    for g in range(K // 128):
        sub = w[:, 128 * g:128 * (g + 1)]
        q_sub, s_sub = oracle.quant_weight(np.ascontiguousarray(sub))
        np.testing.assert_array_equal(wq2[:, 128 * g:128 * (g + 1)], q_sub)
        np.testing.assert_array_equal(s2[:, g], s_sub)
    with pytest.raises(ValueError):
        oracle.quant_weight(w[:, :200], group=128)


# ------------------------------------------------------ INT32 GEMM ------

def test_mm_i32_brute_force_and_library():
    a = synth.int8_uniform((16, 256), seed=0)
    b = synth.int8_uniform((128, 256), seed=1)
    acc = oracle.mm_i32(a, b)
    # library route: numpy int64 matmul (exact)
    np.testing.assert_array_equal(acc, a.astype(np.int64) @ b.astype(np.int64).T)
    # pure-Python brute force on a few entries
    for (m, n) in [(0, 0), (15, 127), (7, 64), (3, 5)]:
        ref = sum(int(a[m, k]) * int(b[n, k]) for k in range(256))
        assert acc[m, n] == ref


def test_mm_i32_one_hot_rows():
    a = synth.int8_uniform((9, 384), seed=2, lo=-127, hi=127)
    b = np.zeros((6, 384), np.int8)
    idx = [0, 5, 127, 128, 200, 383]
    for n, i in enumerate(idx):
        b[n, i] = 127
    acc = oracle.mm_i32(a, b)
    for n, i in enumerate(idx):
        np.testing.assert_array_equal(acc[:, n], 127 * a[:, i].astype(np.int32))


def test_mm_i32_extremes_and_overflow():
    K = 4096
    a = np.full((2, K), -128, np.int8)
    b = np.full((3, K), -128, np.int8)
    b[1] = 127
    acc = oracle.mm_i32(a, b)
    assert acc[0, 0] == 128 * 128 * K and acc[0, 1] == -128 * 127 * K
    a_big = np.full((1, 131072), -128, np.int8)
    with pytest.raises(OverflowError):
        oracle.mm_i32(a_big, a_big)


# -------------------------------------------------------- epilogue ------

def test_epilogue_exact_rational():
    rng = np.random.default_rng(7)
    acc = rng.integers(-82_000_000, 82_000_000, size=(6, 40)).astype(np.int32)
    acc[0, :5] = [0, 1, -1, 16_777_217, -16_777_219]  # int->fp32 rounding
    s_tok = synth.uniform_f32((6,), 1, 1e-3, 0.5)
    s_ch = synth.uniform_f32((40,), 2, 1e-5, 1e-3)
    y = oracle.epilogue_channel(acc, s_tok, s_ch)
    for m in range(6):
        for n in range(40):
            v = fp32(Fraction(int(acc[m, n])))
            v = fp32(v * Fraction(float(s_tok[m])))
            v = fp32(v * Fraction(float(s_ch[n])))
            assert y[m, n] == bf16_bits_of(bf16(v)), (m, n)


def test_epilogue_product_order_targeted():
    """Triples where (acc*s_tok)*s_ch and (acc*s_ch)*s_tok round to different
    bf16 values: the oracle follows the token-scale-first order."""
    rng = np.random.default_rng(11)
    acc = rng.integers(-80_000_000, 80_000_000, size=4_000_000).astype(np.int32)
    st = rng.uniform(1e-3, 1.0, size=4_000_000).astype(np.float32)
    sc = rng.uniform(1e-5, 1e-2, size=4_000_000).astype(np.float32)
    fa = acc.astype(np.float32)
    y1 = synth.bf16_bits(torch.from_numpy((fa * st) * sc).to(torch.bfloat16))
    y2 = synth.bf16_bits(torch.from_numpy((fa * sc) * st).to(torch.bfloat16))
    idx = np.nonzero(y1 != y2)[0][:64]
    assert len(idx) >= 4
    for i in idx:
        y = oracle.epilogue_channel(acc[i:i + 1].reshape(1, 1), st[i:i + 1],
                                    sc[i:i + 1])
        v = fp32(Fraction(int(acc[i])))
        v = fp32(v * Fraction(float(st[i])))
        v = fp32(v * Fraction(float(sc[i])))
        assert y[0, 0] == bf16_bits_of(bf16(v))


def test_epilogue_unit_scales_is_identity_on_small_ints():
    acc = np.arange(-256, 257, dtype=np.int32).reshape(1, -1)
    y = oracle.epilogue_channel(acc, np.ones(1, np.float32),
                                np.ones(acc.shape[1], np.float32))
    np.testing.assert_array_equal(_f32(y[0]), acc[0].astype(np.float32))


def test_scaled_mm_equals_mm_then_epilogue():
    a = synth.int8_uniform((5, 512), seed=11)
    b = synth.int8_uniform((24, 512), seed=12)
    s_tok = synth.uniform_f32((5,), 3, 1e-3, 1.0)
    s_ch = synth.uniform_f32((24,), 4, 1e-4, 1e-2)
    acc = a.astype(np.int64) @ b.astype(np.int64).T  # library route
    y1 = oracle.scaled_mm(a, b, s_tok, s_ch)
    y2 = oracle.epilogue_channel(acc.astype(np.int32), s_tok, s_ch)
    np.testing.assert_array_equal(y1, y2)


# ------------------------------------------------------- group 128 ------

def test_group128_exact_rational_chain():
    M, N, K = 3, 5, 512
    a = synth.int8_uniform((M, K), seed=21)
    b = synth.int8_uniform((N, K), seed=22)
    s_tok = synth.uniform_f32((M,), 5, 1e-3, 0.5)
    s_grp = synth.uniform_f32((N, K // 128), 6, 1e-5, 1e-3)
    y = oracle.scaled_mm_group128(a, b, s_tok, s_grp)
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for g in range(K // 128):
                p = int(np.dot(a[m, 128 * g:128 * g + 128].astype(np.int64),
                               b[n, 128 * g:128 * g + 128].astype(np.int64)))
                # fused multiply-add: one rounding of the exact p*s + acc
                acc = fp32(Fraction(p) * Fraction(float(s_grp[n, g])) + acc)
            v = fp32(acc * Fraction(float(s_tok[m])))
            assert y[m, n] == bf16_bits_of(bf16(v)), (m, n)


def test_group128_accumulates_in_ascending_group_order():
    """p0*s0 = 2^24, p1*s1 = 1, p2*s2 = -2^24: ascending fma order gives 0
    (2^24 + 1 ties to 2^24), descending order would give 1."""
    K = 384
    a = np.zeros((1, K), np.int8)
    b = np.zeros((1, K), np.int8)
    a[0, [0, 128, 256]] = 1
    b[0, 0], b[0, 128], b[0, 256] = 64, 1, -64
    s_grp = np.array([[2.0 ** 18, 1.0, 2.0 ** 18]], np.float32)
    y = oracle.scaled_mm_group128(a, b, np.ones(1, np.float32), s_grp)
    assert y[0, 0] == 0
    b[0, 0], b[0, 256] = -64, 64  # mirrored: ascending now gives +1
    y = oracle.scaled_mm_group128(a, b, np.ones(1, np.float32), s_grp)
    assert _f32(y)[0, 0] == 1.0


def test_group128_reduces_to_per_channel_within_bound():
    M, N, K = 4, 32, 1024
    a = synth.int8_uniform((M, K), seed=31, lo=-127, hi=127)
    b = synth.int8_uniform((N, K), seed=32, lo=-127, hi=127)
    s_tok = synth.uniform_f32((M,), 7, 1e-3, 0.5)
    s_ch = synth.uniform_f32((N,), 8, 1e-4, 1e-2)
    s_grp = np.repeat(s_ch[:, None], K // 128, axis=1)
    yg = _f32(oracle.scaled_mm_group128(a, b, s_tok, s_grp)).astype(np.float64)
    yc = _f32(oracle.scaled_mm(a, b, s_tok, s_ch)).astype(np.float64)
    ai = a.astype(np.int64)
    bi = b.astype(np.int64)
    absum = np.zeros((M, N))
    for g in range(K // 128):
        sl = slice(128 * g, 128 * g + 128)
        absum += np.abs(ai[:, sl] @ bi[:, sl].T)
    bound = (2.0 ** -8) * (np.abs(yg) + np.abs(yc)) + (K // 128 + 3) * \
        2.0 ** -23 * absum * s_ch[None, :] * s_tok[:, None]
    assert np.all(np.abs(yg - yc) <= bound)
    with pytest.raises(ValueError):
        oracle.scaled_mm_group128(a[:, :200], b[:, :200], s_tok,
                                  np.ones((N, 1), np.float32))


# ------------------------------------------------------------ W8A16 -----

def test_w8a16_ref_matches_torch_fp64():
    xb = synth.bf16_bits(synth.activations(synth.WORKLOADS["w8a16"], seed=0,
                                           M=12, K=384))
    wq = synth.int8_uniform((20, 384), seed=41, lo=-127, hi=127)
    s_ch = synth.uniform_f32((20,), 9, 1e-4, 1e-2)
    y, mag = oracle.w8a16_ref(xb, wq, s_ch, with_mag=True)
    xt = torch.from_numpy(_f32(xb).astype(np.float64))
    wt = torch.from_numpy(wq.astype(np.float64))
    ref = (xt @ wt.T) * torch.from_numpy(s_ch.astype(np.float64))[None, :]
    assert np.all(np.abs(y - ref.numpy()) <= 1e-12 * mag + 1e-300)
    mref = (xt.abs() @ wt.abs().T) * torch.from_numpy(
        s_ch.astype(np.float64))[None, :]
    np.testing.assert_allclose(mag, mref.numpy(), rtol=1e-12)


# ------------------------------------------------------- smoothing fold -

def test_smooth_scales_golden():
    rows = _golden_rows("smooth_scales.txt")
    cmax = [float(r[0][0]) for r in rows]
    expect = np.array([float(r[1][0]) for r in rows], np.float32)
    x = np.zeros((3, len(cmax)), np.float32)
    sign = np.where(np.arange(len(cmax)) % 2 == 0, 1.0, -1.0)
    x[0] = sign * np.array(cmax)  # odd columns: the largest magnitude is < 0
    x[1] = [v / 2 for v in cmax]
    x[2] = [-v / 4 for v in cmax]
    s = oracle.smooth_scales(_bits(x.tolist()))
    np.testing.assert_array_equal(s, expect)
    with pytest.raises(ValueError):
        oracle.smooth_scales(np.zeros((2, 4), np.uint16))


def test_smooth_fold_power_of_two_is_exact_identity():
    """With power-of-two scales the fold is exact: X'W'^T == XW^T bit for bit
    in fp64, and W'/W is the separable rank-1 ratio 1 * s^T."""
    rng = np.random.default_rng(5)
    M, N, K = 24, 16, 64
    x = rng.standard_normal((M, K)).astype(np.float32)
    targets = 4.0 ** rng.integers(-3, 6, size=K)  # column maxima 4^t
    x = np.clip(x, -1.0, 1.0) * 0.5 * targets[None, :]
    x[0] = targets
    xb = _bits(x.tolist())
    w = synth.weights(synth.WORKLOADS["tiny"], seed=9, N=N, K=K).numpy()
    s = oracle.smooth_scales(xb)
    np.testing.assert_array_equal(
        s, np.minimum(16.0, np.sqrt(targets)).astype(np.float32))
    xo = oracle.smooth_fold_x(xb, s)
    wo = oracle.smooth_fold_w(w, s)
    lhs = _f32(xo).astype(np.float64) @ wo.astype(np.float64).T
    rhs = _f32(xb).astype(np.float64) @ w.astype(np.float64).T
    np.testing.assert_array_equal(lhs, rhs)
    ratio = wo.astype(np.float64) / w.astype(np.float64)
    np.testing.assert_array_equal(ratio, np.broadcast_to(s, (N, K)))


def test_smooth_fold_general_within_rounding():
    wl = synth.WORKLOADS["prefill"]
    xb = synth.bf16_bits(synth.activations(wl, seed=0, M=64, K=512))
    w = synth.weights(wl, seed=0, N=32, K=512).numpy()
    s = oracle.smooth_scales(xb)
    xo = oracle.smooth_fold_x(xb, s)
    wo = oracle.smooth_fold_w(w, s)
    xf = _f32(xb).astype(np.float64)
    lhs = _f32(xo).astype(np.float64) @ wo.astype(np.float64).T
    rhs = xf @ w.astype(np.float64).T
    mag = np.abs(xf) @ np.abs(w.astype(np.float64)).T
    # X' rounded to bf16 (rel 2^-8 incl. the fp32 quotient), W' to fp32
    assert np.all(np.abs(lhs - rhs) <= mag * (2.0 ** -8 + 2.0 ** -22))
    # rank-1 separable ratio, to fp32 rounding
    ratio = wo.astype(np.float64) / w.astype(np.float64)
    assert np.all(np.abs(ratio / s.astype(np.float64)[None, :] - 1) <= 2.0 ** -24)


def _bf16_of_f32(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 (torch's RNE cast), returned as fp32 values."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16).float().numpy()


def test_smooth_fold_x_divides_rather_than_multiplying_by_reciprocal():
    """X' = bf16(fl32(x / s)): one correctly rounded division, not x times
    fl32(1/s).  Pairs (x, s) with a general fp32 s where the two routes give
    different bf16 values are found by a float32 search (numpy's float32 '/'
    and '*' are IEEE), confirmed with exact rationals, and the oracle must
    give the quotient's rounding."""
    g = np.random.default_rng(5)
    n = 4_000_000
    s = (1 + 15 * g.random(n)).astype(np.float32)
    x = _bf16_of_f32((g.random(n) * 2 - 1) * 8)
    q_div = _bf16_of_f32(x / s)
    q_rcp = _bf16_of_f32(x * (np.float32(1) / s))
    hit = np.nonzero(q_div != q_rcp)[0]
    assert len(hit) >= 5
    xs, ss = x[hit], s[hit]
    for xv, sv in zip(xs, ss):
        fx, fs = Fraction(float(xv)), Fraction(float(sv))
        stated = bf16(fp32(fx / fs))
        other = bf16(fp32(fx * fp32(1 / fs)))
        assert stated != other
    # one column per pair: the oracle folds x_j by its s_j
    xb = _bits([xs.tolist()])
    out = oracle.smooth_fold_x(xb, ss.astype(np.float32))
    for j, (xv, sv) in enumerate(zip(xs, ss)):
        assert bf16_bits_value(int(out[0, j])) == bf16(fp32(Fraction(float(xv)) / Fraction(float(sv))))


def test_smooth_fold_routes_agree_on_the_folds_own_scales():
    """Within the fold step itself the scale is s = min(16, sqrtf(a)) for a
    bf16 column maximum a, and every |x| <= a.  On that domain the division
    and the reciprocal product give the same bf16 value for every pair:
    exhaustively over every such s with every bf16 significand of x (the
    rounding of a normal quotient depends on the significands only), and
    over every bf16 x small enough for the quotient to be subnormal in fp32.
    So the fold's bf16 outputs cannot tell the two routes apart, and the
    explicit-scale pin above is what fixes the oracle's division."""
    allb = np.arange(1, 0x7F80, dtype=np.uint32)
    vals = (allb << 16).view(np.float32)
    a = vals[vals <= 256]
    s = np.unique(np.minimum(np.float32(16), np.sqrt(a).astype(np.float32)))
    r = np.float32(1) / s
    xm = (1 + np.arange(128) / 128).astype(np.float32)
    for xe in (-1, 0, 1):
        X = (xm * np.float32(2.0 ** xe))[:, None]
        assert np.array_equal(_bf16_of_f32(X / s[None, :]), _bf16_of_f32(X * r[None, :]))
    tiny = vals[vals <= np.float32(2.0 ** -119)]
    for i in range(0, len(tiny), 128):
        X = tiny[i:i + 128][:, None]
        assert np.array_equal(_bf16_of_f32(X / s[None, :]), _bf16_of_f32(X * r[None, :]))


# --------------------------------------------- end to end vs unquantized -

@pytest.mark.parametrize("name", ["tiny", "decode"])
def test_end_to_end_within_quantization_bound(name):
    """|y_q - X W^T| <= sum_k s_t s_c (|qx|/2 + |qw|/2 + 1/4) (+ rounding),
    the closed-form error of symmetric rounding of both operands."""
    wl = synth.WORKLOADS[name]
    M = wl.M if wl.M <= 16 else 16
    N = min(wl.N, 256)
    xb = synth.bf16_bits(synth.activations(wl, seed=0, M=M))
    w = synth.weights(wl, seed=0, N=N).numpy()
    xq, s_tok = oracle.quant_per_token(xb)
    wq, s_ch = oracle.quant_weight(w)
    y = _f32(oracle.scaled_mm(xq, wq, s_tok, s_ch)).astype(np.float64)
    exact = _f32(xb).astype(np.float64) @ w.astype(np.float64).T
    e = 0.5 + 2.0 ** -16
    qx = np.abs(xq.astype(np.float64))
    qw = np.abs(wq.astype(np.float64))
    term = (qx.sum(1)[:, None] * e + qw.sum(1)[None, :] * e +
            wl.K * e * e)
    bound = term * s_tok[:, None].astype(np.float64) * \
        s_ch[None, :].astype(np.float64)
    bound = bound * (1 + 1e-6) + np.abs(y) * 2.0 ** -8 + 1e-30
    assert np.all(np.abs(y - exact) <= bound)
    # and a wrong sign / transposed operand would be far outside it
    assert not np.all(np.abs(-y - exact) <= bound)


# ------------------------------- residual add + RMSNorm + per-token quant --
# Fused normalization before the linear layer: "Qwen3.8-27B -- SmoothQuant +
# activation-aware GPTQ, W8A8 INT8 (v3)", "Recipe" (smoothing folded into the
# preceding norm); "Qwen3.8-27B-GPTQ-INT8-W8A8-GS128", "Serving (vLLM, gfx908
# fork)" (residual add, RMSNorm and INT8 quantization fused).

def _norm_inputs(M, K, seed, scale=1.0):
    g = np.random.default_rng(seed)
    x = synth.bf16_bits(torch.from_numpy((g.standard_normal((M, K)) * scale).astype(np.float32)).to(torch.bfloat16))
    gam = synth.bf16_bits(torch.from_numpy((0.5 + g.random(K)).astype(np.float32)).to(torch.bfloat16))
    return x, gam


def test_rmsnorm_power_of_two_scale_invariance():
    """With eps = 0, RMSNorm of 2^j * x equals RMSNorm of x bit for bit
    (squares, the sum, the mean and the root all scale exactly)."""
    x, gam = _norm_inputs(6, 768, 1)
    ref = oracle.rmsnorm_quant(x, gam, 0.0)
    for j in (-3, 2, 5):
        xs = synth.bf16_bits(torch.from_numpy(_f32(x) * np.float32(2.0 ** j)).to(torch.bfloat16))
        assert np.array_equal(_f32(xs), _f32(x) * np.float32(2.0 ** j))  # exact scaling
        got = oracle.rmsnorm_quant(xs, gam, 0.0)
        for a, b in zip(ref[:3], got[:3]):
            np.testing.assert_array_equal(a, b)


def test_rmsnorm_constant_row_closed_form():
    """Row of ones, eps = 3: mean square 1, rstd = 1/sqrt(4) = 0.5 exactly,
    so y = gamma / 2 exactly (pins the division by K and the + eps)."""
    K = 512
    x = _bits([[1.0] * K, [-1.0] * K])
    _, gam = _norm_inputs(1, K, 2)
    xq, s, y, _ = oracle.rmsnorm_quant(x, gam, 3.0)
    np.testing.assert_array_equal(_f32(y[0]), _f32(gam) / 2)
    np.testing.assert_array_equal(_f32(y[1]), -_f32(gam) / 2)
    np.testing.assert_array_equal(s, np.float32(np.abs(_f32(gam)).max() / 2) / np.float32(127))


@pytest.mark.parametrize("k", [0, 5, 8, 63 * 8 + 7, 64 * 8, 64 * 8 + 3, 100 * 8 + 6, 1023])
def test_rmsnorm_single_element_rows_cover_every_position(k):
    """One nonzero v = -4 at position k of a K = 1024 row, eps = 0: mean
    square 16/1024, rstd = 1/sqrt(1/64) = 8, so y[k] = -32 * gamma[k]
    exactly and zero elsewhere.  A dropped or doubled element in the sum of
    squares changes y[k]."""
    K = 1024
    row = [0.0] * K
    row[k] = -4.0
    x = _bits([row])
    _, gam = _norm_inputs(1, K, 3)
    xq, s, y, _ = oracle.rmsnorm_quant(x, gam, 0.0)
    expect = np.zeros(K, np.float32)
    expect[k] = -32.0 * _f32(gam)[k]
    np.testing.assert_array_equal(_f32(y[0]), expect)
    assert xq[0, k] == -127 and np.count_nonzero(xq[0]) == 1


def test_rmsnorm_matches_torch_rms_norm():
    """Against torch's RMSNorm in fp32 (its own summation order and rsqrt):
    every output within 1 bf16 ulp, nearly all identical."""
    M, K = 16, 5120
    x, gam = _norm_inputs(M, K, 4, scale=3.0)
    eps = 1e-6
    _, _, y, _ = oracle.rmsnorm_quant(x, gam, eps)
    h = torch.from_numpy(_f32(x))
    t = torch.nn.functional.rms_norm(h, (K,), torch.from_numpy(_f32(gam)), eps)
    tb = synth.bf16_bits(t.to(torch.bfloat16))

    def ordered(u):
        u = u.astype(np.int32)
        return np.where(u & 0x8000, -(u & 0x7FFF), u)
    d = np.abs(ordered(y) - ordered(tb))
    assert d.max() <= 1 and (d == 0).mean() > 0.99


def test_rmsnorm_residual_add_matches_torch_bf16_add():
    """The residual stream becomes bf16(x + res) (torch's bf16 addition), and
    the norm is taken of that sum."""
    M, K = 5, 640
    x, gam = _norm_inputs(M, K, 5)
    r, _ = _norm_inputs(M, K, 6, scale=4.0)
    xq, s, y, res_out = oracle.rmsnorm_quant(x, gam, 1e-6, res_bf16=r)
    tsum = synth.bits_to_bf16(x) + synth.bits_to_bf16(r)
    np.testing.assert_array_equal(res_out, synth.bf16_bits(tsum))
    ref = oracle.rmsnorm_quant(res_out, gam, 1e-6)
    for a, b in zip((xq, s, y), ref[:3]):
        np.testing.assert_array_equal(a, b)


def test_rmsnorm_quant_is_the_per_token_quant_of_y():
    x, gam = _norm_inputs(9, 1024, 7)
    xq, s, y, _ = oracle.rmsnorm_quant(x, gam, 1e-6)
    xq2, s2 = oracle.quant_per_token(y)
    np.testing.assert_array_equal(xq, xq2)
    np.testing.assert_array_equal(s, s2)


def test_rmsnorm_rejects_k_not_multiple_of_8():
    x, gam = _norm_inputs(1, 12, 8)
    with pytest.raises(ValueError):
        oracle.rmsnorm_quant(x, gam, 1e-6)


def test_rmsnorm_product_order_targeted():
    """The normalized value is (h * rstd) * gamma, each product rounded to
    fp32, then to bf16.  Rows of K = 256 with h = 1 except one entry v, and
    eps = fl(1/3), so rstd is not a power of two.  Candidate (v, gamma) pairs
    where h * (rstd * gamma) would round to a different bf16 are found with a
    float64 search (every step is a product or quotient of fp32/bf16 values,
    which float64 rounds innocuously to fp32); each found pair is confirmed
    with exact rationals and a correctly rounded root, and the oracle must
    give the stated order."""
    from tests.exact import sqrt_fp32

    def to_bf16_f64(a):  # fp32 values (as float64) -> bf16 RNE (as float64)
        u = a.astype(np.float32).view(np.uint32).astype(np.uint64)
        u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
        return u.astype(np.uint32).view(np.float32).astype(np.float64)

    K = 256
    vs = np.unique(to_bf16_f64(np.linspace(1.0, 4.0, 700)))
    gms = np.unique(to_bf16_f64(np.linspace(0.5, 2.0, 600)))
    pairs = []
    for e in range(400):
        eps32 = np.float32(np.float32(1.0) / np.float32(3.0 + e))
        for v in vs:
            ss = np.float64(K - 1) + v * v
            var = np.float32(ss / K)
            ve = np.float32(np.float64(var) + np.float64(eps32))
            rstd = np.float32(1.0 / np.float64(np.float32(np.sqrt(np.float64(ve)))))
            t = np.float64(np.float32(v * np.float64(rstd)))
            stated = to_bf16_f64(np.float32(t * gms).astype(np.float64))
            rg = np.float32(np.float64(rstd) * gms).astype(np.float64)
            other = to_bf16_f64(np.float32(v * rg).astype(np.float64))
            hit = np.nonzero(stated != other)[0]
            if len(hit):
                pairs.append((float(v), float(gms[hit[0]]), float(eps32)))
                break
        if len(pairs) >= 4:
            break
    assert len(pairs) >= 3
    for v, gm, e32 in pairs:
        v, gm, eps = Fraction(v), Fraction(gm), Fraction(e32)
        ss = Fraction(K - 1) + v * v
        var = fp32(ss / K)
        rstd = fp32(1 / sqrt_fp32(fp32(var + eps)))
        stated = bf16(fp32(fp32(v * rstd) * gm))
        other = bf16(fp32(v * fp32(rstd * gm)))
        assert stated != other  # the float64 search agrees with exact arithmetic
        row = [1.0] * K
        row[100] = float(v)
        gam = [0.75] * K
        gam[100] = float(gm)
        _, _, y, _ = oracle.rmsnorm_quant(_bits([row]), _bits(gam), e32)
        assert bf16_bits_value(int(y[0, 100])) == stated
        assert bf16_bits_value(int(y[0, 0])) == bf16(fp32(fp32(rstd) * Fraction(3, 4)))


def _exact_ss_fp32(row_bits) -> Fraction:
    """The exact sum of the squares of a row of bf16 bits, rounded once to
    fp32, in rational arithmetic."""
    tot = Fraction(0)
    for u in row_bits:
        v = bf16_bits_value(int(u))
        tot += v * v
    return fp32(tot)


def test_rmsnorm_sum_of_squares_is_exact_then_rounded_once():
    """ss is the exact sum of the row's squares rounded once to fp32: checked
    against rational arithmetic on random rows (moderate, wide-range and
    subnormal values, K up to 8192), and on two constructed rows that an
    fp32 running sum and an fp64 running sum each get wrong."""
    g = np.random.default_rng(21)
    rows = [g.standard_normal(5120) * 3,
            g.standard_normal(8192) * 2.0 ** g.integers(-60, 40, 8192),
            g.standard_normal(1024) * 2.0 ** -128,  # subnormal bf16 values
            np.concatenate([[2.0 ** 63], g.standard_normal(511)])]
    for r in rows:
        b = _bits([r.astype(np.float32).tolist()])
        ss = oracle.sum_squares_bf16(b)
        assert Fraction(float(ss[0])) == _exact_ss_fp32(b[0])
    # 2^20 + 17 * 2^-8: the small squares are each below half an fp32 ulp of
    # 2^20 (2^-4), so a running fp32 sum keeps 2^20, but together they pass
    # the midpoint and the exact sum rounds up to 2^20 + 2^-3
    row = [1024.0] + [2.0 ** -4] * 17 + [0.0] * 14
    ss = oracle.sum_squares_bf16(_bits([row]))[0]
    assert ss == np.float32(2.0 ** 20 + 2.0 ** -3)
    run = np.float32(0)
    for v in row:
        run = np.float32(run + np.float32(v) * np.float32(v))
    assert run == np.float32(2.0 ** 20)
    # 2^60 + 2^36 + 2^-40: the first two make an exact fp32 tie, the third
    # breaks it upwards; an fp64 running sum loses 2^-40 and rounds the tie
    # to even (2^60), the exact sum rounds to 2^60 + 2^37
    row = [2.0 ** 30, 2.0 ** 18, 2.0 ** -20] + [0.0] * 5
    ss = oracle.sum_squares_bf16(_bits([row]))[0]
    assert ss == np.float32(2.0 ** 60 + 2.0 ** 37)
    d64 = 0.0
    for v in row:
        d64 += v * v
    assert np.float32(d64) == np.float32(2.0 ** 60)
    # the full step uses the same ss
    ss_step = oracle.rmsnorm_quant(_bits([row]), _bits([[1.0] * 8])[0], 1e-6, return_ss=True)[4]
    assert ss_step[0] == np.float32(2.0 ** 60 + 2.0 ** 37)


def test_rmsnorm_at_ss_reproduces_the_step():
    """The normalization at a given ss (used by the validity check) equals
    the full step when given the step's own ss."""
    x, gam = _norm_inputs(12, 2048, 31, scale=2.0)
    r, _ = _norm_inputs(12, 2048, 32)
    xq, s, y, h, ss = oracle.rmsnorm_quant(x, gam, 1e-5, res_bf16=r, return_ss=True)
    xq2, s2, y2 = oracle.rmsnorm_quant_at_ss(h, gam, 1e-5, ss)
    for a, b in ((xq, xq2), (s, s2), (y, y2)):
        np.testing.assert_array_equal(a, b)


def test_norm_check_accepts_bounded_sums_and_rejects_a_dropped_term():
    """The validity check used on the GPU accepts the outputs at fp32 sums of
    squares a few ulps from the exact one (any summation order within the
    stated bound), and rejects outputs computed from a sum that misses one
    square (an error far outside the bound)."""
    from tests.norm_check import check_rows
    M, K = 64, 5120
    h, gam = _norm_inputs(M, K, 41, scale=1.5)
    ss = oracle.sum_squares_bf16(h)
    off = np.array([0, 1, -1, 3, -4, 7] * (M // 6 + 1))[:M]
    cand = (ss.view(np.int32) + off.astype(np.int32)).view(np.float32)
    xq, s, _ = oracle.rmsnorm_quant_at_ss(h, gam, 1e-6, cand)
    n_exact, n_nb, _ = check_rows(h, gam, 1e-6, xq, s)
    assert n_exact + n_nb == M and n_nb > 0
    drop = h.copy()
    drop[:, 5] = 0  # one square missing from every row's sum
    ss_d = oracle.sum_squares_bf16(drop)
    xq_d, s_d, _ = oracle.rmsnorm_quant_at_ss(h, gam, 1e-6, ss_d)
    changed = np.any(xq_d != oracle.rmsnorm_quant_at_ss(h, gam, 1e-6, ss)[0], axis=1)
    assert changed.sum() > M // 2
    with pytest.raises(AssertionError):
        check_rows(h, gam, 1e-6, xq_d, s_d)


# -------------------- per-token-per-group activations, group-128 weights --
# "Qwen3.8-27B-GPTQ-INT8-W8A8-GS128", "Serving (vLLM, gfx908 fork)"
# (per-group INT8 quant-out before the GEMM) and "Quantization details"
# (group 128, natural K order); "Qwen3.8-27B -- FP8 block + AWQ", "Recipe"
# (dynamic per-group activation scales).

def test_quant_per_group128_is_per_token_quant_of_each_block():
    """Grouping only: each 128-wide block equals the (separately pinned)
    per-token quantizer applied to that block as a row."""
    x = synth.activations(synth.WORKLOADS["decode"], 0)[:, :1024].contiguous()
    xb = synth.bf16_bits(x)
    xq, s = oracle.quant_per_group128(xb)
    M, K = xb.shape
    xq2, s2 = oracle.quant_per_token(xb.reshape(M * K // 128, 128))
    np.testing.assert_array_equal(xq, xq2.reshape(M, K))
    np.testing.assert_array_equal(s, s2.reshape(M, K // 128))
    # invariants: range, block absmax -> +-127, round trip within s/2
    assert np.abs(xq.astype(np.int32)).max() <= 127
    blocks = np.abs(_f32(xb)).reshape(M, K // 128, 128)
    codes = np.abs(xq.astype(np.int32)).reshape(M, K // 128, 128)
    am = blocks.argmax(axis=2)
    assert (np.take_along_axis(codes, am[..., None], 2) == 127).all()
    err = np.abs(_f32(xb).reshape(M, K // 128, 128).astype(np.float64)
                 - xq.reshape(M, K // 128, 128) * s[..., None].astype(np.float64))
    assert (err <= s[..., None] * (0.5 + 2 ** -15)).all()


def test_group128_act_exact_rational_chain():
    """fl32(s_x * s_w) first, then one fused multiply-add per block in
    ascending order, bf16 at the end: exact rationals, one rounding each."""
    M, N, K = 3, 4, 640
    a = synth.int8_uniform((M, K), seed=31)
    b = synth.int8_uniform((N, K), seed=32)
    s_x = synth.uniform_f32((M, K // 128), 33, 1e-3, 0.5)
    s_w = synth.uniform_f32((N, K // 128), 34, 1e-5, 1e-3)
    y = oracle.scaled_mm_group128_act(a, b, s_x, s_w)
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for g in range(K // 128):
                p = int(np.dot(a[m, 128 * g:128 * g + 128].astype(np.int64),
                               b[n, 128 * g:128 * g + 128].astype(np.int64)))
                sc = fp32(Fraction(float(s_x[m, g])) * Fraction(float(s_w[n, g])))
                acc = fp32(Fraction(p) * sc + acc)
            assert y[m, n] == bf16_bits_of(bf16(acc)), (m, n)


def test_group128_act_reduces_to_group128_with_unit_activation_scales():
    """With every activation block scale 1, the result is the group-128
    weight-scale GEMM with token scale 1, bit for bit."""
    M, N, K = 7, 32, 1024
    a = synth.int8_uniform((M, K), seed=35)
    b = synth.int8_uniform((N, K), seed=36)
    s_w = synth.uniform_f32((N, K // 128), 37, 1e-5, 1e-3)
    y = oracle.scaled_mm_group128_act(a, b, np.ones((M, K // 128), np.float32), s_w)
    y2 = oracle.scaled_mm_group128(a, b, np.ones(M, np.float32), s_w)
    np.testing.assert_array_equal(y, y2)


def test_group128_act_scale_product_order_targeted():
    """The block scale is fl32(s_x * s_w), applied to the exact block sum in
    one rounding (not fl32(p * s_x) * s_w).  Scale pairs where the two
    readings give different bf16 results are found by a float64 search
    (products of fp32 values round innocuously from float64), confirmed with
    exact rationals, and the oracle must give the stated one."""
    g = np.random.default_rng(41)
    a = synth.int8_uniform((1, 128), seed=42)
    b = synth.int8_uniform((1, 128), seed=43)
    p = int(np.dot(a[0].astype(np.int64), b[0].astype(np.int64)))
    assert p != 0
    sx = g.uniform(1e-3, 1.0, 400000).astype(np.float32).astype(np.float64)
    sw = g.uniform(1e-4, 1e-2, 400000).astype(np.float32).astype(np.float64)

    def bf16_of(v32):
        u = v32.astype(np.float32).view(np.uint32).astype(np.uint64)
        return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    sc = (sx * sw).astype(np.float32).astype(np.float64)
    stated = bf16_of((p * sc).astype(np.float32))
    other = bf16_of(((p * sx).astype(np.float32).astype(np.float64) * sw).astype(np.float32))
    idx = np.nonzero(stated != other)[0][:3]
    assert len(idx) >= 2
    for i in idx:
        fx, fw = Fraction(float(sx[i])), Fraction(float(sw[i]))
        exact_stated = bf16(fp32(Fraction(p) * fp32(fx * fw)))
        exact_other = bf16(fp32(fp32(Fraction(p) * fx) * fw))
        assert exact_stated != exact_other
        y = oracle.scaled_mm_group128_act(a, b, np.array([[sx[i]]], np.float32),
                                          np.array([[sw[i]]], np.float32))
        assert bf16_bits_value(int(y[0, 0])) == exact_stated
