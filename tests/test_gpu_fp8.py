"""GPU parity of the FP8 block W8A8 path against the CPU oracle.

Codes and scales of both quantizers must be bit-exact.  The GEMM runs on the
FP8 matrix cores (v_mfma_f32_32x32x64_f8f6f4), which do not sum products in
fp32: measured on this hardware, each group of 8 consecutive products of a
K block is aligned to the group's largest product with 13 fractional bits
and truncated; the group sums are then combined exactly enough not to show
in the same measurement.  The GEMM is therefore checked against the
oracle's exact (fp64) value with the bound of that arithmetic:
  |y - ref| <= 2^-8 |ref|                        (bf16 rounding of the result)
             + sum_g |s_x s_w| sum_groups sum_k min(|p_k|, 2^-12 max_group |p|)
                                                 (truncation inside a group,
                                                  with a factor 2 of slack on
                                                  the grid)
             + 1.01 (K/128 + 130) 2^-24 mag      (fp32 sums, scale product and
                                                  one fused multiply-add per
                                                  block)
where mag = sum_g |s_x s_w| sum_k |a b|.  A wrong scale, block or operand
gives errors of the size of ref itself.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import synth
import w8a8_int8_gemm_token_amd as q8

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True, file=sys.stderr)


def dev(t):
    if isinstance(t, np.ndarray):
        t = torch.from_numpy(np.ascontiguousarray(t))
    return t.to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu()


def bits(t_bf16_cpu):
    return synth.bf16_bits(t_bf16_cpu)


def u8(t_fp8):
    return host(t_fp8).view(torch.uint8).numpy()


_E4M3 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()


def group8_truncation_bound(xq, wq, sx, sw):
    """sum_g |s_x s_w| sum over groups of 8 consecutive k of
    sum_k min(|p_k|, 2^-12 max_group |p|), p_k = a[m,k] b[n,k]."""
    M, K = xq.shape
    N, G = wq.shape[0], K // 128
    A, W = _E4M3[xq], _E4M3[wq]
    out = np.empty((M, N))
    step = max(1, 4_000_000 // (N * K))
    for m0 in range(0, M, step):
        P = np.abs(A[m0:m0 + step, None, :] * W[None, :, :]).reshape(-1, N, K // 8, 8)
        t = np.minimum(P, P.max(axis=3, keepdims=True) * 2.0 ** -12).sum(axis=3)
        t = t.reshape(-1, N, G, 16).sum(axis=3)
        sc = np.abs(sx[m0:m0 + step, None, :].astype(np.float64) * sw[np.arange(N) // 128][None].astype(np.float64))
        out[m0:m0 + step] = (t * sc).sum(axis=2)
    return out


def check_fp8_mm(y_gpu, xq, wq, sx, sw, what, rows=None):
    K = xq.shape[1]
    y_ref, mag = oracle.fp8_block_mm(xq, wq, sx, sw, with_mag=True)
    y = host(y_gpu).float().numpy().astype(np.float64)
    if rows is not None:
        y = y[rows]
    err = np.abs(y - y_ref)
    bound = (2.0 ** -8 * np.abs(y_ref) + group8_truncation_bound(xq, wq, sx, sw)
             + 1.01 * (K / 128 + 130) * 2.0 ** -24 * mag)
    ratio = (err / np.maximum(bound, 1e-300)).max() if err.size else 0.0
    rel = np.linalg.norm(y - y_ref, axis=1) / np.maximum(np.linalg.norm(y_ref, axis=1), 1e-30)
    say(f"{what}: max err/bound {ratio:.3f}, max row rel {rel.max() if rel.size else 0:.2e}")
    assert np.all(err <= bound), what
    assert rel.size == 0 or rel.max() <= 1e-2, what


@pytest.mark.parametrize("M,K,pad", [(1, 128, 0), (3, 640, 8), (8, 5120, 0), (130, 1024, 16),
                                     (33, 4096, 0)])
def test_fp8_quant_per_group128(M, K, pad):
    say("fp8 quant per group128", M, K, pad)
    xf, _ = synth.custom(M, K + pad, 16, seed=M + 7 * K, outlier_cols=max(1, K // 100))
    x = xf[:, :K].contiguous()
    x[M // 2, :128] = 0              # an all-zero block
    x[0, K - 128:] = -0.0            # a block of negative zeros
    xf[:, :K] = x
    xq_ref, s_ref = oracle.quant_fp8_per_group128(bits(x))
    xq, s = q8.q8_quant_fp8_per_group128(dev(xf)[:, :K])
    np.testing.assert_array_equal(host(s).numpy(), s_ref)
    np.testing.assert_array_equal(u8(xq), xq_ref)


def test_fp8_quant_near_halfway_subnormal_range_and_tiny_scales():
    """Blocks built from bf16 values whose quotient and reciprocal product
    round to different E4M3 codes, values that land in the E4M3 subnormal
    range, exact halfway quotients, and blocks with subnormal scales."""
    allbf = (np.arange(0, 0x7F80, dtype=np.uint32) << 16).view(np.float32)
    rng = np.random.default_rng(3)
    blocks = []
    for _ in range(400):
        a = allbf[rng.integers(0x3F00, 0x4400)]
        s = np.float32(np.float32(a) / np.float32(448.0))
        xs = allbf[allbf <= a]
        q_div = torch.from_numpy((xs / s).astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        q_rec = torch.from_numpy((xs * (np.float32(1.0) / s)).astype(np.float32)).to(
            torch.float8_e4m3fn).view(torch.uint8).numpy()
        idx = np.nonzero(q_div != q_rec)[0][:60]
        low = xs[(xs / s >= 2.0 ** -11) & (xs / s < 2.0 ** -5)][:40]  # E4M3 subnormal range
        blk = np.concatenate([[a], xs[idx], -xs[idx], low, -low])[:128]
        blocks.append(np.pad(blk, (0, 128 - len(blk))).astype(np.float32))
    # exact halfway quotients: absmax 448 gives s = 1, values at code midpoints
    vals = np.array([oracle.e4m3_value(c) for c in range(0x7F)])
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    mids = mids[torch.from_numpy(mids).to(torch.bfloat16).float().numpy() == mids]
    for i in range(0, len(mids), 120):
        blk = np.concatenate([[448.0], mids[i:i + 120]])
        blocks.append(np.pad(blk, (0, 128 - len(blk))).astype(np.float32))
    for amax in (1e-38, 2e-37, 1e-40):  # subnormal and near-subnormal scales
        blk = np.zeros(128, np.float32)
        blk[:7] = np.array([1, 0.5, -0.25, 0.75, 0.3, -1, 0.01], np.float32) * amax
        blocks.append(blk)
    nb = len(blocks) + (-len(blocks)) % 4
    mat = np.zeros((nb, 128), np.float32)
    mat[:len(blocks)] = np.stack(blocks)
    x = torch.from_numpy(mat.reshape(nb // 4, 512)).to(torch.bfloat16)
    xq_ref, s_ref = oracle.quant_fp8_per_group128(bits(x))
    xq, s = q8.q8_quant_fp8_per_group128(dev(x))
    np.testing.assert_array_equal(host(s).numpy(), s_ref)
    np.testing.assert_array_equal(u8(xq), xq_ref)


@pytest.mark.parametrize("N,K", [(128, 128), (384, 640), (256, 5120)])
def test_fp8_quant_weight_block128(N, K):
    say("fp8 weight blocks", N, K)
    _, w = synth.custom(4, K, N, seed=N + K)
    w = w.numpy().copy()
    w[:128, :128] *= 100.0  # blocks of different magnitudes
    w[N - 1, K - 1] = 1.0   # a block maximum in a corner
    wq_ref, s_ref = oracle.quant_weight_fp8_block128(w)
    wq, s = q8.q8_quant_weight_fp8_block128(dev(w))
    np.testing.assert_array_equal(host(s).numpy(), s_ref)
    np.testing.assert_array_equal(u8(wq), wq_ref)


@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (8, 256, 1024), (64, 384, 640),
                                   (65, 256, 1152), (130, 512, 384), (200, 384, 2048),
                                   (257, 128, 256),
                                   # tiles by workgroup count: 64 x 128, then 128 x 128
                                   (300, 5120, 256), (600, 5120, 256)])
def test_fp8_block_scaled_mm_shapes(M, N, K):
    say("fp8 block mm", M, N, K)
    x, w = synth.custom(M, K, N, seed=M * 5 + N, outlier_cols=3)
    xq, sx = q8.q8_quant_fp8_per_group128(dev(x))
    wq, sw = q8.q8_quant_weight_fp8_block128(dev(w))
    xq_ref, sx_ref = oracle.quant_fp8_per_group128(bits(x))
    wq_ref, sw_ref = oracle.quant_weight_fp8_block128(w.numpy())
    np.testing.assert_array_equal(u8(xq), xq_ref)
    np.testing.assert_array_equal(host(sx).numpy(), sx_ref)
    np.testing.assert_array_equal(u8(wq), wq_ref)
    np.testing.assert_array_equal(host(sw).numpy(), sw_ref)
    y = q8.q8_fp8_block_scaled_mm(xq, wq, sx, sw)
    check_fp8_mm(y, xq_ref, wq_ref, sx_ref, sw_ref, f"fp8 {M}x{N}x{K}")


def test_fp8_block_scaled_mm_strided_and_zero_rows():
    M, N, K = 70, 256, 768
    x, w = synth.custom(M, K, N, seed=91, outlier_cols=2)
    x[5] = 0
    xq, sx = q8.q8_quant_fp8_per_group128(dev(x))
    wq, sw = q8.q8_quant_weight_fp8_block128(dev(w))
    a = torch.zeros((M, K + 64), dtype=torch.float8_e4m3fn, device=DEV)
    a[:, :K] = xq
    b = torch.zeros((N, K + 32), dtype=torch.float8_e4m3fn, device=DEV)
    b[:, :K] = wq
    out = torch.full((M, N + 8), 7.0, dtype=torch.bfloat16, device=DEV)
    q8.q8_fp8_block_scaled_mm(a[:, :K], b[:, :K], sx, sw, out=out[:, :N])
    o = host(out)
    assert (o[:, N:] == 7.0).all()
    assert (o[5, :N] == 0).all()
    xq_ref, sx_ref = oracle.quant_fp8_per_group128(bits(x))
    wq_ref, sw_ref = oracle.quant_weight_fp8_block128(w.numpy())
    np.testing.assert_array_equal(u8(xq), xq_ref)
    np.testing.assert_array_equal(host(sx).numpy(), sx_ref)
    np.testing.assert_array_equal(u8(wq), wq_ref)
    np.testing.assert_array_equal(host(sw).numpy(), sw_ref)
    check_fp8_mm(out[:, :N], xq_ref, wq_ref, sx_ref, sw_ref, "fp8 strided")


def test_fp8_full_size_sampled_rows():
    """The FP8 workload at its full size (M=8192, N=15360, K=5120), in the
    launch configuration the benchmark times; sampled rows against the
    oracle, codes and scales checked whole."""
    wl = synth.WORKLOADS["fp8_block"]
    say("fp8 full size")
    x = synth.activations(wl, 0)
    w = synth.weights(wl, 0)
    xo, wo, _ = q8.q8_smooth_fold(dev(x), dev(w))
    s_ref = oracle.smooth_scales(bits(x))
    xo_ref = oracle.smooth_fold_x(bits(x), s_ref)
    wo_ref = oracle.smooth_fold_w(w.numpy(), s_ref)
    del w
    np.testing.assert_array_equal(bits(host(xo)), xo_ref)
    np.testing.assert_array_equal(host(wo).numpy(), wo_ref)
    xq, sx = q8.q8_quant_fp8_per_group128(xo)
    wq, sw = q8.q8_quant_weight_fp8_block128(wo)
    del wo
    xq_ref, sx_ref = oracle.quant_fp8_per_group128(xo_ref)
    wq_ref, sw_ref = oracle.quant_weight_fp8_block128(wo_ref)
    del wo_ref
    np.testing.assert_array_equal(host(sx).numpy(), sx_ref)
    np.testing.assert_array_equal(u8(xq), xq_ref)
    np.testing.assert_array_equal(host(sw).numpy(), sw_ref)
    np.testing.assert_array_equal(u8(wq), wq_ref)
    y = q8.q8_fp8_block_scaled_mm(xq, wq, sx, sw)
    rng = np.random.default_rng(9)
    rows = np.unique(np.concatenate([[0, 1, 127, 128, 255, 256, 4095, 8190, 8191, 1234],
                                     rng.integers(0, wl.M, 38)]))
    check_fp8_mm(y, xq_ref[rows], wq_ref, sx_ref[rows], sw_ref, "fp8 sampled rows",
                 rows=rows)


def test_fp8_repeat_calls_bitwise_identical():
    M, N, K = 300, 512, 1024
    x, w = synth.custom(M, K, N, seed=5, outlier_cols=3)
    xq, sx = q8.q8_quant_fp8_per_group128(dev(x))
    wq, sw = q8.q8_quant_weight_fp8_block128(dev(w))
    y1 = host(q8.q8_fp8_block_scaled_mm(xq, wq, sx, sw))
    y2 = host(q8.q8_fp8_block_scaled_mm(xq, wq, sx, sw))
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


def test_fp8_empty_and_zero_inputs():
    """M = 0 is a no-op; all-zero activations give zero scales, +0 codes and
    zero outputs (no NaN from 0/0)."""
    x0 = torch.empty((0, 256), dtype=torch.bfloat16, device=DEV)
    xq0, sx0 = q8.q8_quant_fp8_per_group128(x0)
    assert xq0.shape == (0, 256) and sx0.shape == (0, 2)
    w = synth.custom(4, 256, 128, seed=3)[1]
    wq, sw = q8.q8_quant_weight_fp8_block128(dev(w))
    y0 = q8.q8_fp8_block_scaled_mm(xq0, wq, sx0, sw)
    assert y0.shape == (0, 128)
    x = torch.zeros((5, 256), dtype=torch.bfloat16, device=DEV)
    xq, sx = q8.q8_quant_fp8_per_group128(x)
    assert (host(sx) == 0).all() and (u8(xq) == 0).all()
    y = host(q8.q8_fp8_block_scaled_mm(xq, wq, sx, sw))
    assert (y == 0).all()


# ------------------------------------------ FP8 matrix-core summation -----

def _group8_truncation_model(a_row, b_row):
    """The summation the FP8 matrix cores perform inside one 128-wide K
    block, as measured: products in groups of 8 consecutive k; each product
    truncated toward zero to the grid 2^(e - 13), e the exponent of the
    group's largest |product|; the truncated products summed exactly."""
    from fractions import Fraction
    import math
    tot = Fraction(0)
    for g0 in range(0, len(a_row), 8):
        ps = [Fraction(float(a)) * Fraction(float(b)) for a, b in zip(a_row[g0:g0 + 8], b_row[g0:g0 + 8])]
        mx = max(abs(p) for p in ps)
        if mx == 0:
            continue
        e = math.floor(math.log2(mx))
        if Fraction(2) ** e > mx:
            e -= 1
        q = Fraction(2) ** (e - 13)
        for p in ps:
            t = abs(p) // q * q
            tot += t if p >= 0 else -t
    return tot


def test_fp8_matrix_core_summation_model():
    """Constructed operands (unit scales, exact E4M3 values) through the FP8
    GEMM: in K block 0 a large product and small ones in the same group of
    8 or the next; K block 1 cancels the large product, so the bf16 output
    is exactly what the matrix cores kept of the small ones.  Each output
    must equal the truncation model above (the summation behind the
    parity bound of this path), and the cases are chosen so that exact
    summation, round-to-nearest, truncation toward minus infinity, summing
    a group before truncating, or groups of another size would each give a
    different value for at least one of them."""
    cases = [({0: 1.0, 1: 2 ** -8, 128: -1.0}, 0.0),            # 2^-14 below the grid: dropped
             ({0: 1.0, 1: 2 ** -7, 128: -1.0}, 2 ** -13),       # on the grid: kept
             ({0: 1.0, 1: 3 * 2 ** -8, 128: -1.0}, 2 ** -13),   # 1.5 grid steps: truncated, not rounded
             ({0: 1.0, 1: -(2 ** -8), 128: -1.0}, 0.0),         # negative: toward zero, not down
             ({0: 1.0, 8: 2 ** -8, 128: -1.0}, 2 ** -14),       # next group: its own grid
             ({0: 1.0, 1: 2 ** -8, 2: 2 ** -8, 128: -1.0}, 0.0),  # truncated one by one
             ({0: 2.0, 1: 2 ** -7, 128: -2.0}, 0.0),            # grid follows the group maximum
             ({0: 2.0, 1: 3 * 2 ** -7, 128: -2.0}, 2 ** -12),
             ({0: -1.0, 1: 2 ** -8, 128: 1.0}, 0.0),            # maximum by magnitude
             ({0: 1.0, 1: -3 * 2 ** -8, 128: -1.0}, -(2 ** -13)),
             ({0: 1.0, 1: 2 ** -7, 2: -(2 ** -8), 128: -1.0}, 2 ** -13),
             ({0: 1.0, **{i: 2 ** -8 for i in range(1, 8)}, 128: -1.0}, 0.0),
             ({0: 1.0, 7: 2 ** -8, 128: -1.0}, 0.0),            # k = 7 is still group 0
             ({8: 1.0, 9: 2 ** -8, 128: -(2 ** -6)}, 2 ** -14)]  # small group maximum, fine grid
    M, N, K = len(cases), 128, 256
    a = np.zeros((M, K), np.float32)
    for i, (d, _) in enumerate(cases):
        for k, v in d.items():
            a[i, k] = v
    b = np.zeros((N, K), np.float32)
    b[:, 0] = 1
    b[:, 128] = 1
    b[:, 1:16] = 2 ** -6
    at = torch.from_numpy(a).to(torch.float8_e4m3fn)
    bt = torch.from_numpy(b).to(torch.float8_e4m3fn)
    assert torch.equal(at.float(), torch.from_numpy(a)) and torch.equal(bt.float(), torch.from_numpy(b))
    sx = torch.ones((M, K // 128), dtype=torch.float32, device=DEV)
    sw = torch.ones((1, K // 128), dtype=torch.float32, device=DEV)
    y = host(q8.q8_fp8_block_scaled_mm(dev(at), dev(bt), sx, sw)).float().numpy()
    assert np.all(y == y[:, :1])  # every channel has the same weights
    exact = (a.astype(np.float64) * b[0].astype(np.float64)).sum(1)
    from fractions import Fraction
    for i, (d, want) in enumerate(cases):
        model = _group8_truncation_model(a[i, :128], b[0, :128]) + \
            _group8_truncation_model(a[i, 128:], b[0, 128:])
        assert model == Fraction(want), f"case {i}: the model gives {float(model)}"
        say(f"  case {i}: gpu {y[i, 0]!r}, model {want!r}, exact {exact[i]!r}")
        assert y[i, 0] == np.float32(want), f"case {i}: gpu {y[i, 0]} != {want}"
    assert np.sum(exact != y[:, 0]) >= 9  # the cases do exercise the truncation
