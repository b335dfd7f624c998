"""GPU parity on seeded random shapes for the group-scaled, FP8-block and
fp16 entry points (the per-channel W8A8 layer and W8A16 have theirs in
test_gpu_parity.py).  Shapes are drawn over 1-600 tokens with N and K on the
entry points' alignment (N a multiple of 16, or of 128 for FP8; K a multiple
of 128), so that every tile choice and ragged edge is reached over the set.
The bars are those of the fixed-shape tests: codes and scales bit-exact,
W8A8 outputs within 1 ulp of the oracle, FP8 and W8A16 within their stated
bounds.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
import w8a8_int8_gemm_token_amd as q8
from tests.test_gpu_f16 import _check_w8a16_f16, hbits
from tests.test_gpu_f16 import assert_ulp1 as assert_ulp1_f16
from tests.test_gpu_fp8 import check_fp8_mm, u8
from tests.test_gpu_parity import assert_ulp1, bits, dev, host, say

pytestmark = pytest.mark.gpu


def _shapes(n, seed, n_mult=16, cap=3e9):
    """n seeded (M, N, K): M from 1-16, 17-128 or 129-600 (equally likely),
    N a multiple of n_mult up to ~6000, K a multiple of 128 up to 6144, with
    M*N*K <= cap so that the oracle finishes each in about a second."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        M = int(rng.choice([rng.integers(1, 17), rng.integers(17, 129), rng.integers(129, 601)]))
        N = n_mult * int(rng.integers(1, 6000 // n_mult + 1))
        K = 128 * int(rng.integers(1, 49))
        if M * N * K <= cap:
            out.append((M, N, K))
    return out


@pytest.mark.parametrize("M,N,K", _shapes(16, 128))
def test_random_group128(M, N, K):
    """Group-128 weight scales with per-token activation scales, and with
    per-token-per-group activation scales (the quantizer included)."""
    say("random group128", M, N, K)
    x, w = synth.custom(M, K, N, seed=M * 11 + N + K, outlier_cols=max(1, K // 100))
    xq_ref, st_ref = oracle.quant_per_token(bits(x))
    wq_ref, sg_ref = oracle.quant_weight(w.numpy(), group=128)
    wq, sg = dev(torch.from_numpy(wq_ref)), dev(torch.from_numpy(sg_ref))
    y = q8.q8_scaled_mm_group128(dev(torch.from_numpy(xq_ref)), wq, dev(torch.from_numpy(st_ref)), sg)
    assert_ulp1(bits(host(y)), oracle.scaled_mm_group128(xq_ref, wq_ref, st_ref, sg_ref),
                f"group128 {M}x{N}x{K}")
    xg_ref, sx_ref = oracle.quant_per_group128(bits(x))
    xg, sx = q8.q8_quant_per_group128(dev(x))
    np.testing.assert_array_equal(host(sx).numpy(), sx_ref)
    np.testing.assert_array_equal(host(xg).numpy(), xg_ref)
    y = q8.q8_scaled_mm_group128_act(xg, wq, sx, sg)
    assert_ulp1(bits(host(y)), oracle.scaled_mm_group128_act(xg_ref, wq_ref, sx_ref, sg_ref),
                f"group128 act {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", _shapes(10, 8, n_mult=128, cap=2e8))
def test_random_fp8_block(M, N, K):
    """FP8 block-[128,128]: both quantizers bit-exact, the GEMM within the
    stated bound of the oracle's fp64 sum."""
    say("random fp8 block", M, N, K)
    x, w = synth.custom(M, K, N, seed=M * 13 + N + K, outlier_cols=max(1, K // 100))
    xq_ref, sx_ref = oracle.quant_fp8_per_group128(bits(x))
    wq_ref, sw_ref = oracle.quant_weight_fp8_block128(w.numpy())
    xq, sx = q8.q8_quant_fp8_per_group128(dev(x))
    wq, sw = q8.q8_quant_weight_fp8_block128(dev(w))
    np.testing.assert_array_equal(u8(xq), xq_ref)
    np.testing.assert_array_equal(host(sx).numpy(), sx_ref)
    np.testing.assert_array_equal(u8(wq), wq_ref)
    np.testing.assert_array_equal(host(sw).numpy(), sw_ref)
    y = q8.q8_fp8_block_scaled_mm(xq, wq, sx, sw)
    check_fp8_mm(y, xq_ref, wq_ref, sx_ref, sw_ref, f"fp8 {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", _shapes(12, 16))
def test_random_f16(M, N, K):
    """fp16 activations: the one-call W8A8 layer (codes and scales
    bit-exact, output within 1 fp16 ulp) and W8A16 (within its bound)."""
    say("random f16", M, N, K)
    x, w = synth.custom(M, K, N, seed=M * 17 + N + K, outlier_cols=max(1, K // 100))
    x = x.float().half()
    xq_ref, st_ref = oracle.quant_per_token_f16(hbits(x))
    wq_ref, sc_ref = oracle.quant_weight(w.numpy())
    wq, sc = dev(torch.from_numpy(wq_ref)), dev(torch.from_numpy(sc_ref))
    y, xq, st = q8.q8_quant_scaled_mm_f16(dev(x), wq, sc)
    np.testing.assert_array_equal(host(st).numpy(), st_ref)
    np.testing.assert_array_equal(host(xq).numpy(), xq_ref)
    assert_ulp1_f16(hbits(host(y)), oracle.scaled_mm_f16(xq_ref, wq_ref, st_ref, sc_ref),
                    f"one-call f16 {M}x{N}x{K}")
    y2 = q8.w8a16_mm_f16(dev(x), wq, sc)
    _check_w8a16_f16(hbits(host(y2)), hbits(x), wq_ref, sc_ref, f"w8a16 f16 {M}x{N}x{K}")
