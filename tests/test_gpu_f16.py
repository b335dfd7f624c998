"""GPU parity of the fp16 variant (fp16 activations in, fp16 outputs)
against the CPU oracle: codes and scales bit-exact, fp16 outputs within 1
fp16 ulp (ordered-integer distance, +0 == -0) -- the same bar as bf16,
since the same fp32 value is rounded once to the output format.  The
weight-only GEMM (fp16 products summed on the matrix cores) is held to an
error bound derived from its arithmetic instead."""
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


def hbits(t_f16_cpu) -> np.ndarray:
    return t_f16_cpu.contiguous().view(torch.int16).numpy().view(np.uint16)


def ulp_dist(a_bits, b_bits):
    def ordered(u):
        u = u.astype(np.int32)
        return np.where(u & 0x8000, -(u & 0x7FFF), u)
    return np.abs(ordered(a_bits) - ordered(b_bits))


def assert_ulp1(got_bits, ref_bits, what):
    d = ulp_dist(got_bits, ref_bits)
    say(f"{what}: max ulp {int(d.max()) if d.size else 0}, {int((d > 0).sum())}/{d.size} not bit-equal")
    assert d.size == 0 or d.max() <= 1, what


def f16_acts(name, seed, M=None, K=None):
    return synth.activations(synth.WORKLOADS[name], seed, M=M, K=K).float().half()


@pytest.mark.parametrize("M,K,pad", [(1, 1, 0), (3, 7, 0), (5, 100, 3), (17, 136, 0), (4, 512, 0),
                                     (300, 2048, 0), (300, 5120, 8), (2, 8192, 0), (3, 8200, 0)])
def test_quant_per_token_f16(M, K, pad):
    say("quant f16", M, K, pad)
    xf, _ = synth.custom(M, K + pad, 16, seed=M * 7 + K, outlier_cols=max(1, K // 100))
    xf = xf.float().half()
    x = xf[:, :K].contiguous()
    xq_ref, s_ref = oracle.quant_per_token_f16(hbits(x))
    xq, s = q8.q8_quant_per_token_f16(dev(xf)[:, :K])
    np.testing.assert_array_equal(host(s).numpy(), s_ref)
    np.testing.assert_array_equal(host(xq).numpy(), xq_ref)


def test_quant_f16_near_ties_subnormals_and_zero_rows():
    """Rows of the fp16 values where x * fl(1/s) and x / s round to
    different codes, fp16 subnormals, and an all-zero row."""
    allh = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float32)
    rng = np.random.default_rng(1)
    rows = []
    for _ in range(300):
        a = allh[rng.integers(0x3C00, 0x7B00)]
        s = np.float32(np.float64(a) / 127.0)
        xs = allh[allh <= a]
        qd = np.rint((xs.astype(np.float64) / np.float64(s)).astype(np.float32))
        qr = np.rint((xs * (np.float32(1.0) / s)).astype(np.float32))
        idx = np.nonzero(qd != qr)[0]
        if len(idx):
            rows.append(np.concatenate([[a], xs[idx], -xs[idx]]).astype(np.float32))
    assert len(rows) >= 10
    K = 512
    mat = np.zeros((len(rows) + 2, K), np.float32)
    for i, r in enumerate(rows):
        mat[i, :len(r)] = r[:K]
    mat[len(rows), :6] = np.array([6e-8, 1.2e-7, -3e-6, 5.9e-5, 0, -6e-8], np.float32)  # subnormal fp16
    x = torch.from_numpy(mat).half()
    for M in (x.shape[0], 300):  # workgroup-per-row and wave-per-row kernels
        xx = torch.cat([x] * (1 + M // x.shape[0]))[:M]
        xq_ref, s_ref = oracle.quant_per_token_f16(hbits(xx))
        xq, st = q8.q8_quant_per_token_f16(dev(xx))
        np.testing.assert_array_equal(host(st).numpy(), s_ref)
        np.testing.assert_array_equal(host(xq).numpy(), xq_ref)


@pytest.mark.parametrize("M,N,K", [(1, 16, 128), (8, 128, 1024), (16, 1040, 2048), (33, 144, 384),
                                   (64, 256, 1024), (100, 1040, 1024),  # 100: two streaming passes
                                   (130, 272, 1152), (300, 2560, 1024),
                                   (200, 9216, 256), (450, 8192, 128)])  # 64 x 128, 128 x 128 tiles
def test_scaled_mm_f16(M, N, K):
    say("scaled_mm f16", M, N, K)
    x, w = synth.custom(M, K, N, seed=M + 3 * N, outlier_cols=3)
    x = x.float().half()
    wq_ref, sc_ref = oracle.quant_weight(w.numpy())
    xq_ref, st_ref = oracle.quant_per_token_f16(hbits(x))
    y_ref = oracle.scaled_mm_f16(xq_ref, wq_ref, st_ref, sc_ref)
    y = q8.q8_scaled_mm_f16(dev(xq_ref), dev(wq_ref), dev(st_ref), dev(sc_ref))
    assert_ulp1(hbits(host(y)), y_ref, f"scaled_mm f16 {M}x{N}x{K}")


@pytest.mark.parametrize("M", [1, 2, 8, 9, 16, 33, 64, 200])
def test_quant_scaled_mm_f16_token_counts(M):
    """Every route of the one-call layer: one-kernel decode (M <= 8), the
    weight-streaming kernel, the tiled kernels."""
    say("quant_scaled_mm f16", M)
    N, K = 5120, 5120
    x = f16_acts("decode", 0, M=M, K=K)
    w = synth.weights(synth.WORKLOADS["decode"], 0, N=N, K=K)
    wq, sc = q8.q8_quant_weight(dev(w))
    y, xq, st = q8.q8_quant_scaled_mm_f16(dev(x), wq, sc)
    xq_ref, st_ref = oracle.quant_per_token_f16(hbits(x))
    wq_ref, sc_ref = oracle.quant_weight(w.numpy())
    np.testing.assert_array_equal(host(wq).numpy(), wq_ref)
    np.testing.assert_array_equal(host(sc).numpy(), sc_ref)
    np.testing.assert_array_equal(host(xq).numpy(), xq_ref)
    np.testing.assert_array_equal(host(st).numpy(), st_ref)
    y_ref = oracle.scaled_mm_f16(xq_ref, wq_ref, st_ref, sc_ref)
    assert_ulp1(hbits(host(y)), y_ref, f"one-call f16 M={M}")


@pytest.mark.parametrize("M,N,K,pad", [(5, 2048, 2304, 0), (12, 4112, 1280, 16), (16, 17408, 5120, 16),
                                     (13, 4112, 3072, 16)])
def test_quant_scaled_mm_f16_few_tokens_outside_decode(M, N, K, pad):
    """fp16 activations, up to 16 tokens outside the one-kernel decode path
    (the quantizer, then the weight-streaming kernel): strided x, w and y, a
    zero row."""
    say("few tokens outside decode f16", M, N, K, pad)
    xf, wf = synth.custom(M, K + pad, N, seed=5 * M + K, outlier_cols=K // 90)
    xf = xf.float().half()
    xf[M // 2] = 0
    x = xf[:, :K].contiguous()
    w = wf[:, :K].contiguous()
    xq_ref, st_ref = oracle.quant_per_token_f16(hbits(x))
    wq_ref, sc_ref = oracle.quant_weight(w.numpy())
    y_ref = oracle.scaled_mm_f16(xq_ref, wq_ref, st_ref, sc_ref)
    wq_full = torch.zeros((N, K + pad), dtype=torch.int8, device=DEV)
    wq_full[:, :K] = dev(torch.from_numpy(wq_ref))
    yfull = torch.full((M, N + pad), -1, dtype=torch.int16, device=DEV).view(torch.float16)
    y, xq, st = q8.q8_quant_scaled_mm_f16(dev(xf)[:, :K], wq_full[:, :K], dev(torch.from_numpy(sc_ref)),
                                          out=yfull[:, :N])
    np.testing.assert_array_equal(host(xq).numpy(), xq_ref)
    np.testing.assert_array_equal(host(st).numpy(), st_ref)
    assert_ulp1(hbits(host(y).contiguous()), y_ref, f"few tokens f16 {M}x{N}x{K}")
    if pad:
        assert (host(yfull)[:, N:].view(torch.int16) == -1).all()


@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (8, 256, 1024), (65, 272, 1152), (200, 384, 2048),
                                   (300, 5120, 256), (600, 5120, 256)])  # 64 x 128, 128 x 128 tiles
def test_group128_act_f16(M, N, K):
    say("group128 act f16", M, N, K)
    x, w = synth.custom(M, K, N, seed=M * 11 + N, outlier_cols=3)
    x = x.float().half()
    xq_ref, sx_ref = oracle.quant_per_group128_f16(hbits(x))
    wq_ref, sw_ref = oracle.quant_weight(w.numpy(), group=128)
    y_ref = oracle.scaled_mm_group128_act_f16(xq_ref, wq_ref, sx_ref, sw_ref)
    xq, sx = q8.q8_quant_per_group128_f16(dev(x))
    np.testing.assert_array_equal(host(xq).numpy(), xq_ref)
    np.testing.assert_array_equal(host(sx).numpy(), sx_ref)
    y = q8.q8_scaled_mm_group128_act_f16(xq, dev(wq_ref), sx, dev(sw_ref))
    assert_ulp1(hbits(host(y)), y_ref, f"group128 act f16 {M}x{N}x{K}")


def test_prefill_f16_full_size_sampled_rows():
    """The prefill shape (8192 x 15360 x 5120) through the fp16 one-call
    layer in one launch; codes and scales whole, outputs on sampled rows."""
    wl = synth.WORKLOADS["prefill"]
    say("prefill f16 full size")
    x = synth.activations(wl, 0).float().half()
    w = synth.weights(wl, 0)
    wq, sc = q8.q8_quant_weight(dev(w))
    y, xq, st = q8.q8_quant_scaled_mm_f16(dev(x), wq, sc)
    xq_ref, st_ref = oracle.quant_per_token_f16(hbits(x))
    wq_ref, sc_ref = oracle.quant_weight(w.numpy())
    np.testing.assert_array_equal(host(wq).numpy(), wq_ref)
    np.testing.assert_array_equal(host(sc).numpy(), sc_ref)
    np.testing.assert_array_equal(host(st).numpy(), st_ref)
    np.testing.assert_array_equal(host(xq).numpy(), xq_ref)
    rng = np.random.default_rng(8)
    rows = np.unique(np.concatenate([[0, 1, 255, 256, 4095, 8190, 8191, 777], rng.integers(0, wl.M, 56)]))
    y_ref = oracle.scaled_mm_f16(xq_ref[rows], wq_ref, st_ref[rows], sc_ref)
    assert_ulp1(hbits(host(y))[rows], y_ref, "prefill f16 sampled rows")


def test_f16_empty_and_overflow_to_infinity():
    """M = 0 is a no-op; an fp32 result beyond the fp16 range becomes
    infinity, as in the oracle."""
    x0 = torch.empty((0, 256), dtype=torch.float16, device=DEV)
    xq0, st0 = q8.q8_quant_per_token_f16(x0)
    assert xq0.shape == (0, 256) and st0.shape == (0,)
    M, N, K = 4, 128, 256
    a = synth.int8_uniform((M, K), seed=91, lo=100, hi=127)
    b = synth.int8_uniform((N, K), seed=92, lo=100, hi=127)
    s_tok = np.full((M,), 1.0, np.float32)
    s_ch = np.full((N,), 0.005, np.float32)
    s_ch[::3] = 1.0   # sums near 3.3e6: times 1.0 they overflow fp16, times 0.005 they stay finite
    y_ref = oracle.scaled_mm_f16(a, b, s_tok, s_ch)
    y = q8.q8_scaled_mm_f16(dev(a), dev(b), dev(s_tok), dev(s_ch))
    yh = hbits(host(y))
    assert (yh[:, ::3] == 0x7C00).all() and (y_ref[:, ::3] == 0x7C00).all()
    assert_ulp1(yh, y_ref, "f16 overflow")


# ------------------------------------------- weight-only INT8, fp16 x ----

def _check_w8a16_f16(y_bits, x_bits, wq, s_ch, what):
    """|y - y_ref| <= 2^-11 |y_ref| (1 + 2^-10) + 2^-25 + K 2^-22 mag: the
    fp16 output rounding (half an ulp, relative; half the subnormal quantum
    near 0) and fp32 accumulation of the exact int8 x fp16 products (at most
    one rounding of the running sum, |sum| <= mag, per product, with 4x
    slack).  mag = s_ch[n] sum_k |x[m,k] w[n,k]|."""
    K = x_bits.shape[1]
    y_ref, mag = oracle.w8a16_ref_f16(x_bits, wq, s_ch, with_mag=True)
    assert np.all(np.abs(y_ref) < 60000.0), "test data must stay in the fp16 range"
    y = y_bits.view(np.float16).astype(np.float64)
    err = np.abs(y - y_ref)
    bound = 2.0 ** -11 * np.abs(y_ref) * (1 + 2.0 ** -10) + 2.0 ** -25 + K * 2.0 ** -22 * mag
    ratio = err / bound
    say(f"{what}: max err/bound {ratio.max() if ratio.size else 0:.3f}")
    assert np.all(np.isfinite(y)), what
    assert np.all(err <= bound), what


def _w8a16_inputs(M, N, K, seed, pad=0):
    wl = synth.WORKLOADS["w8a16"]
    xf = synth.activations(wl, seed, M=M, K=K + pad).float()
    xf[0] = xf[0] * 50  # a position-outlier row, as in the W8A16 workload
    xf = xf.half()
    w = synth.weights(wl, seed, N=N, K=K)
    wq_ref, sc_ref = oracle.quant_weight(w.numpy())
    return xf, wq_ref, sc_ref


@pytest.mark.parametrize("M,N,K,pad", [
    (16, 128, 256, 0), (33, 144, 384, 8),          # few tokens, K not a multiple of 1024
    (1, 16, 1024, 0), (5, 4112, 2048, 16), (16, 5120, 5120, 0), (33, 1040, 4096, 0),
    (64, 2048, 3072, 0),                            # few tokens: weight streaming
    (65, 272, 1152, 0), (100, 1040, 2048, 8),       # 65-112 tokens: two streaming passes
    (192, 5120, 1024, 0), (300, 5120, 512, 8),      # 32 x 128 and 64 x 128 tiles
    (130, 256, 1024, 8), (300, 128, 13824, 0)])     # tiled
def test_w8a16_f16_shapes(M, N, K, pad):
    """Each route of the weight-only GEMM with fp16 activations (small-M
    tiles, the weight-streaming ring, the tiled kernel), strided x and y."""
    say("w8a16 f16", M, N, K, pad)
    xf, wq_ref, sc_ref = _w8a16_inputs(M, N, K, seed=M + N, pad=pad)
    x = xf[:, :K].contiguous()
    yfull = torch.full((M, N + pad), -1, dtype=torch.int16, device=DEV).view(torch.float16)
    y = q8.w8a16_mm_f16(dev(xf)[:, :K], dev(wq_ref), dev(sc_ref), out=yfull[:, :N])
    _check_w8a16_f16(hbits(host(y)), hbits(x), wq_ref, sc_ref, f"w8a16 f16 {M}x{N}x{K}")
    if pad:
        assert (host(yfull)[:, N:].view(torch.int16) == -1).all()


def test_w8a16_f16_full_size_sampled_rows():
    """The W8A16 workload's full shape in one launch (the 256 x 128 tiles),
    outputs checked on sampled rows."""
    wl = synth.WORKLOADS["w8a16"]
    say("w8a16 f16 full size")
    x = synth.activations(wl, 0).float().half()
    w = synth.weights(wl, 0)
    wq_ref, sc_ref = oracle.quant_weight(w.numpy())
    wq, sc = q8.q8_quant_weight(dev(w))
    y = q8.w8a16_mm_f16(dev(x), wq, sc)
    rows = np.array([0, 1, 40, 81, 82, 83, 127, 128, 4096, 8190, 8191])
    _check_w8a16_f16(hbits(host(y))[rows], np.ascontiguousarray(hbits(x)[rows]), wq_ref, sc_ref,
                     "w8a16 f16 sampled rows")


def test_w8a16_f16_big_tiles_sampled_rows():
    """The 256 x 320 tiles (4100 x 4000: 544 tiles of 256 x 128 against 221),
    ragged on both edges; sampled rows, every column."""
    M, N, K = 4100, 4000, 256
    say("w8a16 f16 big tiles", M, N, K)
    xf, wq_ref, sc_ref = _w8a16_inputs(M, N, K, seed=5)
    y = q8.w8a16_mm_f16(dev(xf), dev(wq_ref), dev(sc_ref))
    rows = np.array([0, 1, 31, 32, 255, 256, 2047, 4095, 4096, 4099])
    _check_w8a16_f16(hbits(host(y))[rows], np.ascontiguousarray(hbits(xf)[rows]), wq_ref, sc_ref,
                     "w8a16 f16 big tiles")


@pytest.mark.parametrize("M", [0, 4, 100])
def test_w8a16_f16_empty_and_overflow_to_infinity(M):
    """M = 0 is a no-op; sums beyond the fp16 range become infinity (small
    M: the streaming ring; M = 100: the tiled kernel)."""
    N, K = 128, 1024
    x = torch.full((M, K), 1024.0, dtype=torch.float16)
    wq = np.full((N, K), 127, np.int8)
    s_ch = np.full((N,), 2.0 ** -12, np.float32)
    s_ch[::3] = 1.0  # 1024 * 127 * 1024 = 127 * 2^20: times 1 it overflows, times 2^-12 it is 32512
    y = q8.w8a16_mm_f16(dev(x), dev(wq), dev(s_ch))
    assert y.shape == (M, N)
    if M == 0:
        return
    yh = hbits(host(y))
    assert (yh[:, ::3] == 0x7C00).all()
    finite = np.ones(N, bool)
    finite[::3] = False
    assert (yh[:, finite].view(np.float16).astype(np.float64) == 32512.0).all()
