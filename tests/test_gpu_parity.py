"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Integer and byte results (codes, scales, int32 sums, weight codes, folded
inputs) must be bit-exact.  bf16 outputs of the W8A8 GEMMs must be within 1
bf16 ulp of the oracle (distance on the ordered-integer map, +0 == -0).
W8A16 outputs are checked against the oracle's fp64 sum with the
floating-point error bound of any summation order (per-row relative norm
<= 2e-2 and elementwise |y - ref| <= 2e-2*|ref| + K*2^-22*mag + bf16
rounding).  Inputs are the seeded synthetic workloads (synth/); at the full
sizes the oracle computes sampled rows.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import synth
import w8a8_int8_gemm_token_amd as q8
from tests.norm_check import check_rows

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


def ulp_dist(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    def ordered(u):
        u = u.astype(np.int32)
        return np.where(u & 0x8000, -(u & 0x7FFF), u)
    return np.abs(ordered(a_bits) - ordered(b_bits))


def assert_ulp1(got_bits, ref_bits, what):
    d = ulp_dist(got_bits, ref_bits)
    n_off = int((d > 0).sum())
    say(f"{what}: max ulp {int(d.max()) if d.size else 0}, {n_off}/{d.size} not bit-equal")
    assert d.size == 0 or d.max() <= 1, what


# ---------------------------------------------------------------- quant --

@pytest.mark.parametrize("name,seed", [("tiny", 0), ("tiny", 1), ("decode", 0),
                                       ("decode", 1), ("decode", 2),
                                       ("group128", 0), ("w8a16", 0)])
def test_quant_per_token_workloads(name, seed):
    say("quant", name, seed)
    x = synth.activations(synth.WORKLOADS[name], seed)
    xq_ref, s_ref = oracle.quant_per_token(bits(x))
    xq, s = q8.q8_quant_per_token(dev(x))
    np.testing.assert_array_equal(host(s).numpy(), s_ref)
    np.testing.assert_array_equal(host(xq).numpy(), xq_ref)


@pytest.mark.parametrize("M,K,pad", [(1, 1, 0), (3, 7, 0), (5, 100, 3), (17, 136, 0),
                                     (4, 512, 0), (9, 520, 8), (6, 2048, 0), (2, 8192, 0),
                                     (3, 8200, 0), (2, 13824, 0), (1, 40000, 8)])
def test_quant_per_token_ragged(M, K, pad):
    say("quant ragged", M, K, pad)
    xfull, _ = synth.custom(M, K + pad, 16, seed=M * 1000 + K, outlier_cols=3)
    x = xfull[:, :K]
    xq_ref, s_ref = oracle.quant_per_token(bits(x.contiguous()))
    xd = dev(xfull)[:, :K]
    xq, s = q8.q8_quant_per_token(xd)
    np.testing.assert_array_equal(host(s).numpy(), s_ref)
    np.testing.assert_array_equal(host(xq).numpy(), xq_ref)


def test_quant_zero_rows_and_ties():
    rows = [
        [127, 2.5, 3.5, -2.5, 0.5, 1.5, -0.5, -1.5],
        [0] * 8,
        [63.5, 1.25, 1.75, -1.25, 0.25, 0.75, -0.75, 62.75],
        [-254, 5, 7, -5, 1, 3, -3, 253],
    ]
    x = torch.tensor(rows, dtype=torch.float32).to(torch.bfloat16)
    x = torch.cat([x] * 64, dim=1)  # K = 512 (vector path)
    xq_ref, s_ref = oracle.quant_per_token(bits(x))
    xq, s = q8.q8_quant_per_token(dev(x))
    np.testing.assert_array_equal(host(s).numpy(), s_ref)
    np.testing.assert_array_equal(host(xq).numpy(), xq_ref)
    assert s_ref[1] == 0 and not xq_ref[1].any()


def test_quant_near_ties_and_tiny_scales():
    """Rows built from the bf16 values where x * fl(1/s) and x / s round to
    different codes (the kernels' reciprocal route must detect each such
    near-tie and divide), plus rows whose scale is subnormal."""
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
            rows.append(np.concatenate([[a], xs[idx], -xs[idx]]).astype(np.float32))
    assert len(rows) >= 10
    K = 512
    mat = np.zeros((len(rows) + 3, K), np.float32)
    for i, r in enumerate(rows):
        mat[i, :len(r)] = r[:K]
    # subnormal and near-subnormal scales: absmax 1e-38, 2e-37, 1e-40
    for j, amax in enumerate([1e-38, 2e-37, 1e-40]):
        mat[len(rows) + j, :7] = np.array([1, 0.5, -0.25, 0.75, 0.3, -1, 0.01], np.float32) * amax
    x = torch.from_numpy(mat).to(torch.bfloat16)
    for M in (len(rows) + 3, 300):  # workgroup-per-row and wave-per-row kernels
        xx = torch.cat([x] * (1 + M // x.shape[0]))[:M]
        xq_ref, s_ref = oracle.quant_per_token(bits(xx))
        xq, st = q8.q8_quant_per_token(dev(xx))
        np.testing.assert_array_equal(host(st).numpy(), s_ref)
        np.testing.assert_array_equal(host(xq).numpy(), xq_ref)


def test_quant_empty():
    x = torch.empty((0, 256), dtype=torch.bfloat16, device=DEV)
    xq, s = q8.q8_quant_per_token(x)
    assert xq.shape == (0, 256) and s.shape == (0,)


# ------------------------------------ residual add + RMSNorm + quant --

def _norm_case(M, K, pad, seed, with_res):
    xf, _ = synth.custom(M, K + pad, 16, seed=seed, outlier_cols=max(1, K // 100))
    g = np.random.default_rng(seed)
    gam = torch.from_numpy((0.25 + g.random(K)).astype(np.float32)).to(torch.bfloat16)
    rf = None
    if with_res:
        rf = torch.from_numpy((g.standard_normal((M, K + pad)) * 2).astype(np.float32)).to(torch.bfloat16)
    return xf, gam, rf


@pytest.mark.parametrize("M,K,with_res,pad", [(1, 8, False, 0), (3, 64, True, 0), (5, 520, False, 8),
                                              (8, 5120, True, 0), (7, 8192, True, 16),
                                              (33, 4096, True, 0), (200, 5120, False, 0),
                                              (130, 1032, True, 24)])
def test_rmsnorm_quant_shapes(M, K, with_res, pad):
    say("rmsnorm_quant", M, K, with_res, pad)
    eps = 1e-6
    xf, gam, rf = _norm_case(M, K, pad, M * 7 + K, with_res)
    x = xf[:, :K].contiguous()
    x[M // 2] = 0
    if with_res:
        rf[M // 2, :K] = 0
    r = None if rf is None else bits(rf[:, :K].contiguous())
    xq_ref, s_ref, _, res_ref = oracle.rmsnorm_quant(bits(x), bits(gam), eps, res_bf16=r)
    xfd = dev(xf)
    xfd[:, :K] = dev(x)
    rd = None if rf is None else dev(rf)
    xq, s = q8.q8_rmsnorm_quant(xfd[:, :K], dev(gam), eps,
                                residual=None if rd is None else rd[:, :K])
    h = res_ref if with_res else bits(x)
    n_exact, n_nb, _ = check_rows(h, bits(gam), eps, host(xq).numpy(), host(s).numpy())
    say(f"  rows bit-exact at the exact sum of squares: {n_exact}/{M}, at a bounded neighbour: {n_nb}")
    assert host(s).numpy()[M // 2] == 0 and s_ref[M // 2] == 0
    if with_res:
        np.testing.assert_array_equal(bits(host(rd)[:, :K].contiguous()), res_ref)
        if pad:  # columns past K of the residual are untouched
            assert torch.equal(host(rd)[:, K:].view(torch.int16), rf[:, K:].view(torch.int16))


def test_rmsnorm_quant_in_place_residual_and_prefill_size():
    """The prefill workload's shape (8192 x 5120), with the residual stream
    updated in place in the buffer x itself."""
    wl = synth.WORKLOADS["prefill"]
    say("rmsnorm_quant prefill size, in place")
    x = synth.activations(wl, 0)
    g = np.random.default_rng(3)
    gam = torch.from_numpy((0.25 + g.random(wl.K)).astype(np.float32)).to(torch.bfloat16)
    r = torch.from_numpy(g.standard_normal((wl.M, wl.K)).astype(np.float32)).to(torch.bfloat16)
    xq_ref, s_ref, _, res_ref = oracle.rmsnorm_quant(bits(r), bits(gam), 1e-6, res_bf16=bits(x))
    buf = dev(x)
    xq, s = q8.q8_rmsnorm_quant(dev(r), dev(gam), 1e-6, residual=buf)
    np.testing.assert_array_equal(bits(host(buf)), res_ref)
    n_exact, n_nb, _ = check_rows(res_ref, bits(gam), 1e-6, host(xq).numpy(), host(s).numpy())
    say(f"  rows bit-exact at the exact sum of squares: {n_exact}/{wl.M}, at a bounded neighbour: {n_nb}")
    # x and the residual the same buffer: h = bf16(x + x) = 2x
    b2 = dev(r)
    xq2, s2 = q8.q8_rmsnorm_quant(b2, dev(gam), 1e-6, residual=b2)
    xq2_ref, s2_ref, _, res2_ref = oracle.rmsnorm_quant(bits(r), bits(gam), 1e-6, res_bf16=bits(r))
    np.testing.assert_array_equal(bits(host(b2)), res2_ref)
    check_rows(res2_ref, bits(gam), 1e-6, host(xq2).numpy(), host(s2).numpy())


# --------------------------------------------------------- weight quant --

@pytest.mark.parametrize("name", ["tiny", "decode", "group128", "w8a16"])
def test_quant_weight(name):
    wl = synth.WORKLOADS[name]
    say("weight quant", name)
    w = synth.weights(wl, 0)
    wd = dev(w)
    wq_ref, s_ref = oracle.quant_weight(w.numpy())
    wq, s = q8.q8_quant_weight(wd)
    np.testing.assert_array_equal(host(s).numpy(), s_ref)
    np.testing.assert_array_equal(host(wq).numpy(), wq_ref)
    wq_ref, s_ref = oracle.quant_weight(w.numpy(), group=128)
    wq, s = q8.q8_quant_weight(wd, group=128)
    np.testing.assert_array_equal(host(s).numpy(), s_ref)
    np.testing.assert_array_equal(host(wq).numpy(), wq_ref)


# ---------------------------------------------------------- smooth fold --

def test_smooth_fold_prefill_full():
    wl = synth.WORKLOADS["prefill"]
    say("smooth fold prefill full size")
    x = synth.activations(wl, 0)
    w = synth.weights(wl, 0)
    s_ref = oracle.smooth_scales(bits(x))
    xo_ref = oracle.smooth_fold_x(bits(x), s_ref)
    wo_ref = oracle.smooth_fold_w(w.numpy(), s_ref)
    xo, wo, s = q8.q8_smooth_fold(dev(x), dev(w))
    np.testing.assert_array_equal(host(s).numpy(), s_ref)
    np.testing.assert_array_equal(bits(host(xo)), xo_ref)
    np.testing.assert_array_equal(host(wo).numpy(), wo_ref)


def test_smooth_fold_cap_and_in_place():
    x = torch.tensor([[1024.0, 4.0, -2.25, 0.5], [3.0, -1.0, 1.0, 0.25]]).to(torch.bfloat16)
    w = torch.ones((16, 4), dtype=torch.float32)
    s_ref = oracle.smooth_scales(bits(x))
    xd, wd = dev(x), dev(w)
    _, _, s = q8.q8_smooth_fold(xd, wd, x_out=xd, w_out=wd)
    np.testing.assert_array_equal(host(s).numpy(), s_ref)
    np.testing.assert_array_equal(bits(host(xd)), oracle.smooth_fold_x(bits(x), s_ref))
    np.testing.assert_array_equal(host(wd).numpy(), oracle.smooth_fold_w(w.numpy(), s_ref))


# ------------------------------------------------------------ INT32 GEMM -

@pytest.mark.parametrize("M,N,K", [(1, 16, 128), (16, 128, 256), (31, 144, 384),
                                   (64, 256, 128), (65, 128, 256), (130, 272, 640),
                                   (257, 400, 1024), (300, 512, 512),
                                   (200, 9216, 256),    # 64 x 128 tiles (504 of 32 x 128)
                                   (450, 8192, 128)])   # 128 x 128 tiles
def test_mm_i32(M, N, K):
    say("mm_i32", M, N, K)
    a = synth.int8_uniform((M, K), seed=M + K)
    b = synth.int8_uniform((N, K), seed=N + 7 * K)
    ref = oracle.mm_i32(a, b)
    got = host(q8.q8_mm_i32(dev(a), dev(b))).numpy()
    np.testing.assert_array_equal(got, ref)


def test_mm_i32_extremes_max_k():
    K = q8.MAX_K
    say("mm_i32 max K", K)
    a = np.full((16, K), -128, np.int8)
    b = np.full((16, K), -128, np.int8)
    b[1] = 127
    b[2, ::2] = 127
    ref = oracle.mm_i32(a, b)
    got = host(q8.q8_mm_i32(dev(a), dev(b))).numpy()
    np.testing.assert_array_equal(got, ref)
    assert ref[0, 0] == 128 * 128 * K


def test_mm_i32_strided_operands():
    M, N, K = 70, 160, 256
    a = synth.int8_uniform((M, K + 64), seed=3)
    b = synth.int8_uniform((N, K + 32), seed=4)
    ref = oracle.mm_i32(np.ascontiguousarray(a[:, :K]), np.ascontiguousarray(b[:, :K]))
    outbuf = torch.zeros((M, N + 12), dtype=torch.int32, device=DEV)
    q8.q8_mm_i32(dev(a)[:, :K], dev(b)[:, :K], out=outbuf[:, :N])
    got = host(outbuf).numpy()
    np.testing.assert_array_equal(got[:, :N], ref)
    assert not got[:, N:].any(), "wrote outside the output view"


# Large problems run the per-channel and int32 GEMMs on 256 x 384 tiles when
# that needs fewer whole waves of tiles (4100 x 4000: 272 tiles of 256 x 256
# against 187 of 256 x 384; 8192 x 5120: 640 against 448), with ragged tiles
# on both edges here.  The sampled rows sit on each side of tile boundaries
# and in the partial last row of tiles; every column is checked.
BIG_ROWS = np.array([0, 1, 31, 32, 127, 128, 255, 256, 2047, 2048, 4095, 4096, 4097, 4099, 8191])


@pytest.mark.parametrize("M,N,K,pad", [(4100, 4000, 256, 0), (4100, 4000, 384, 48), (8192, 5120, 1024, 0)])
def test_big_tiles_mm_i32_sampled_rows(M, N, K, pad):
    say("big tiles mm_i32", M, N, K, pad)
    a = synth.int8_uniform((M, K + pad), seed=M + K)
    b = synth.int8_uniform((N, K + pad), seed=N + 3 * K)
    rows = BIG_ROWS[BIG_ROWS < M]
    outbuf = torch.full((M, N + pad), -7, dtype=torch.int32, device=DEV)
    q8.q8_mm_i32(dev(a)[:, :K], dev(b)[:, :K], out=outbuf[:, :N])
    got = host(outbuf).numpy()
    ref = oracle.mm_i32(np.ascontiguousarray(a[rows, :K]), np.ascontiguousarray(b[:, :K]))
    np.testing.assert_array_equal(got[rows, :N], ref)
    if pad:
        assert (got[:, N:] == -7).all(), "wrote outside the output view"


@pytest.mark.parametrize("M,N,K", [(4100, 4000, 256), (8192, 5120, 1024)])
def test_big_tiles_scaled_mm_sampled_rows(M, N, K):
    say("big tiles scaled_mm", M, N, K)
    a = synth.int8_uniform((M, K), seed=M + 5 * K, lo=-127)
    b = synth.int8_uniform((N, K), seed=N + 7 * K, lo=-127)
    st = synth.uniform_f32((M,), seed=M, lo=1e-4, hi=2e-2)
    sc = synth.uniform_f32((N,), seed=N, lo=1e-4, hi=2e-2)
    rows = BIG_ROWS[BIG_ROWS < M]
    y = q8.q8_scaled_mm(dev(a), dev(b), dev(st), dev(sc))
    ref = oracle.scaled_mm(np.ascontiguousarray(a[rows]), b, st[rows], sc)
    assert_ulp1(bits(host(y))[rows], ref, f"big tiles scaled_mm {M}x{N}x{K}")
    yh = q8.q8_scaled_mm_f16(dev(a), dev(b), dev(st), dev(sc))
    ref_h = oracle.scaled_mm_f16(np.ascontiguousarray(a[rows]), b, st[rows], sc)
    got_h = host(yh).contiguous().view(torch.int16).numpy().view(np.uint16)[rows]
    assert_ulp1(got_h, ref_h, f"big tiles scaled_mm_f16 {M}x{N}x{K}")


@pytest.mark.parametrize("f16", [False, True])
def test_big_tiles_persistent_ragged_strided_output(f16):
    """The per-channel 256 x 384 kernel runs one workgroup per CU taking the
    tiles in turn (here 33 x 41 = 1,353 tiles, ragged in both directions):
    every row on each side of a tile boundary and in the partial last row of
    tiles matches the oracle, and the stores of the ragged tiles, issued by
    every lane and dropped past C's buffer resource, leave the padding
    columns of a strided output and the rows below it untouched."""
    M, N, K, pad = 8200, 15376, 256, 24
    say("big tiles persistent ragged", M, N, K, pad, f16)
    a = synth.int8_uniform((M, K), seed=41, lo=-127)
    b = synth.int8_uniform((N, K), seed=43, lo=-127)
    st = synth.uniform_f32((M,), seed=47, lo=1e-4, hi=2e-2)
    sc = synth.uniform_f32((N,), seed=53, lo=1e-4, hi=2e-2)
    dt = torch.float16 if f16 else torch.bfloat16
    buf = torch.full((M + 2, N + pad), -1, dtype=torch.int16, device=DEV).view(dt)
    fn = q8.q8_scaled_mm_f16 if f16 else q8.q8_scaled_mm
    fn(dev(a), dev(b), dev(st), dev(sc), out=buf[:M, :N])
    rows = np.array([0, 1, 255, 256, 4095, 4096, 8191, 8192, 8198, 8199])
    got = host(buf).contiguous().view(torch.int16).numpy().view(np.uint16)
    ref = (oracle.scaled_mm_f16 if f16 else oracle.scaled_mm)(np.ascontiguousarray(a[rows]), b, st[rows], sc)
    assert_ulp1(got[rows, :N], ref, f"persistent big tiles f16={f16}")
    assert (got[:M, N:] == 0xFFFF).all(), "wrote into the padding columns"
    assert (got[M:] == 0xFFFF).all(), "wrote below the output"


# ------------------------------------------------------------ W8A8 layer -

def _layer_inputs(name, seed, M=None):
    wl = synth.WORKLOADS[name]
    x = synth.activations(wl, seed, M=M)
    w = synth.weights(wl, seed)
    return wl, x, w


@pytest.mark.parametrize("name,seed", [("tiny", 0), ("tiny", 1), ("tiny", 2),
                                       ("decode", 0), ("decode", 1), ("decode", 2)])
def test_scaled_mm_small_workloads(name, seed):
    say("scaled_mm", name, seed)
    wl, x, w = _layer_inputs(name, seed)
    xq_ref, st_ref = oracle.quant_per_token(bits(x))
    wq_ref, sc_ref = oracle.quant_weight(w.numpy())
    y_ref = oracle.scaled_mm(xq_ref, wq_ref, st_ref, sc_ref)
    wq, sc = q8.q8_quant_weight(dev(w))
    # two-step path
    xq, st = q8.q8_quant_per_token(dev(x))
    y = q8.q8_scaled_mm(xq, wq, st, sc)
    assert_ulp1(bits(host(y)), y_ref, f"{name}/{seed} two-step")
    # one-call path (fused kernel for M <= 16)
    y2, xq2, st2 = q8.q8_quant_scaled_mm(dev(x), wq, sc)
    np.testing.assert_array_equal(host(xq2).numpy(), xq_ref)
    np.testing.assert_array_equal(host(st2).numpy(), st_ref)
    assert_ulp1(bits(host(y2)), y_ref, f"{name}/{seed} fused")


@pytest.mark.parametrize("M", [1, 2, 3, 4, 8, 15, 16, 17, 33, 64, 65, 200])
def test_quant_scaled_mm_token_counts(M):
    say("quant_scaled_mm M", M)
    K, N = 5120, 1024
    x, w = synth.custom(M, K, N, seed=M, outlier_cols=52)
    xq_ref, st_ref = oracle.quant_per_token(bits(x))
    wq_ref, sc_ref = oracle.quant_weight(w.numpy())
    y_ref = oracle.scaled_mm(xq_ref, wq_ref, st_ref, sc_ref)
    wq, sc = q8.q8_quant_weight(dev(w))
    y, xq, st = q8.q8_quant_scaled_mm(dev(x), wq, sc)
    np.testing.assert_array_equal(host(xq).numpy(), xq_ref)
    np.testing.assert_array_equal(host(st).numpy(), st_ref)
    assert_ulp1(bits(host(y)), y_ref, f"M={M}")
    y3 = q8.q8_scaled_mm(xq, wq, st, sc)
    assert_ulp1(bits(host(y3)), y_ref, f"M={M} scaled_mm")


@pytest.mark.parametrize("M,N,K,pad", [
    (1, 16, 1024, 0),      # 4 channels per workgroup, 4 workgroups
    (8, 1040, 3072, 16),   # 8 per workgroup, strided operands
    (3, 4112, 2048, 0),    # 20 per workgroup, last one ragged (12 channels)
    (8, 5120, 5120, 0),    # the decode workload's shape
    (5, 8192, 2048, 32),   # 32 per workgroup: two weight rows per wave
    (7, 2048, 8192, 0),    # the largest K of the one-kernel path
    (8, 17408, 5120, 0),   # gate/up: quantizer + streaming kernel (the fused tile would
                           # stream 32 KB more per CU)
    (2, 15360, 5120, 16),  # q/k/v-like: three workgroups per CU
    (4, 13824, 5120, 0),   # 692 workgroups of 20 channels, the last wave partly filled
    (8, 5120, 8192, 0),    # tile does not fit in LDS: two-kernel path
    (9, 1024, 2048, 0),    # more tokens than the one-kernel path takes
    # K a multiple of 128 only: the last 1024-wide segment is partial
    (8, 3584, 3584, 0),    # 3.5 segments
    (1, 18944, 3584, 16),  # several workgroups per CU, strided operands
    (5, 1040, 1152, 0),    # one full segment and 128 more
    (7, 2048, 7296, 16),   # eight segments, the last of 128
    (3, 2048, 4352, 16),
])
def test_decode_one_call_shapes(M, N, K, pad):
    """The one-call layer at decode batch sizes (one kernel for M <= 8 when
    the channel tile fits in LDS, else quantizer + weight-streaming GEMM):
    codes, scales and outputs against the oracle, with zero and near-tie
    rows and strided x, w and y."""
    say("decode one-call", M, N, K, pad)
    xf, wf = synth.custom(M, K + pad, N, seed=N + K + M, outlier_cols=K // 100)
    x = xf[:, :K].contiguous()
    x[M // 2] = 0
    if M > 2:  # a row whose codes come from the division fallback
        x[M - 1, :4] = torch.tensor([1.0, 0.5, -0.5, 0.75])  # 0.5/fl(1/127) ~ 63.5
        x[M - 1, 4:] = 0
    xf[:, :K] = x
    w = wf[:, :K].contiguous()
    xq_ref, st_ref = oracle.quant_per_token(bits(x))
    wq_ref, sc_ref = oracle.quant_weight(w.numpy())
    y_ref = oracle.scaled_mm(xq_ref, wq_ref, st_ref, sc_ref)
    wq_full = torch.zeros((N, K + pad), dtype=torch.int8, device=DEV)
    wq_full[:, :K] = dev(torch.from_numpy(wq_ref))
    wq = wq_full[:, :K]
    sc = dev(torch.from_numpy(sc_ref))
    yfull = torch.full((M, N + pad), -1, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    y = yfull[:, :N]
    xd = dev(xf)[:, :K]
    y, xq, st = q8.q8_quant_scaled_mm(xd, wq, sc, out=y)
    np.testing.assert_array_equal(host(st).numpy(), st_ref)
    np.testing.assert_array_equal(host(xq).numpy(), xq_ref)
    assert_ulp1(bits(host(y)), y_ref, f"decode M={M} N={N} K={K}")
    if pad:  # the padding columns of y are untouched
        assert (host(yfull)[:, N:].view(torch.int16) == -1).all()


@pytest.mark.parametrize("M,N,K,pad", [
    (1, 16, 128, 0),        # one partial segment, one K block per active wave
    (8, 1040, 1152, 16),    # 1024 + 128, strided operands
    (17, 4112, 4480, 0),    # two token groups, last workgroup ragged
    (33, 2048, 13824, 16),  # four token groups, 13.5 segments
    (64, 5120, 2176, 0),
])
def test_scaled_mm_few_tokens_partial_segment(M, N, K, pad):
    """Few tokens with K a multiple of 128 but not of 1024: the
    weight-streaming kernel's last K segment is partial (loads past K read
    nothing, its K blocks past K are skipped). q8_scaled_mm and the one-call
    layer against the oracle, strided x, w and y."""
    say("scaled_mm partial segment", M, N, K, pad)
    xf, wf = synth.custom(M, K + pad, N, seed=3 * M + K, outlier_cols=K // 64)
    x = xf[:, :K].contiguous()
    w = wf[:, :K].contiguous()
    xq_ref, st_ref = oracle.quant_per_token(bits(x))
    wq_ref, sc_ref = oracle.quant_weight(w.numpy())
    y_ref = oracle.scaled_mm(xq_ref, wq_ref, st_ref, sc_ref)
    wq_full = torch.zeros((N, K + pad), dtype=torch.int8, device=DEV)
    wq_full[:, :K] = dev(torch.from_numpy(wq_ref))
    wq = wq_full[:, :K]
    sc = dev(torch.from_numpy(sc_ref))
    xq_full = torch.zeros((M, K + pad), dtype=torch.int8, device=DEV)
    xq_full[:, :K] = dev(torch.from_numpy(xq_ref))
    yfull = torch.full((M, N + pad), -1, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    y = q8.q8_scaled_mm(xq_full[:, :K], wq, dev(torch.from_numpy(st_ref)), sc, out=yfull[:, :N])
    assert_ulp1(bits(host(y).contiguous()), y_ref, f"scaled_mm {M}x{N}x{K}")
    if pad:
        assert (host(yfull)[:, N:].view(torch.int16) == -1).all()
    y2, xq2, st2 = q8.q8_quant_scaled_mm(dev(xf)[:, :K], wq, sc)
    np.testing.assert_array_equal(host(xq2).numpy(), xq_ref)
    np.testing.assert_array_equal(host(st2).numpy(), st_ref)
    assert_ulp1(bits(host(y2)), y_ref, f"quant_scaled_mm {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K,pad", [
    (16, 128, 256, 0),      # the tiny workload's shape: two workgroups
    (1, 16, 128, 0),        # one wave's channels, one K block pair
    (5, 1040, 640, 16),     # last workgroup ragged (16 of 64 channels), strided operands
    (8, 2048, 896, 16),     # the largest K below 1024 (code rows of 56 units)
    (9, 64, 384, 0),        # 24 units per code row
    (12, 4096, 512, 0),
    (7, 208, 896, 32),
    (13, 512, 128, 16),     # 16 tokens' tile, 8 units per code row
])
def test_small_layer_kernel(M, N, K, pad):
    """Few tokens with K < 1024 and a small weight matrix: the one-call
    layer in one kernel (weight fragments straight to registers, the rows
    quantized into an LDS code tile, 16 x 16 MFMA tiles). Codes,
    scales and outputs against the oracle, with a zero row, a near-tie row,
    strided x, w and y (padding untouched), and the fp16 variant."""
    say("small layer kernel", M, N, K, pad)
    xf, wf = synth.custom(M, K + pad, N, seed=19 * M + N + K, outlier_cols=max(1, K // 64))
    x = xf[:, :K].contiguous()
    x[M // 2] = 0
    if M > 2:  # a row whose codes come from the division fallback
        x[M - 1, :4] = torch.tensor([1.0, 0.5, -0.5, 0.75])
        x[M - 1, 4:] = 0
    xf[:, :K] = x
    w = wf[:, :K].contiguous()
    xq_ref, st_ref = oracle.quant_per_token(bits(x))
    wq_ref, sc_ref = oracle.quant_weight(w.numpy())
    y_ref = oracle.scaled_mm(xq_ref, wq_ref, st_ref, sc_ref)
    wq_full = torch.zeros((N, K + pad), dtype=torch.int8, device=DEV)
    wq_full[:, :K] = dev(torch.from_numpy(wq_ref))
    wq = wq_full[:, :K]
    sc = dev(torch.from_numpy(sc_ref))
    yfull = torch.full((M, N + pad), -1, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    y, xq, st = q8.q8_quant_scaled_mm(dev(xf)[:, :K], wq, sc, out=yfull[:, :N])
    np.testing.assert_array_equal(host(st).numpy(), st_ref)
    np.testing.assert_array_equal(host(xq).numpy(), xq_ref)
    assert_ulp1(bits(host(y).contiguous()), y_ref, f"small layer {M}x{N}x{K}")
    if pad:
        assert (host(yfull)[:, N:].view(torch.int16) == -1).all()
    xh = x.float().half()
    xqh_ref, sth_ref = oracle.quant_per_token_f16(host(xh).view(torch.int16).numpy().view(np.uint16))
    yh, xqh, sth = q8.q8_quant_scaled_mm_f16(dev(xh), wq, sc)
    np.testing.assert_array_equal(host(sth).numpy(), sth_ref)
    np.testing.assert_array_equal(host(xqh).numpy(), xqh_ref)
    assert_ulp1(host(yh).view(torch.int16).numpy().view(np.uint16),
                oracle.scaled_mm_f16(xqh_ref, wq_ref, sth_ref, sc_ref), f"small layer f16 {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K,pad", [
    (1, 16, 1024, 0),       # one workgroup of 4 channels, one segment
    (16, 16, 8192, 16),     # 16 tokens, eight segments, strided operands
    (9, 1040, 2048, 16),    # 8 channels per workgroup, the last one ragged
    (5, 2064, 3072, 0),     # 12 channels per workgroup, the last one of 4
    (16, 4096, 4096, 16),   # 16 channels per workgroup, 256 workgroups
    (12, 3008, 8192, 0),
    (3, 4096, 1024, 0),
])
def test_codes_decode_kernel(M, N, K, pad):
    """Up to 16 tokens of int8 codes with K a multiple of 1024 and N <= 4096:
    the decode kernel's whole-tile weight stream on the codes, B fragments
    loaded from global memory (q8_scaled_mm; the one-call layer from 9
    tokens, behind the row quantizer). Against the oracle, strided codes,
    weights and output, padding left untouched; fp16 output as well."""
    say("codes decode kernel", M, N, K, pad)
    xf, wf = synth.custom(M, K + pad, N, seed=17 * M + N + K, outlier_cols=K // 64)
    x = xf[:, :K].contiguous()
    x[M // 2] = 0  # a zero row: scale 0, codes 0
    xf[:, :K] = x
    w = wf[:, :K].contiguous()
    xq_ref, st_ref = oracle.quant_per_token(bits(x))
    wq_ref, sc_ref = oracle.quant_weight(w.numpy())
    y_ref = oracle.scaled_mm(xq_ref, wq_ref, st_ref, sc_ref)
    wq_full = torch.zeros((N, K + pad), dtype=torch.int8, device=DEV)
    wq_full[:, :K] = dev(torch.from_numpy(wq_ref))
    wq = wq_full[:, :K]
    sc = dev(torch.from_numpy(sc_ref))
    st = dev(torch.from_numpy(st_ref))
    xq_full = torch.full((M, K + pad), 77, dtype=torch.int8, device=DEV)
    xq_full[:, :K] = dev(torch.from_numpy(xq_ref))
    yfull = torch.full((M, N + pad), -1, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    y = q8.q8_scaled_mm(xq_full[:, :K], wq, st, sc, out=yfull[:, :N])
    assert_ulp1(bits(host(y).contiguous()), y_ref, f"codes decode {M}x{N}x{K}")
    if pad:
        assert (host(yfull)[:, N:].view(torch.int16) == -1).all()
    assert q8.q8_wait_timeouts(reset=True) == 0
    y2, xq2, st2 = q8.q8_quant_scaled_mm(dev(xf)[:, :K], wq, sc)
    np.testing.assert_array_equal(host(xq2).numpy(), xq_ref)
    np.testing.assert_array_equal(host(st2).numpy(), st_ref)
    np.testing.assert_array_equal(bits(host(y2)), bits(host(y).contiguous()))
    yh = q8.q8_scaled_mm_f16(xq_full[:, :K], wq, st, sc)
    yh_ref = oracle.scaled_mm_f16(xq_ref, wq_ref, st_ref, sc_ref)
    assert_ulp1(host(yh).view(torch.int16).numpy().view(np.uint16), yh_ref, f"codes decode f16 {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K,pad", [
    (65, 1040, 1024, 16),   # 64 + 1 tokens
    (100, 5120, 1152, 0),   # the second pass has 36 tokens and a partial K segment
    (128, 2048, 4096, 16),
])
def test_scaled_mm_two_streaming_passes(M, N, K, pad):
    """65-128 tokens with under 64 channel tiles run the weight-streaming
    kernel twice (tokens 0-63, then the rest). q8_scaled_mm and the one-call
    layer against the oracle, with a zero row in each pass and strided x, w
    and y."""
    say("scaled_mm two passes", M, N, K, pad)
    xf, wf = synth.custom(M, K + pad, N, seed=7 * M + N, outlier_cols=K // 64)
    x = xf[:, :K].contiguous()
    x[3] = 0
    x[M - 2] = 0
    xf[:, :K] = x
    w = wf[:, :K].contiguous()
    xq_ref, st_ref = oracle.quant_per_token(bits(x))
    wq_ref, sc_ref = oracle.quant_weight(w.numpy())
    y_ref = oracle.scaled_mm(xq_ref, wq_ref, st_ref, sc_ref)
    wq_full = torch.zeros((N, K + pad), dtype=torch.int8, device=DEV)
    wq_full[:, :K] = dev(torch.from_numpy(wq_ref))
    wq = wq_full[:, :K]
    sc = dev(torch.from_numpy(sc_ref))
    xq_full = torch.zeros((M, K + pad), dtype=torch.int8, device=DEV)
    xq_full[:, :K] = dev(torch.from_numpy(xq_ref))
    yfull = torch.full((M, N + pad), -1, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    y = q8.q8_scaled_mm(xq_full[:, :K], wq, dev(torch.from_numpy(st_ref)), sc, out=yfull[:, :N])
    assert_ulp1(bits(host(y).contiguous()), y_ref, f"scaled_mm {M}x{N}x{K}")
    if pad:
        assert (host(yfull)[:, N:].view(torch.int16) == -1).all()
    y2, xq2, st2 = q8.q8_quant_scaled_mm(dev(xf)[:, :K], wq, sc)
    np.testing.assert_array_equal(host(xq2).numpy(), xq_ref)
    np.testing.assert_array_equal(host(st2).numpy(), st_ref)
    assert_ulp1(bits(host(y2)), y_ref, f"quant_scaled_mm {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K,pad", [
    (16, 16, 256, 0),       # one partial segment, one workgroup
    (3, 2048, 4352, 16),    # few tokens where the one-kernel decode path does not fit (K % 1024)
    (12, 4112, 1280, 16),   # partial last segment, ragged last workgroup, strided operands
    (9, 5120, 5120, 0),     # o_proj-like
    (16, 15360, 5120, 16),  # q/k/v-like, strided
    (16, 17408, 5120, 0),   # gate/up-like
])
def test_quant_scaled_mm_few_tokens_outside_decode(M, N, K, pad):
    """Up to 16 tokens outside the one-kernel decode path (more than 8
    tokens, or K not a multiple of 1024): the quantizer, then the
    weight-streaming kernel. Codes and scales bit-exact, outputs within 1
    ulp of the oracle, with a zero row, a row whose codes take the division
    fallback, strided x, w and y."""
    say("few tokens outside decode", M, N, K, pad)
    xf, wf = synth.custom(M, K + pad, N, seed=11 * M + N + K, outlier_cols=K // 80)
    x = xf[:, :K].contiguous()
    x[M // 2] = 0
    if M > 2:
        x[M - 1, :4] = torch.tensor([1.0, 0.5, -0.5, 0.75])
        x[M - 1, 4:] = 0
    xf[:, :K] = x
    w = wf[:, :K].contiguous()
    xq_ref, st_ref = oracle.quant_per_token(bits(x))
    wq_ref, sc_ref = oracle.quant_weight(w.numpy())
    y_ref = oracle.scaled_mm(xq_ref, wq_ref, st_ref, sc_ref)
    wq_full = torch.zeros((N, K + pad), dtype=torch.int8, device=DEV)
    wq_full[:, :K] = dev(torch.from_numpy(wq_ref))
    sc = dev(torch.from_numpy(sc_ref))
    yfull = torch.full((M, N + pad), -1, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    y, xq, st = q8.q8_quant_scaled_mm(dev(xf)[:, :K], wq_full[:, :K], sc, out=yfull[:, :N])
    np.testing.assert_array_equal(host(st).numpy(), st_ref)
    np.testing.assert_array_equal(host(xq).numpy(), xq_ref)
    assert_ulp1(bits(host(y).contiguous()), y_ref, f"few tokens {M}x{N}x{K}")
    if pad:
        assert (host(yfull)[:, N:].view(torch.int16) == -1).all()


@pytest.mark.parametrize("M,N,K,pad", [
    (9, 16, 1024, 0),       # one K segment, one small channel tile
    (16, 1040, 2048, 16),   # last channel tile ragged, strided operands
    (13, 4112, 3072, 0),    # three segments
    (10, 8192, 4096, 32),   # four segments, strided
    (16, 5120, 5120, 0),    # o_proj-like, five segments
    (11, 15360, 5120, 16),  # q/k/v-like: three workgroups per CU, strided
])
def test_quant_scaled_mm_9_16_tokens(M, N, K, pad):
    """9-16 tokens, K a multiple of 1024 (the quantizer, then the
    weight-streaming kernel with one or two 16-token groups), over one to
    five K segments, small and ragged channel tiles and several workgroups
    per CU. Codes and scales bit-exact, outputs within 1 ulp of the oracle,
    with a zero row, a row whose codes take the division fallback, strided
    x, w and y; the padding columns of y untouched."""
    say("9-16 tokens", M, N, K, pad)
    xf, wf = synth.custom(M, K + pad, N, seed=13 * M + N + K, outlier_cols=K // 70)
    x = xf[:, :K].contiguous()
    x[M // 3] = 0
    x[M - 1, :4] = torch.tensor([1.0, 0.5, -0.5, 0.75])  # 0.5/fl(1/127) ~ 63.5
    x[M - 1, 4:] = 0
    xf[:, :K] = x
    w = wf[:, :K].contiguous()
    xq_ref, st_ref = oracle.quant_per_token(bits(x))
    wq_ref, sc_ref = oracle.quant_weight(w.numpy())
    y_ref = oracle.scaled_mm(xq_ref, wq_ref, st_ref, sc_ref)
    wq_full = torch.zeros((N, K + pad), dtype=torch.int8, device=DEV)
    wq_full[:, :K] = dev(torch.from_numpy(wq_ref))
    sc = dev(torch.from_numpy(sc_ref))
    yfull = torch.full((M, N + pad), -1, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    y, xq, st = q8.q8_quant_scaled_mm(dev(xf)[:, :K], wq_full[:, :K], sc, out=yfull[:, :N])
    np.testing.assert_array_equal(host(st).numpy(), st_ref)
    np.testing.assert_array_equal(host(xq).numpy(), xq_ref)
    assert_ulp1(bits(host(y).contiguous()), y_ref, f"9-16 tokens {M}x{N}x{K}")
    if pad:
        assert (host(yfull)[:, N:].view(torch.int16) == -1).all()


@pytest.mark.parametrize("M,N,K", [(97, 9216, 384), (200, 9216, 256), (450, 8192, 128),
                                   # over 512 tiles of 128 x 128: one round of 256 x 256
                                   (520, 16384, 256), (601, 16400, 384)])
def test_scaled_mm_mid_token_tiles(M, N, K):
    """65-1024 tokens where 256 x 256 tiles are too few to fill the chip:
    32 x 128, 64 x 128 and 128 x 128 tiles by workgroup count, and 256 x 256
    tiles where 128 x 128 would need a second round (ragged M and N), every
    output against the oracle."""
    say("scaled_mm mid tiles", M, N, K)
    x, w = synth.custom(M, K, N, seed=M + N + K, outlier_cols=4)
    xq_ref, st_ref = oracle.quant_per_token(bits(x))
    wq_ref, sc_ref = oracle.quant_weight(w.numpy())
    y_ref = oracle.scaled_mm(xq_ref, wq_ref, st_ref, sc_ref)
    y = q8.q8_scaled_mm(dev(torch.from_numpy(xq_ref)), dev(torch.from_numpy(wq_ref)),
                        dev(torch.from_numpy(st_ref)), dev(torch.from_numpy(sc_ref)))
    assert_ulp1(bits(host(y)), y_ref, f"mid tiles {M}x{N}x{K}")


def test_scaled_mm_ragged_and_zero_rows():
    M, N, K = 131, 208, 384
    x, w = synth.custom(M, K, N, seed=5, outlier_cols=4)
    x[7] = 0
    x[130] = 0
    xq_ref, st_ref = oracle.quant_per_token(bits(x))
    wq_ref, sc_ref = oracle.quant_weight(w.numpy())
    y_ref = oracle.scaled_mm(xq_ref, wq_ref, st_ref, sc_ref)
    wq, sc = q8.q8_quant_weight(dev(w))
    y, xq, st = q8.q8_quant_scaled_mm(dev(x), wq, sc)
    yb = bits(host(y))
    assert_ulp1(yb, y_ref, "ragged")
    assert not (yb[7] & 0x7FFF).any() and not (yb[130] & 0x7FFF).any()


def test_prefill_full_size_every_row():
    """The prefill workload at full size, in the benchmark's launch
    configuration (fold, weight quant, then the one-call layer): codes and
    scales bit-exact, and every one of the 8192 x 15360 outputs within 1 ulp
    of the oracle."""
    wl = synth.WORKLOADS["prefill"]
    say("prefill full size, every row")
    x = synth.activations(wl, 0)
    w = synth.weights(wl, 0)
    s_ref = oracle.smooth_scales(bits(x))
    xo_ref = oracle.smooth_fold_x(bits(x), s_ref)
    wo_ref = oracle.smooth_fold_w(w.numpy(), s_ref)
    wq_ref, sc_ref = oracle.quant_weight(wo_ref)
    xq_ref, st_ref = oracle.quant_per_token(xo_ref)
    xo, wo, s = q8.q8_smooth_fold(dev(x), dev(w))
    del w
    wq, sc = q8.q8_quant_weight(wo)
    y, xq, st = q8.q8_quant_scaled_mm(xo, wq, sc)
    np.testing.assert_array_equal(host(st).numpy(), st_ref)
    np.testing.assert_array_equal(host(xq).numpy(), xq_ref)
    np.testing.assert_array_equal(host(sc).numpy(), sc_ref)
    np.testing.assert_array_equal(host(wq).numpy(), wq_ref)
    yh = bits(host(y))
    del y
    y_ref = oracle.scaled_mm(xq_ref, wq_ref, st_ref, sc_ref)
    assert_ulp1(yh, y_ref, "prefill every row")


def test_mm_i32_prefill_shape_sampled_rows():
    """The raw INT32 product at exactly the prefill shape 8192 x 15360 x 5120
    (the 256 x 384 tiles), on the workload's own codes: sampled rows (tile
    edges of both tilings and random) bit-exact against the oracle."""
    wl = synth.WORKLOADS["prefill"]
    say("mm_i32 8192 x 15360 x 5120")
    x = synth.activations(wl, 0)
    w = synth.weights(wl, 0)
    s_ref = oracle.smooth_scales(bits(x))
    xq_ref, _ = oracle.quant_per_token(oracle.smooth_fold_x(bits(x), s_ref))
    wq_ref, _ = oracle.quant_weight(oracle.smooth_fold_w(w.numpy(), s_ref))
    del w
    c = q8.q8_mm_i32(dev(torch.from_numpy(xq_ref)), dev(torch.from_numpy(wq_ref)))
    rng = np.random.default_rng(4)
    rows = np.unique(np.concatenate([[0, 1, 31, 32, 255, 256, 383, 384, 4095, 4096, 8190, 8191],
                                     rng.integers(0, wl.M, 52)]))
    ch = host(c)[torch.from_numpy(rows)].numpy()
    del c
    ref = oracle.mm_i32(xq_ref[rows], wq_ref)
    np.testing.assert_array_equal(ch, ref)


def test_group128_int32_partials_on_k_slices():
    """The group-128 epilogue folds the exact int32 sum of each 128-wide K
    block.  Those block sums are checked on their own: q8_mm_i32 on the
    128-wide K slice of each chosen block (pointer offsets into the full
    operands, leading dimension K), at the group-scaled workload's shape
    4096 x 5120 x 5120, every row, bit-exact against the oracle."""
    wl = synth.WORKLOADS["group128"]
    say("group-128 int32 partials on K slices")
    x = synth.activations(wl, 0)
    w = synth.weights(wl, 0)
    xq_ref, _ = oracle.quant_per_token(bits(x))
    wq_ref, _ = oracle.quant_weight(w.numpy(), group=128)
    xd, wd = dev(torch.from_numpy(xq_ref)), dev(torch.from_numpy(wq_ref))
    G = wl.K // 128
    for g in (0, 1, 17, G - 2, G - 1):
        sl = slice(128 * g, 128 * g + 128)
        c = q8.q8_mm_i32(xd[:, sl], wd[:, sl])
        ref = oracle.mm_i32(np.ascontiguousarray(xq_ref[:, sl]), np.ascontiguousarray(wq_ref[:, sl]))
        np.testing.assert_array_equal(host(c).numpy(), ref)
        assert np.abs(ref).max() < 2 ** 24  # (float)p_g is exact in the fold


def _at_allocation_end(t: torch.Tensor) -> torch.Tensor:
    """A copy of t on the GPU placed at the very end of an allocation whose
    size is a whole number of 2 MiB (the caching allocator's segment
    granule), so that no byte past its last element belongs to it."""
    nb = t.numel() * t.element_size()
    total = -(-(nb + (1 << 20)) // (2 << 20)) * (2 << 20)
    buf = torch.empty(total, dtype=torch.uint8, device=DEV)
    v = buf[total - nb:].view(t.dtype).view(t.shape)
    v.copy_(t.to(DEV))
    return v


@pytest.mark.parametrize("M,N,K", [(4100, 4000, 512),    # 256 x 384; group 128 x 128; W8A16 256 x 320
                                   (4000, 4000, 384),    # 256 x 256; W8A16 on the 256 x 128 tiles
                                   (1100, 4112, 384),    # 128 x 128 tiles
                                   (300, 1040, 256)])    # 32 x 128 tiles
def test_operands_ending_at_allocation_end(M, N, K):
    """Operands whose last byte is the last byte of their allocation, with
    ragged tiles in M and N: the tiled kernels read only the caller's bytes
    (tile rows past the edge, and the stage after K that the last stage
    prefetches, read as zero instead of from past the allocation).  The
    int32 product, the per-channel and group-scaled epilogues and W8A16,
    every row against the oracle."""
    say("operands at allocation end", M, N, K)
    x, w = synth.custom(M, K, N, seed=M + 3 * N, outlier_cols=3)
    xq_ref, st_ref = oracle.quant_per_token(bits(x))
    wq_ref, sc_ref = oracle.quant_weight(w.numpy())
    xa = _at_allocation_end(torch.from_numpy(xq_ref))
    wa = _at_allocation_end(torch.from_numpy(wq_ref))
    c = q8.q8_mm_i32(xa, wa)
    np.testing.assert_array_equal(host(c).numpy(), oracle.mm_i32(xq_ref, wq_ref))
    y = q8.q8_scaled_mm(xa, wa, dev(st_ref), dev(sc_ref))
    assert_ulp1(bits(host(y)), oracle.scaled_mm(xq_ref, wq_ref, st_ref, sc_ref), "at allocation end")
    wg_ref, sg_ref = oracle.quant_weight(w.numpy(), group=128)
    wga = _at_allocation_end(torch.from_numpy(wg_ref))
    y = q8.q8_scaled_mm_group128(xa, wga, dev(st_ref), dev(sg_ref))
    assert_ulp1(bits(host(y)), oracle.scaled_mm_group128(xq_ref, wg_ref, st_ref, sg_ref),
                "group128 at allocation end")
    xb = _at_allocation_end(x)
    y = q8.w8a16_mm(xb, wa, dev(sc_ref))
    rows = np.unique(np.concatenate([np.arange(max(0, M - 40), M), [0, 1, 255, 256]]))
    _check_w8a16(bits(host(y))[rows], np.ascontiguousarray(bits(x)[rows]), wq_ref, sc_ref,
                 "w8a16 at allocation end")


# ----------------------------- per-group activations, group-128 weights --

@pytest.mark.parametrize("M,K,pad", [(1, 128, 0), (3, 640, 8), (8, 5120, 0), (130, 1024, 16),
                                     (33, 4096, 0)])
def test_quant_per_group128(M, K, pad):
    say("quant per group128", M, K, pad)
    xf, _ = synth.custom(M, K + pad, 16, seed=M + K, outlier_cols=max(1, K // 100))
    x = xf[:, :K].contiguous()
    x[M // 2, :128] = 0  # an all-zero block
    xf[:, :K] = x
    xq_ref, s_ref = oracle.quant_per_group128(bits(x))
    xq, s = q8.q8_quant_per_group128(dev(xf)[:, :K])
    np.testing.assert_array_equal(host(s).numpy(), s_ref)
    np.testing.assert_array_equal(host(xq).numpy(), xq_ref)


@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (8, 256, 1024), (64, 144, 640),
                                   (65, 272, 1152), (200, 384, 2048), (257, 128, 256),
                                   # tiles by workgroup count: 64 x 128, then 128 x 128
                                   (300, 5120, 256), (600, 5120, 256), (1100, 5120, 128)])
def test_scaled_mm_group128_act_shapes(M, N, K):
    say("group128 act", M, N, K)
    x, w = synth.custom(M, K, N, seed=M * 3 + N, outlier_cols=3)
    xq_ref, sx_ref = oracle.quant_per_group128(bits(x))
    wq_ref, sw_ref = oracle.quant_weight(w.numpy(), group=128)
    y_ref = oracle.scaled_mm_group128_act(xq_ref, wq_ref, sx_ref, sw_ref)
    xq, sx = q8.q8_quant_per_group128(dev(x))
    wq, sw = q8.q8_quant_weight(dev(w), group=128)
    y = q8.q8_scaled_mm_group128_act(xq, wq, sx, sw)
    assert_ulp1(bits(host(y)), y_ref, f"group128 act {M}x{N}x{K}")


def test_group128_act_full_size_every_row():
    """The group-128 workload's shape (4096 x 5120 x 5120) with per-group
    activation scales, in one launch; every row against the oracle."""
    wl = synth.WORKLOADS["group128"]
    say("group128 act full size")
    x = synth.activations(wl, 0)
    w = synth.weights(wl, 0)
    xq_ref, sx_ref = oracle.quant_per_group128(bits(x))
    wq_ref, sw_ref = oracle.quant_weight(w.numpy(), group=128)
    xq, sx = q8.q8_quant_per_group128(dev(x))
    wq, sw = q8.q8_quant_weight(dev(w), group=128)
    np.testing.assert_array_equal(host(xq).numpy(), xq_ref)
    np.testing.assert_array_equal(host(sx).numpy(), sx_ref)
    np.testing.assert_array_equal(host(sw).numpy(), sw_ref)
    np.testing.assert_array_equal(host(wq).numpy(), wq_ref)
    y = q8.q8_scaled_mm_group128_act(xq, wq, sx, sw)
    y_ref = oracle.scaled_mm_group128_act(xq_ref, wq_ref, sx_ref, sw_ref)
    assert_ulp1(bits(host(y)), y_ref, "group128 act every row")


# ------------------------------------------------------------ group 128 --

@pytest.mark.parametrize("M,N,K", [(16, 128, 256), (33, 144, 384), (130, 256, 1024),
                                   (257, 128, 128),
                                   # tiles by workgroup count: 32, 64 and 128 tokens
                                   (100, 1040, 512), (300, 5120, 256), (600, 5120, 256),
                                   (1100, 5120, 128)])
def test_group128_shapes(M, N, K):
    say("group128", M, N, K)
    x, w = synth.custom(M, K, N, seed=M + N, outlier_cols=3)
    xq_ref, st_ref = oracle.quant_per_token(bits(x))
    wq_ref, sg_ref = oracle.quant_weight(w.numpy(), group=128)
    y_ref = oracle.scaled_mm_group128(xq_ref, wq_ref, st_ref, sg_ref)
    xq, st = q8.q8_quant_per_token(dev(x))
    wq, sg = q8.q8_quant_weight(dev(w), group=128)
    y = q8.q8_scaled_mm_group128(xq, wq, st, sg)
    assert_ulp1(bits(host(y)), y_ref, f"group128 {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K,pad", [
    (1, 16, 128, 0),         # one block, one workgroup of 4 channels
    (8, 5120, 5120, 16),     # the decode shape, strided operands
    (16, 1040, 1152, 0),     # a partial last K segment (9 blocks), ragged workgroups
    (17, 4112, 3072, 16),    # two token groups
    (33, 272, 896, 0),       # four token groups, one partial segment
    (64, 5120, 17408, 0),    # the down projection's K: 136 blocks, 17 segments
    (5, 17408, 5120, 0),     # several workgroups per CU
])
def test_group128_few_tokens_streaming(M, N, K, pad):
    """Up to 64 tokens: both group-scaled GEMMs stream the weights once,
    each multiplying wave folding its tile's 128-wide block sums in
    ascending order. Against the oracle with strided codes, weights and
    output (padding untouched), a zero row, and the fp16 per-group form."""
    say("group128 streaming", M, N, K, pad)
    x, w = synth.custom(M, K, N, seed=23 * M + N + K, outlier_cols=max(1, K // 100))
    x[M // 2] = 0
    xq_ref, st_ref = oracle.quant_per_token(bits(x))
    wq_ref, sg_ref = oracle.quant_weight(w.numpy(), group=128)
    xg_ref, sx_ref = oracle.quant_per_group128(bits(x))

    def strided(a, rows, cols):
        full = torch.full((rows, cols + pad), 99, dtype=torch.int8, device=DEV)
        full[:, :cols] = dev(torch.from_numpy(a))
        return full[:, :cols]
    wq, sg = strided(wq_ref, N, K), dev(torch.from_numpy(sg_ref))
    yfull = torch.full((M, N + pad), -1, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    y = q8.q8_scaled_mm_group128(strided(xq_ref, M, K), wq, dev(torch.from_numpy(st_ref)), sg, out=yfull[:, :N])
    assert_ulp1(bits(host(y).contiguous()), oracle.scaled_mm_group128(xq_ref, wq_ref, st_ref, sg_ref),
                f"group128 streaming {M}x{N}x{K}")
    if pad:
        assert (host(yfull)[:, N:].view(torch.int16) == -1).all()
    y = q8.q8_scaled_mm_group128_act(strided(xg_ref, M, K), wq, dev(torch.from_numpy(sx_ref)), sg)
    assert_ulp1(bits(host(y)), oracle.scaled_mm_group128_act(xg_ref, wq_ref, sx_ref, sg_ref),
                f"group128 act streaming {M}x{N}x{K}")
    yh = q8.q8_scaled_mm_group128_act_f16(strided(xg_ref, M, K), wq, dev(torch.from_numpy(sx_ref)), sg)
    assert_ulp1(host(yh).view(torch.int16).numpy().view(np.uint16),
                oracle.scaled_mm_group128_act_f16(xg_ref, wq_ref, sx_ref, sg_ref),
                f"group128 act f16 streaming {M}x{N}x{K}")
    assert q8.q8_wait_timeouts(reset=True) == 0


def test_group_scaled_large_tiles_ragged():
    """Several 128 x 128 group-scaled tiles per CU (more than two rounds),
    with a ragged last tile in M and in N: both group-scaled epilogues,
    sampled rows (including the ragged ones) against the oracle."""
    M, N, K = 2100, 3728, 640
    say("group-scaled large tiles", M, N, K)
    x, w = synth.custom(M, K, N, seed=97, outlier_cols=5)
    rows = np.array([0, 1, 255, 256, 1023, 2047, 2048, 2098, 2099, 777])
    wq_ref, sg_ref = oracle.quant_weight(w.numpy(), group=128)
    xq_ref, st_ref = oracle.quant_per_token(bits(x))
    wq, sg = q8.q8_quant_weight(dev(w), group=128)
    y = q8.q8_scaled_mm_group128(dev(xq_ref), wq, dev(st_ref), sg)
    y_ref = oracle.scaled_mm_group128(xq_ref[rows], wq_ref, st_ref[rows], sg_ref)
    assert_ulp1(bits(host(y))[rows], y_ref, "group128 large tiles")
    xg_ref, sx_ref = oracle.quant_per_group128(bits(x))
    y = q8.q8_scaled_mm_group128_act(dev(xg_ref), wq, dev(sx_ref), sg)
    y_ref = oracle.scaled_mm_group128_act(xg_ref[rows], wq_ref, sx_ref[rows], sg_ref)
    assert_ulp1(bits(host(y))[rows], y_ref, "group128 act large tiles")


def test_group128_full_size_every_row():
    """The group-scaled workload 4096 x 5120 x 5120 in one launch: codes and
    scales bit-exact, every output within 1 ulp."""
    wl = synth.WORKLOADS["group128"]
    say("group128 full size, every row")
    x = synth.activations(wl, 0)
    w = synth.weights(wl, 0)
    xq_ref, st_ref = oracle.quant_per_token(bits(x))
    wq_ref, sg_ref = oracle.quant_weight(w.numpy(), group=128)
    xq, st = q8.q8_quant_per_token(dev(x))
    wq, sg = q8.q8_quant_weight(dev(w), group=128)
    np.testing.assert_array_equal(host(sg).numpy(), sg_ref)
    np.testing.assert_array_equal(host(wq).numpy(), wq_ref)
    np.testing.assert_array_equal(host(xq).numpy(), xq_ref)
    np.testing.assert_array_equal(host(st).numpy(), st_ref)
    y = q8.q8_scaled_mm_group128(xq, wq, st, sg)
    y_ref = oracle.scaled_mm_group128(xq_ref, wq_ref, st_ref, sg_ref)
    assert_ulp1(bits(host(y)), y_ref, "group128 every row")


# --------------------------------------------------------------- W8A16 --

def _check_w8a16(y_bits, x_bits, wq, s_ch, what):
    """Each row within 2e-2 relative (2-norm), and elementwise
    |y - y_ref| <= 2^-8 |y_ref| (1 + 2^-7) + 2^-134 + K 2^-22 mag: the bf16
    output rounding (half an ulp is at most 2^-8 of the value; half the
    subnormal quantum near 0) and fp32 accumulation of the exact int8 x bf16
    products (at most one rounding of the running sum, |sum| <= mag, per
    product, with 4x slack).  mag = s_ch[n] sum_k |x[m,k] w[n,k]|.  The
    elementwise bound is below 2e-2 |y_ref| + K 2^-22 mag, so it is the
    stricter of the two readings of "2e-2 relative"."""
    K = x_bits.shape[1]
    y_ref, mag = oracle.w8a16_ref(x_bits, wq, s_ch, with_mag=True)
    y = (y_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    err = np.abs(y - y_ref)
    bound = 2.0 ** -8 * np.abs(y_ref) * (1 + 2.0 ** -7) + 2.0 ** -134 + K * 2.0 ** -22 * mag
    rel = np.linalg.norm(y - y_ref, axis=1) / np.maximum(np.linalg.norm(y_ref, axis=1), 1e-30)
    say(f"{what}: max row rel {rel.max():.2e}, max err/bound {(err / bound).max():.3f}")
    assert np.all(np.isfinite(y)), what
    assert rel.max() <= 2e-2, what
    assert np.all(err <= bound), what


@pytest.mark.parametrize("M,N,K", [(16, 128, 256), (33, 144, 384), (130, 256, 1024),
                                   (64, 512, 2048), (300, 128, 13824)])
def test_w8a16_shapes(M, N, K):
    say("w8a16", M, N, K)
    wl = synth.WORKLOADS["w8a16"]
    x = synth.activations(wl, 0, M=M, K=K)
    w = synth.weights(wl, 0, N=N, K=K)
    wq_ref, sc_ref = oracle.quant_weight(w.numpy())
    wq, sc = q8.q8_quant_weight(dev(w))
    y = q8.w8a16_mm(dev(x), wq, sc)
    _check_w8a16(bits(host(y)), bits(x), wq_ref, sc_ref, f"w8a16 {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K,pad", [(1, 16, 1024, 0), (2, 1040, 3072, 16), (5, 4112, 2048, 0),
                                       (8, 5120, 17408, 0), (16, 5120, 5120, 32),
                                       (3, 17408, 5120, 0), (16, 8192, 1024, 0),
                                       (17, 5120, 3072, 16), (33, 1040, 4096, 0),
                                       (64, 5120, 17408, 0),
                                       # K not a multiple of 1024: a partial last segment
                                       (1, 16, 128, 0), (8, 5120, 13824, 0), (33, 1040, 1152, 16),
                                       (64, 4112, 4480, 0), (17, 2048, 13824, 16),
                                       # 65-112 tokens, few channel tiles: two streaming passes
                                       (65, 1040, 2048, 16), (97, 5120, 3072, 0), (112, 4112, 1152, 0),
                                       # more tokens, few channel tiles: 32 x 128 and 64 x 128 tiles
                                       (192, 5120, 1024, 0), (300, 5120, 512, 16), (130, 9216, 256, 0)])
def test_w8a16_few_tokens_weight_stream(M, N, K, pad):
    """The weight-streaming kernel (ring of 1024-deep K segments in LDS; 1,
    2 or 4 groups of 16 tokens): M <= 64 in one pass, and 65-112 tokens with
    under 64 channel tiles in two (64, then the rest), then the tiles that
    follow them (32 x 128, 64 x 128); including the down
    projection's 5120 x 17408, several workgroups per CU for large N, and K
    with a partial last segment (the W8A16 workload's 13824); strided x, w
    and y."""
    say("w8a16 stream", M, N, K, pad)
    wl = synth.WORKLOADS["w8a16"]
    xf = synth.activations(wl, 1, M=M, K=K + pad)
    xf[0] = xf[0] * 50  # a position-outlier row (as in the W8A16 workload)
    x = xf[:, :K].contiguous()
    w = synth.weights(wl, 1, N=N, K=K)
    wq_ref, sc_ref = oracle.quant_weight(w.numpy())
    wq_full = torch.zeros((N, K + pad), dtype=torch.int8, device=DEV)
    wq_full[:, :K] = dev(torch.from_numpy(wq_ref))
    yfull = torch.full((M, N + pad), -1, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    y = q8.w8a16_mm(dev(xf)[:, :K], wq_full[:, :K], dev(torch.from_numpy(sc_ref)), out=yfull[:, :N])
    _check_w8a16(bits(host(y).contiguous()), bits(x), wq_ref, sc_ref, f"w8a16 stream {M}x{N}x{K}")
    if pad:
        assert (host(yfull)[:, N:].view(torch.int16) == -1).all()


@pytest.mark.parametrize("M,N,K,pad", [(4100, 4000, 256, 0), (8192, 5120, 1024, 0), (4100, 4000, 384, 64),
                                       # one round of 256 x 128 tiles (200), and 128 x 128 below 160
                                       (1100, 5120, 512, 0), (600, 5104, 384, 32)])
def test_w8a16_big_tiles_sampled_rows(M, N, K, pad):
    """Large problems run on 256 x 320 tiles when that needs fewer whole
    waves (4100 x 4000: 544 tiles of 256 x 128 against 221 of 256 x 320);
    below one wave, on 256 x 128 tiles while they cover at least 160 CUs,
    else on 128 x 128 tiles.  Ragged tiles on both edges and, with pad,
    strided x, w and y; sampled rows, every column."""
    say("w8a16 big tiles", M, N, K, pad)
    wl = synth.WORKLOADS["w8a16"]
    xf = synth.activations(wl, 2, M=M, K=K + pad)
    x = xf[:, :K].contiguous()
    w = synth.weights(wl, 2, N=N, K=K)
    wq_ref, sc_ref = oracle.quant_weight(w.numpy())
    wq_full = torch.zeros((N, K + pad), dtype=torch.int8, device=DEV)
    wq_full[:, :K] = dev(torch.from_numpy(wq_ref))
    yfull = torch.full((M, N + pad), -1, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    y = q8.w8a16_mm(dev(xf)[:, :K], wq_full[:, :K], dev(torch.from_numpy(sc_ref)), out=yfull[:, :N])
    rows = np.unique(np.concatenate([BIG_ROWS[BIG_ROWS < M], [M - 2, M - 1]]))
    _check_w8a16(bits(host(y).contiguous())[rows], np.ascontiguousarray(bits(x)[rows]), wq_ref, sc_ref,
                 f"w8a16 big tiles {M}x{N}x{K}")
    if pad:
        assert (host(yfull)[:, N:].view(torch.int16) == -1).all(), "wrote outside the output view"


def test_w8a16_full_size_sampled_rows():
    """The W8A16 workload 8192 x 5120 x 13824 (256 x 320 tiles): weight codes
    bit-exact, and about 240 rows (all 82 position-outlier rows, tile edges,
    random) against the oracle's fp64 sums, every column."""
    wl = synth.WORKLOADS["w8a16"]
    say("w8a16 full size")
    x = synth.activations(wl, 0)
    w = synth.weights(wl, 0)
    wq_ref, sc_ref = oracle.quant_weight(w.numpy())
    wq, sc = q8.q8_quant_weight(dev(w))
    np.testing.assert_array_equal(host(wq).numpy(), wq_ref)
    np.testing.assert_array_equal(host(sc).numpy(), sc_ref)
    y = q8.w8a16_mm(dev(x), wq, sc)
    rng = np.random.default_rng(6)
    rows = np.unique(np.concatenate([np.arange(0, 84), [127, 128, 255, 256, 4095, 4096, 8190, 8191],
                                     rng.integers(84, wl.M, 150)]))
    xb = bits(x)
    _check_w8a16(bits(host(y))[rows], np.ascontiguousarray(xb[rows]), wq_ref, sc_ref,
                 "w8a16 sampled rows")


# ------------------------------------------------------- determinism ----

def test_repeat_calls_bitwise_identical():
    M, N, K = 300, 512, 1024
    x, w = synth.custom(M, K, N, seed=9, outlier_cols=10)
    wq, sc = q8.q8_quant_weight(dev(w))
    xd = dev(x)
    y1, _, _ = q8.q8_quant_scaled_mm(xd, wq, sc)
    y2, _, _ = q8.q8_quant_scaled_mm(xd, wq, sc)
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


def _random_shapes(n, seed):
    """n seeded (M, N, K) shapes over every route of the one-call layer:
    1-600 tokens, N a multiple of 16, K a multiple of 128 up to 6144, sized
    so that the oracle finishes each in well under a second."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        M = int(rng.choice([rng.integers(1, 17), rng.integers(17, 129), rng.integers(129, 601)]))
        N = 16 * int(rng.integers(1, 376))
        K = 128 * int(rng.integers(1, 49))
        if M * N * K <= 3e9:
            out.append((M, N, K))
    return out


@pytest.mark.parametrize("M,N,K", _random_shapes(24, 2026))
def test_random_shapes_every_route(M, N, K):
    """Seeded random shapes through q8_quant_scaled_mm and w8a16_mm, and
    their _ws forms where the library splits K: W8A8 codes and scales
    bit-exact and outputs within 1 ulp of the oracle (the _ws output the same
    bits as the plain call), W8A16 within its stated bound."""
    say("random shape", M, N, K, "workspace", q8.q8_workspace_bytes(M, N, K))
    x, w = synth.custom(M, K, N, seed=M * 7 + N + K, outlier_cols=max(1, K // 100))
    xq_ref, st_ref = oracle.quant_per_token(bits(x))
    wq_ref, sc_ref = oracle.quant_weight(w.numpy())
    y_ref = oracle.scaled_mm(xq_ref, wq_ref, st_ref, sc_ref)
    wq, sc = dev(torch.from_numpy(wq_ref)), dev(torch.from_numpy(sc_ref))
    xd = dev(x)
    y, xq, st = q8.q8_quant_scaled_mm(xd, wq, sc)
    np.testing.assert_array_equal(host(st).numpy(), st_ref)
    np.testing.assert_array_equal(host(xq).numpy(), xq_ref)
    yb = bits(host(y))
    assert_ulp1(yb, y_ref, f"random {M}x{N}x{K}")
    y3 = q8.w8a16_mm(xd, wq, sc)
    _check_w8a16(bits(host(y3)), bits(x), wq_ref, sc_ref, f"random w8a16 {M}x{N}x{K}")
    if q8.q8_workspace_bytes(M, N, K):
        y2, _, _ = q8.q8_quant_scaled_mm_ws(xd, wq, sc)
        np.testing.assert_array_equal(bits(host(y2)), yb)
        y4 = q8.w8a16_mm_ws(xd, wq, sc)
        _check_w8a16(bits(host(y4)), bits(x), wq_ref, sc_ref, f"random w8a16_ws {M}x{N}x{K}")
