"""GPU parity of the split-K entry points (caller workspace) against the
unsplit entry points and the CPU oracle.

W8A8: the planes hold exact int32 partial sums, so q8_scaled_mm_ws and
q8_quant_scaled_mm_ws must give the same bits as q8_scaled_mm /
q8_quant_scaled_mm, and within 1 bf16 ulp of the oracle.  W8A16: the fp32
partial sums are added in another order, so w8a16_mm_ws is held to the
W8A16 bound against the oracle's fp64 sums (as w8a16_mm is).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
import w8a8_int8_gemm_token_amd as q8
from tests.test_gpu_parity import DEV, _check_w8a16, assert_ulp1, bits, dev, host, say

pytestmark = pytest.mark.gpu

W8A8_SHAPES = [(65, 5120, 5120), (128, 5120, 5120), (200, 15360, 5120), (256, 5120, 5120),
               (300, 5120, 5120), (512, 5120, 5120), (97, 1040, 2048), (130, 272, 2048),
               (450, 4112, 1536),
               # 33-64 tokens: 64 x 128 tiles where the tiled kernel would run
               (40, 15360, 5120), (64, 17408, 5120), (33, 9216, 2048)]


@pytest.mark.parametrize("M,N,K", W8A8_SHAPES)
def test_scaled_mm_ws_same_bits_as_unsplit(M, N, K):
    say("scaled_mm_ws", M, N, K, "workspace", q8.q8_workspace_bytes(M, N, K))
    assert q8.q8_workspace_bytes(M, N, K) > 0  # these sizes do split
    x, w = synth.custom(M, K, N, seed=M * 7 + N + K, outlier_cols=3)
    xq_ref, st_ref = oracle.quant_per_token(bits(x))
    wq_ref, sc_ref = oracle.quant_weight(w.numpy())
    a, b = dev(torch.from_numpy(xq_ref)), dev(torch.from_numpy(wq_ref))
    st, sc = dev(torch.from_numpy(st_ref)), dev(torch.from_numpy(sc_ref))
    y0 = q8.q8_scaled_mm(a, b, st, sc)
    # a workspace larger than needed, holding garbage from an earlier use
    ws = torch.full((q8.q8_workspace_bytes(M, N, K) // 4 + 1000,), -123456789, dtype=torch.int32, device=DEV)
    y1 = q8.q8_scaled_mm_ws(a, b, st, sc, workspace=ws)
    y2 = q8.q8_scaled_mm_ws(a, b, st, sc, workspace=ws)  # the same workspace again
    assert torch.equal(host(y1).view(torch.int16), host(y0).view(torch.int16))
    assert torch.equal(host(y2).view(torch.int16), host(y0).view(torch.int16))
    rows = np.arange(M) if M * N <= 2_000_000 else np.unique(np.r_[0, 1, 127, 128, M - 1, np.arange(0, M, 37)])
    y_ref = oracle.scaled_mm(xq_ref[rows], wq_ref, st_ref[rows], sc_ref)
    assert_ulp1(bits(host(y1))[rows], y_ref, f"scaled_mm_ws {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(65, 15360, 5120), (128, 17408, 5120), (256, 5120, 5120), (97, 1040, 2048)])
def test_quant_scaled_mm_ws(M, N, K):
    """The one-call layer with a workspace: codes and scales bit-exact, the
    output the same bits as q8_quant_scaled_mm and within 1 ulp of the
    oracle; strided activations and output."""
    say("quant_scaled_mm_ws", M, N, K)
    pad = 32
    xf, _ = synth.custom(M, K + pad, N, seed=M + 5 * N, outlier_cols=3)
    x = xf[:, :K].contiguous()
    xq_ref, st_ref = oracle.quant_per_token(bits(x))
    wq_ref, sc_ref = oracle.quant_weight(synth.weights(synth.WORKLOADS["decode"], 3, N=N, K=K).numpy())
    wq, sc = dev(torch.from_numpy(wq_ref)), dev(torch.from_numpy(sc_ref))
    xd = dev(xf)[:, :K]
    yfull = torch.full((M, N + 16), -1, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    y, xq, st = q8.q8_quant_scaled_mm_ws(xd, wq, sc, out=yfull[:, :N])
    y0, _, _ = q8.q8_quant_scaled_mm(xd, wq, sc)
    np.testing.assert_array_equal(host(xq).numpy(), xq_ref)
    np.testing.assert_array_equal(host(st).numpy(), st_ref)
    assert torch.equal(host(y).contiguous().view(torch.int16), host(y0).view(torch.int16))
    assert (host(yfull)[:, N:].view(torch.int16) == -1).all(), "wrote outside the output view"
    rows = np.unique(np.r_[0, 1, M - 1, np.arange(0, M, 11)])
    y_ref = oracle.scaled_mm(xq_ref[rows], wq_ref, st_ref[rows], sc_ref)
    assert_ulp1(bits(host(y).contiguous())[rows], y_ref, f"quant_scaled_mm_ws {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(65, 5120, 17408), (128, 5120, 13824), (300, 1040, 2048),
                                   (512, 5120, 13824), (200, 4112, 4480),
                                   (40, 5120, 17408), (64, 5120, 13824), (33, 1040, 4096),
                                   (24, 5120, 17408), (32, 5120, 13824), (27, 2064, 3072)])
def test_w8a16_mm_ws(M, N, K):
    say("w8a16_mm_ws", M, N, K, "workspace", q8.q8_workspace_bytes(M, N, K))
    assert q8.q8_workspace_bytes(M, N, K) > 0
    wl = synth.WORKLOADS["w8a16"]
    x = synth.activations(wl, 3, M=M, K=K)
    x[0] = x[0] * 50
    w = synth.weights(wl, 3, N=N, K=K)
    wq_ref, sc_ref = oracle.quant_weight(w.numpy())
    y = q8.w8a16_mm_ws(dev(x), dev(torch.from_numpy(wq_ref)), dev(torch.from_numpy(sc_ref)))
    rows = np.unique(np.r_[0, 1, 2, M - 1, np.arange(0, M, 9)])
    _check_w8a16(bits(host(y))[rows], np.ascontiguousarray(bits(x)[rows]), wq_ref, sc_ref,
                 f"w8a16_mm_ws {M}x{N}x{K}")


def test_ws_entry_points_without_split_take_the_plain_routes():
    """Where no split is planned (few tokens, large problems), or the W8A8
    weight-streaming kernel runs (o_proj-like 5120 x 5120 at 33-64 tokens),
    the _ws entry points give the plain entry points' bits."""
    for M, N, K in ((8, 5120, 5120), (40, 1040, 1024), (2048, 4096, 1024), (48, 5120, 5120)):
        assert q8.q8_workspace_bytes(M, N, K) == 0 or M == 48
        x, w = synth.custom(M, K, N, seed=M + N, outlier_cols=2)
        wq, sc = q8.q8_quant_weight(dev(w))
        y0, _, _ = q8.q8_quant_scaled_mm(dev(x), wq, sc)
        y1, _, _ = q8.q8_quant_scaled_mm_ws(dev(x), wq, sc)
        assert torch.equal(host(y0).view(torch.int16), host(y1).view(torch.int16))
        if q8.q8_workspace_bytes(M, N, K) == 0:  # (W8A16 splits wherever a plan exists)
            z0 = q8.w8a16_mm(dev(x), wq, sc)
            z1 = q8.w8a16_mm_ws(dev(x), wq, sc)
            assert torch.equal(host(z0).view(torch.int16), host(z1).view(torch.int16))


def test_ws_graph_replay_matches_eager():
    """The split path captured in a HIP graph (its two kernels, no memset)
    and replayed several times, with eager work in between: every replay
    equals the eager result."""
    M, N, K = 128, 5120, 5120
    x, w = synth.custom(M, K, N, seed=44, outlier_cols=3)
    wq, sc = q8.q8_quant_weight(dev(w))
    xd = dev(x)
    ws = torch.empty((q8.q8_workspace_bytes(M, N, K),), dtype=torch.uint8, device=DEV)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    xq = torch.empty((M, K), dtype=torch.int8, device=DEV)
    st = torch.empty((M,), dtype=torch.float32, device=DEV)
    y_eager, _, _ = q8.q8_quant_scaled_mm(xd, wq, sc)
    ref = host(y_eager).view(torch.int16).clone()
    q8.q8_quant_scaled_mm_ws(xd, wq, sc, out=y, xq_out=xq, scale_tok_out=st, workspace=ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        q8.q8_quant_scaled_mm_ws(xd, wq, sc, out=y, xq_out=xq, scale_tok_out=st, workspace=ws)
    for i in range(4):
        y.zero_()
        ws.fill_(i + 7)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(host(y).view(torch.int16), ref), f"replay {i}"
