"""The allocation-free variant of the one-call layer (q8_quant_scaled_mm_noalloc,
for callers that cannot allocate device memory) against the workspace entry
point it stands for (q8_quant_scaled_mm_ws), through the C ABI.

Two calls in a row on the library's one array per GPU, the second with a
smaller input, each bit-identical to q8_quant_scaled_mm_ws with a workspace
of the caller's (W8A8 sums are exact, so the two must agree bit for bit):
the second call must not see the first one's partial sums.  Then a size that
does not split K (no array use), and the host-side checks.
"""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth
import w8a8_int8_gemm_token_amd as q8

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _layer_inputs(M, N, K, seed):
    x, _ = synth.custom(M, K, N, seed=seed, outlier_cols=3)
    w = synth.weights(synth.WORKLOADS["decode"], seed, N=N, K=K)
    wq, sc = q8.q8_quant_weight(w.to(DEV))
    return x.to(DEV), wq, sc


def _run_both(M, N, K, seed):
    x, wq, sc = _layer_inputs(M, N, K, seed)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    xq = torch.empty((M, K), dtype=torch.int8, device=DEV)
    st = torch.empty((M,), dtype=torch.float32, device=DEV)
    q8.q8_quant_scaled_mm_noalloc(x, wq, sc, y, xq, st)
    y_ws, xq_ws, st_ws = q8.q8_quant_scaled_mm_ws(x, wq, sc)
    torch.cuda.synchronize()
    assert torch.equal(xq.cpu(), xq_ws.cpu())
    assert torch.equal(st.cpu().view(torch.int32), st_ws.cpu().view(torch.int32))
    assert torch.equal(y.cpu().view(torch.int16), y_ws.cpu().view(torch.int16))
    return x, wq, sc, y, xq, st


def test_noalloc_two_calls_match_the_workspace_entry_point():
    # first call: the largest workspace the split rule asks for (30 MiB)
    M1, N1, K1 = 256, 5120, 5120
    assert q8.q8_workspace_bytes(M1, N1, K1) == 480 * 128 * 128 * 4
    _run_both(M1, N1, K1, seed=11)
    # second call, smaller, on the same array: its own sums only
    M2, N2, K2 = 97, 1040, 2048
    assert 0 < q8.q8_workspace_bytes(M2, N2, K2) < q8.q8_workspace_bytes(M1, N1, K1)
    x, wq, sc, y, xq, st = _run_both(M2, N2, K2, seed=12)
    # and against the oracle (1 ulp), sampled rows
    xq_ref, st_ref = oracle.quant_per_token(synth.bf16_bits(x.cpu()))
    np.testing.assert_array_equal(xq.cpu().numpy(), xq_ref)
    rows = np.array([0, 1, 50, 95, 96])
    y_ref = oracle.scaled_mm(xq_ref[rows], wq.cpu().numpy(), st_ref[rows], sc.cpu().numpy())
    yb = synth.bf16_bits(y.cpu())[rows].astype(np.int32)
    o = lambda u: np.where(u & 0x8000, -(u & 0x7FFF), u)  # noqa: E731
    assert np.abs(o(yb) - o(y_ref.astype(np.int32))).max() <= 1


def test_noalloc_without_split_and_host_checks():
    # a size that does not split K: the array is not used
    assert q8.q8_workspace_bytes(8, 5120, 5120) == 0
    _run_both(8, 5120, 5120, seed=13)
    lib = q8.load()
    A, B, C, S = 0x10000, 0x20000, 0x30000, 0x40000
    f = lib.q8_quant_scaled_mm_noalloc
    assert f(A, 256, B, 256, S, C, 128, A, S, 0, 128, 256, None) == 0          # empty
    assert f(None, 256, B, 256, S, C, 128, A, S, 8, 128, 256, None) == 1       # null x
    assert f(A, 256, B, 256, S, C, 128, None, S, 8, 128, 256, None) == 1       # null xq
    assert f(A, 256, B, 256, S, C, 128, A + 4, S, 8, 128, 256, None) == 2      # misaligned xq
    assert f(A, 256, B, 256, S, C, 128, A, S, 8, 120, 256, None) == 2          # N % 16
    assert q8.NOALLOC_MAX_WORKSPACE >= 480 * 128 * 128 * 4
