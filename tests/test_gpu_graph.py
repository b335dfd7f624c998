"""The library's calls captured in a HIP graph (as the benchmark times the
decode path): every replay, with eager work and synchronizations between
replays, must reproduce the eager result bit for bit."""
from __future__ import annotations

import pytest
import torch

import synth
import w8a8_int8_gemm_token_amd as q8

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,K,N", [(1, 1024, 512), (8, 1024, 512), (300, 1024, 512),
                                   (8, 5120, 5120),    # one-kernel decode, five K segments
                                   (3, 5120, 15360),   # ... three workgroups per CU
                                   (16, 5120, 5120),   # quantizer + weight-streaming kernel
                                   (16, 256, 128),     # the small-layer kernel (the tiny workload)
                                   (5, 640, 2064)])    # ... three workgroups, the last one ragged
def test_graph_replay_matches_eager(M, K, N):
    dev = "cuda:0"
    x, w = synth.custom(M, K, N, seed=40 + M, outlier_cols=8)
    x, w = x.to(dev), w.to(dev)
    wq, sc = q8.q8_quant_weight(w)
    y_ref, xq_ref, st_ref = q8.q8_quant_scaled_mm(x, wq, sc)
    torch.cuda.synchronize()
    y = torch.empty_like(y_ref)
    xq = torch.empty_like(xq_ref)
    st = torch.empty_like(st_ref)
    q8.q8_quant_scaled_mm(x, wq, sc, out=y, xq_out=xq, scale_tok_out=st)  # warm up
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        q8.q8_quant_scaled_mm(x, wq, sc, out=y, xq_out=xq, scale_tok_out=st)
    for r in range(4):
        y.zero_()
        xq.zero_()
        st.zero_()
        q8.q8_quant_per_token(x)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), r
        assert torch.equal(xq, xq_ref), r
        assert torch.equal(st, st_ref), r
