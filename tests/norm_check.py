"""Validity check for the fused residual add + RMSNorm + per-token quant.

The plain definition (the oracle) takes ss, the sum of the squares of the
row, as the exact sum rounded once to fp32.  A kernel sums in fp32 in an
order of its own, so its ss may differ from that value by the error of its
summation.  The library states that error for its kernel: every square is
exact, and the K squares are added in 64 running partial sums of at most
8*ceil(K/512) terms each, then combined pairwise in 6 levels, so

    |ss_kernel - S| <= n_d * u * (1 + n_d * u) * S,   n_d = 8*ceil(K/512) + 6,

with S the exact sum and u = 2^-24 (the standard bound for a summation tree
of depth n_d over nonnegative terms).  A row is valid when the kernel's codes
and scale equal the oracle's normalization and quantization at one fp32 ss
inside that interval (q8o_rmsnorm_quant_at_ss computes them).  Candidates are
tried outwards from the correctly rounded value, so a row usually settles at
the first or second one; a row that matches none of them is a failure.
"""
from __future__ import annotations

import numpy as np

import oracle

U = 2.0 ** -24


def depth(K: int) -> int:
    return 8 * -(-K // 512) + 6


def check_rows(h_bits, gamma_bits, eps, xq_got, s_got, max_fail_report=5):
    """h_bits: the rows after the residual add (bf16 bits [M,K]); xq_got,
    s_got: the kernel's codes and scales.  Returns (n_exact, n_neighbour,
    offsets) and raises AssertionError naming the rows that fit no ss in the
    stated interval."""
    h = np.ascontiguousarray(h_bits, dtype=np.uint16)
    M, K = h.shape
    ss0 = oracle.sum_squares_bf16(h)
    xq0, s0, _ = oracle.rmsnorm_quant_at_ss(h, gamma_bits, eps, ss0)
    ok = np.all(xq0 == xq_got, axis=1) & (s0.view(np.int32) == np.asarray(s_got, np.float32).view(np.int32))
    n_exact = int(ok.sum())
    nd = depth(K)
    # half an ulp of ss0 covers the difference between S and its rounding
    bound = nd * U * (1 + nd * U) * ss0.astype(np.float64) * (1 + U) + \
        np.spacing(ss0).astype(np.float64) / 2
    todo = np.nonzero(~ok)[0]
    # fp32 values below ss0 are at least half its spacing apart
    half_sp = np.spacing(ss0).astype(np.float64) / 2
    reach = np.ceil(bound / np.maximum(half_sp, 2.0 ** -149)).astype(np.int64) + 1
    offsets = {}
    step_max = int(reach[todo].max()) if len(todo) else 0
    for mag in range(1, step_max + 1):
        for step in (mag, -mag):
            if not len(todo):
                break
            cand_bits = ss0[todo].view(np.int32).astype(np.int64) + step
            inside = cand_bits >= 0
            cand = np.where(inside, cand_bits, 0).astype(np.int32).view(np.float32)
            inside &= np.abs(cand.astype(np.float64) - ss0[todo].astype(np.float64)) <= bound[todo]
            rows = todo[inside]
            if not len(rows):
                continue
            xq1, s1, _ = oracle.rmsnorm_quant_at_ss(h[rows], gamma_bits, eps, cand[inside])
            hit = np.all(xq1 == xq_got[rows], axis=1) & \
                (s1.view(np.int32) == np.asarray(s_got, np.float32)[rows].view(np.int32))
            for r in rows[hit]:
                offsets[int(r)] = step
            todo = np.setdiff1d(todo, rows[hit])
    if len(todo):
        raise AssertionError(f"{len(todo)} rows fit no sum of squares within {nd} u of the exact one, "
                             f"e.g. rows {todo[:max_fail_report].tolist()}")
    return n_exact, len(offsets), offsets
