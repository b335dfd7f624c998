"""Host-side checks of the C ABI (no GPU needed, no kernel is launched).

The library must load, export every entry point that include/q8.h declares,
and reject invalid arguments with the documented status code before any HIP
call (so these calls are safe on a machine without a GPU).
"""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import w8a8_int8_gemm_token_amd as q8

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, EINVAL, EUNSUP = 0, 1, 2
A = 0x10000  # fake, 16-byte aligned "device" addresses: never dereferenced
B = 0x20000
C = 0x30000
S = 0x40000


def _declared():
    text = open(os.path.join(ROOT, "include", "q8.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(q8_\w+|w8a16_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(q8.lib_path()):
        pytest.skip("libq8.so not built")
    return q8.load()


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert set(names) == set(q8.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code in range(4):
        assert lib.q8_status_str(code)
    assert b"unknown" in lib.q8_status_str(99)


def _mm(lib, a=A, lda=256, b=B, ldb=256, st=S, sc=S, c=C, ldc=128, M=16, N=128, K=256):
    return lib.q8_scaled_mm(a, lda, b, ldb, st, sc, c, ldc, M, N, K, None)


def test_scaled_mm_validation(lib):
    assert _mm(lib, M=0) == OK                      # empty: nothing enqueued
    assert _mm(lib, M=-1) == EINVAL
    assert _mm(lib, a=None) == EINVAL
    assert _mm(lib, st=None) == EINVAL
    assert _mm(lib, K=0) == EINVAL
    assert _mm(lib, lda=128) == EINVAL               # ld < K
    assert _mm(lib, ldc=64) == EINVAL                # ld < N
    assert _mm(lib, N=120, ldc=128) == EUNSUP        # N % 16
    assert _mm(lib, K=200, lda=256, ldb=256) == EUNSUP  # K % 128
    assert _mm(lib, K=q8.MAX_K + 128, lda=10**6, ldb=10**6) == EUNSUP
    assert _mm(lib, a=A + 8) == EUNSUP               # misaligned
    assert _mm(lib, lda=264) == EUNSUP               # ld not a multiple of 16
    assert _mm(lib, ldc=132) == EUNSUP               # ldc not a multiple of 8
    assert _mm(lib, sc=S + 2) == EUNSUP              # misaligned scale


def test_other_entry_points_validation(lib):
    assert lib.q8_quant_per_token(A, 256, B, 256, S, 0, 256, None) == OK
    assert lib.q8_quant_per_token(None, 256, B, 256, S, 4, 256, None) == EINVAL
    assert lib.q8_quant_per_token(A, 100, B, 256, S, 4, 256, None) == EINVAL
    assert lib.q8_quant_per_token(A, 256, B, 256, S, 4, 0, None) == EINVAL
    assert lib.q8_scaled_mm_group128(A, 256, B, 256, S, None, C, 128, 16, 128, 256, None) == EINVAL
    assert lib.q8_scaled_mm_group128(A, 256, B, 256, S, S, C, 128, 16, 128, 192, None) == EUNSUP
    assert lib.w8a16_mm(A, 260, B, 256, S, C, 128, 16, 128, 256, None) == EUNSUP
    assert lib.w8a16_mm(A, 256, B, 256, None, C, 128, 16, 128, 256, None) == EINVAL
    assert lib.q8_mm_i32(A, 256, B, 256, C, 130, 16, 128, 256, None) == EUNSUP
    assert lib.q8_quant_scaled_mm(A, 256, B, 256, S, C, 128, None, S, 8, 128, 256, None) == EINVAL
    assert lib.q8_quant_scaled_mm(A, 256, B, 256, S, C, 128, A + 4, S, 8, 128, 256, None) == EUNSUP
    assert lib.q8_quant_weight(A, 256, B, 256, S, 16, 256, 100, None) == EUNSUP
    assert lib.q8_quant_weight(A, 256, B, 256, S, 0, 256, 128, None) == OK
    assert lib.q8_quant_weight(A, 256, B, 256, S, 16, 256, 0, None) == EINVAL
    f = ctypes.c_float
    assert lib.q8_smooth_fold(A, 256, B, 256, S, C, 256, C, 256, 0, 8, 256, f(16.0), None) == EINVAL
    assert lib.q8_smooth_fold(A, 256, B, 256, S, C, 256, C, 256, 4, 8, 256, f(0.0), None) == EINVAL


def test_rmsnorm_quant_validation(lib):
    f = ctypes.c_float
    rn = lib.q8_rmsnorm_quant
    assert rn(A, 256, None, 0, B, f(1e-6), C, 256, S, 0, 256, None) == OK   # M == 0
    assert rn(None, 256, None, 0, B, f(1e-6), C, 256, S, 4, 256, None) == EINVAL
    assert rn(A, 256, None, 0, None, f(1e-6), C, 256, S, 4, 256, None) == EINVAL
    assert rn(A, 200, None, 0, B, f(1e-6), C, 256, S, 4, 256, None) == EINVAL  # ldx < K
    assert rn(A, 256, A, 128, B, f(1e-6), C, 256, S, 4, 256, None) == EINVAL   # ldr < K
    assert rn(A, 256, None, 0, B, f(-1.0), C, 256, S, 4, 256, None) == EINVAL  # eps < 0
    assert rn(A, 256, None, 0, B, f(1e-6), C, 256, S, 4, 12, None) == EUNSUP   # K % 8
    assert rn(A, 9000, None, 0, B, f(1e-6), C, 9000, S, 4, 8200, None) == EUNSUP  # K > 8192
    assert rn(A + 8, 256, None, 0, B, f(1e-6), C, 256, S, 4, 256, None) == EUNSUP  # x misaligned
    assert rn(A, 260, None, 0, B, f(1e-6), C, 256, S, 4, 256, None) == EUNSUP  # ldx % 8
    assert rn(A, 256, None, 0, B, f(1e-6), C + 4, 256, S, 4, 256, None) == EUNSUP  # xq misaligned


def test_per_group_entry_points_validation(lib):
    qg = lib.q8_quant_per_group128
    assert qg(A, 256, B, 256, S, 0, 256, None) == OK
    assert qg(None, 256, B, 256, S, 4, 256, None) == EINVAL
    assert qg(A, 256, B, 256, S, 4, 192, None) == EUNSUP     # K % 128
    assert qg(A, 260, B, 256, S, 4, 256, None) == EUNSUP     # ldx % 8
    assert qg(A, 256, B + 4, 256, S, 4, 256, None) == EUNSUP  # xq misaligned
    ga = lib.q8_scaled_mm_group128_act
    assert ga(A, 256, B, 256, None, S, C, 128, 16, 128, 256, None) == EINVAL
    assert ga(A, 256, B, 256, S, None, C, 128, 16, 128, 256, None) == EINVAL
    assert ga(A, 256, B, 256, S, S, C, 128, 16, 128, 192, None) == EUNSUP


def test_fp8_entry_points_validation(lib):
    qf = lib.q8_quant_fp8_per_group128
    assert qf(A, 256, B, 256, S, 0, 256, None) == OK
    assert qf(None, 256, B, 256, S, 4, 256, None) == EINVAL
    assert qf(A, 256, B, 256, S, 4, 192, None) == EUNSUP     # K % 128
    assert qf(A, 260, B, 256, S, 4, 256, None) == EUNSUP     # ldx % 8
    assert qf(A, 256, B + 4, 256, S, 4, 256, None) == EUNSUP  # xq misaligned
    qw = lib.q8_quant_weight_fp8_block128
    assert qw(A, 256, B, 256, S, 0, 256, None) == OK
    assert qw(A, 256, B, 256, None, 128, 256, None) == EINVAL
    assert qw(A, 200, B, 256, S, 128, 256, None) == EINVAL   # ldw < K
    assert qw(A, 256, B, 256, S, 64, 256, None) == EUNSUP    # N % 128
    assert qw(A, 256, B, 256, S, 128, 192, None) == EUNSUP   # K % 128
    assert qw(A + 2, 256, B, 256, S, 128, 256, None) == EUNSUP
    fm = lib.q8_fp8_block_scaled_mm
    assert fm(A, 256, B, 256, S, S, C, 128, 0, 128, 256, None) == OK
    assert fm(A, 256, B, 256, None, S, C, 128, 16, 128, 256, None) == EINVAL
    assert fm(A, 256, B, 256, S, None, C, 128, 16, 128, 256, None) == EINVAL
    assert fm(A, 256, B, 256, S, S, C, 128, 16, 128, 192, None) == EUNSUP   # K % 128
    assert fm(A, 256, B, 256, S, S, C, 128, 16, 64, 256, None) == EUNSUP    # N % 128
    assert fm(A, 256, B, 256, S, S, C, 128, 16, 144, 256, None) == EINVAL   # ldc < N


def test_f16_entry_points_validation(lib):
    assert lib.q8_quant_per_token_f16(A, 256, B, 256, S, 0, 256, None) == OK
    assert lib.q8_quant_per_token_f16(None, 256, B, 256, S, 4, 256, None) == EINVAL
    assert lib.q8_scaled_mm_f16(A, 256, B, 256, S, S, C, 128, 16, 120, 256, None) == EUNSUP
    assert lib.q8_scaled_mm_f16(A, 256, B, 256, None, S, C, 128, 16, 128, 256, None) == EINVAL
    assert lib.q8_quant_scaled_mm_f16(A, 256, B, 256, S, C, 128, None, S, 16, 128, 256, None) == EINVAL
    assert lib.q8_quant_scaled_mm_f16(A, 256, B, 256, S, C, 128, B + 8, S, 16, 128, 256, None) == EUNSUP
    assert lib.q8_quant_per_group128_f16(A, 256, B, 256, S, 4, 192, None) == EUNSUP
    assert lib.q8_scaled_mm_group128_act_f16(A, 256, B, 256, S, None, C, 128, 16, 128, 256, None) == EINVAL
    assert lib.w8a16_mm_f16(A, 256, B, 256, S, C, 128, 0, 128, 256, None) == OK
    assert lib.w8a16_mm_f16(A, 260, B, 256, S, C, 128, 16, 128, 256, None) == EUNSUP
    assert lib.w8a16_mm_f16(A, 256, B, 256, None, C, 128, 16, 128, 256, None) == EINVAL
    assert lib.w8a16_mm_f16(A, 256, B, 256, S, C, 100, 16, 128, 256, None) == EINVAL


def test_binding_rejects_cpu_tensors():
    import torch
    x = torch.zeros((4, 256), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        q8.q8_quant_per_token(x)


def test_workspace_bytes_rule(lib):
    """K is split only between the few-token kernels and the large tiles,
    and the workspace never exceeds 480 tiles of 128 x 128 int32 values
    (30 MiB): checked over the model's shapes and 1-16384 tokens."""
    wb = lib.q8_workspace_bytes
    assert wb(0, 5120, 5120) == 0 and wb(-1, 16, 128) == 0
    for M in (1, 8, 16, 23):
        assert wb(M, 5120, 5120) == 0            # the streaming kernels
    assert wb(32, 5120, 17408) == 10 * 32 * 5120 * 4  # 32 x 128 tiles from 24 tokens
    assert wb(64, 5120, 17408) == 10 * 64 * 5120 * 4  # 64 x 128 tiles from 33 tokens
    assert wb(8192, 15360, 5120) == 0            # the large tiles
    seen = 0
    for N, K in ((5120, 5120), (15360, 5120), (17408, 5120), (5120, 17408), (5120, 13824)):
        for M in list(range(24, 1025, 7)) + [2048, 4096, 8192, 16384]:
            b = wb(M, N, K)
            assert 0 <= b <= 480 * 128 * 128 * 4
            if b:
                ks = b // (4 * M * N)
                assert b == ks * 4 * M * N and 2 <= ks <= 10
                seen += 1
    assert seen > 100
    assert wb(128, 5120, 5120) == 6 * 128 * 5120 * 4   # 40 tiles: 6 splits of 896 (5 x 896 + 640)


def test_workspace_validation(lib):
    """A call that needs a workspace rejects a missing or short one with
    Q8_EINVAL and a misaligned one with Q8_EUNSUPPORTED, before any HIP
    call; when none is needed, NULL is accepted.  Covers every size the
    removed split-K prototype's script swept (ks up to 12 at N = 15360,
    M <= 512), where a fixed 256 MiB buffer was too short for 9-12 planes
    of 512 x 15360 int32 values: the
    library now sizes the planes itself and refuses a short workspace."""
    M, N, K = 128, 5120, 5120
    need = lib.q8_workspace_bytes(M, N, K)
    assert need > 0
    W = 0x50000
    for fn, args in (
            (lib.q8_scaled_mm_ws, (A, K, B, K, S, S, C, N, M, N, K)),
            (lib.q8_quant_scaled_mm_ws, (A, K, B, K, S, C, N, A, S, M, N, K)),
            (lib.w8a16_mm_ws, (A, K, B, K, S, C, N, M, N, K))):
        assert fn(*args, None, need, None) == EINVAL
        assert fn(*args, W, need - 1, None) == EINVAL
        assert fn(*args, W + 8, need, None) == EUNSUP
        assert fn(*args[:-3], 0, N, K, None, 0, None) == OK   # M = 0: nothing to do
    # no split below 24 tokens: no workspace needed (NULL accepted)
    assert lib.q8_workspace_bytes(16, N, K) == 0
    # the old prototype's sweep: 256 MiB against the planes it wrote
    old = 64 << 20 << 2
    short = [(m, ks) for m in (65, 128, 256, 512) for ks in range(2, 13)
             if ks * m * 15360 * 4 > old]
    assert short == [(512, ks) for ks in range(9, 13)]   # what overran it
    for m in (65, 128, 256, 512):
        assert lib.q8_workspace_bytes(m, 15360, 5120) <= 480 * 128 * 128 * 4 < old
