// w8a16.hpp -- weight-only INT8 GEMM with bf16 activations on CDNA4 bf16
// MFMA (v_mfma_f32_32x32x16_bf16), fp32 accumulation, bf16 out:
//   y[m,n] = bf16_rne( s_ch[n] * sum_k x[m,k] * bf16(w[n,k]) )
// "Qwen3.8-27B -- SmoothQuant + activation-aware GPTQ, W8A8 INT8 (v3)",
// section "Recipe" (W8A16 modules: INT8 per-channel weights, BF16
// activations); "lued/Qwen3.8-27B-INT8-W8A16-MTP", section "Why W8A16 on
// Ampere" (weight-only kernels rebuild the weights for a 16-bit GEMM).
//
// This kernel serves M <= 64 when the weight-streaming kernel does not apply;
// larger M runs the tiled INT8 GEMM's bf16 mode (EPI_W8A16 in gemm_i8.hpp).
// F16: fp16 activations and outputs instead (v_mfma_f32_32x32x16_f16; the
// int8 weights are exact in fp16 as well).
//
// Design: same tile/wave structure as the INT8 GEMM.  The int8 weight tile
// is read from HBM as int8 (half the bytes of bf16) and converted exactly to
// bf16 once per workgroup while it is written to LDS (|q| <= 128 fits bf16's
// 8-bit significand), so every wave that reads a weight fragment gets bf16
// without re-converting.  The channel scale is applied once, in the fp32
// epilogue.
#pragma once

#include "q8_device.hpp"

namespace q8 {

struct W8A16Args {
    const uint16_t* x;  // [M, ldx] bf16 (fp16 when F16)
    int64_t ldx;
    const int8_t* w;  // [N, ldw] int8
    int64_t ldw;
    const float* s_ch;  // [N]
    uint16_t* c;        // [M, ldc] bf16 (fp16 when F16)
    int64_t ldc;
    int M, N, K;
};

template <int BM, int BN, int BK, int WM, int WN, int GM, bool F16>
__global__ __launch_bounds__(WM* WN * 64) void w8a16_kernel(W8A16Args p) {
    constexpr int NT = WM * WN * 64;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int TM = WTM / 32, TN = WTN / 32;
    constexpr int LDSW = 2 * BK + 16;  // bf16 rows, padded (bytes)
    constexpr int XCPR = 2 * BK / 16;  // 16-byte chunks of x per row
    constexpr int WCPR = BK / 16;      // 16-byte chunks of w (int8) per row
    constexpr int XCH = BM * XCPR / NT;
    constexpr int WCH = BN * WCPR / NT;
    constexpr int KK = BK / 16;
    static_assert(TM * 32 * WM == BM && TN * 32 * WN == BN, "tile shape");
    static_assert(XCH * NT == BM * XCPR && WCH * NT == BN * WCPR, "load split");

    __shared__ __attribute__((aligned(16))) uint8_t lx[2][BM * LDSW];
    __shared__ __attribute__((aligned(16))) uint8_t lw[2][BN * LDSW];

    const int M = p.M, N = p.N, K = p.K;
    const int nbm = (M + BM - 1) / BM, nbn = (N + BN - 1) / BN;
    const int id = xcd_remap(blockIdx.x, nbm * nbn);
    const int per_group = GM * nbn;
    const int first_m = (id / per_group) * GM;
    const int gsz = min(nbm - first_m, GM);
    const int tile_m = first_m + (id % per_group) % gsz;
    const int tile_n = (id % per_group) / gsz;
    const int m0 = tile_m * BM, n0 = tile_n * BN;

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int wm = wid % WM, wn = wid / WM;

    const uint8_t* xs[XCH];
    int xo[XCH];
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
        const int cidx = tid + i * NT, r = cidx / XCPR, q = cidx % XCPR;
        xs[i] = reinterpret_cast<const uint8_t*>(p.x + (int64_t)min(m0 + r, M - 1) * p.ldx) + q * 16;
        xo[i] = r * LDSW + q * 16;
    }
    const int8_t* ws[WCH];
    int wo[WCH];
#pragma unroll
    for (int i = 0; i < WCH; ++i) {
        const int cidx = tid + i * NT, r = cidx / WCPR, q = cidx % WCPR;
        ws[i] = p.w + (int64_t)min(n0 + r, N - 1) * p.ldw + q * 16;
        wo[i] = r * LDSW + q * 32;
    }

    v4i rx[XCH], rw[WCH];
    v16f acc[TM][TN];
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int b = 0; b < TN; ++b) acc[a][b] = v16f{};

    auto gload = [&](int kt) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < XCH; ++i) rx[i] = *reinterpret_cast<const v4i*>(xs[i] + (int64_t)kt * 2 * BK);
#pragma unroll
        for (int i = 0; i < WCH; ++i) rw[i] = *reinterpret_cast<const v4i*>(ws[i] + (int64_t)kt * BK);
    };
    auto lstore = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < XCH; ++i) *reinterpret_cast<v4i*>(&lx[buf][xo[i]]) = rx[i];
#pragma unroll
        for (int i = 0; i < WCH; ++i) {
            const v2u a = i8x4_to_h16x4<F16>(rw[i][0]), b = i8x4_to_h16x4<F16>(rw[i][1]);
            const v2u c = i8x4_to_h16x4<F16>(rw[i][2]), d = i8x4_to_h16x4<F16>(rw[i][3]);
            *reinterpret_cast<v4u*>(&lw[buf][wo[i]]) = v4u{a[0], a[1], b[0], b[1]};
            *reinterpret_cast<v4u*>(&lw[buf][wo[i] + 16]) = v4u{c[0], c[1], d[0], d[1]};
        }
    };

    const int frow = lane & 31, fk = (lane >> 5) * 16;
    auto compute = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            v8bf fw[TN], fx[TM];
#pragma unroll
            for (int b = 0; b < TN; ++b)
                fw[b] = *reinterpret_cast<const v8bf*>(
                    &lw[buf][(wn * WTN + b * 32 + frow) * LDSW + kk * 32 + fk]);
#pragma unroll
            for (int a = 0; a < TM; ++a)
                fx[a] = *reinterpret_cast<const v8bf*>(
                    &lx[buf][(wm * WTM + a * 32 + frow) * LDSW + kk * 32 + fk]);
#pragma unroll
            for (int a = 0; a < TM; ++a)
#pragma unroll
                for (int b = 0; b < TN; ++b) {
                    if constexpr (F16)
                        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, fw[b]),
                                                                           __builtin_bit_cast(v8h, fx[a]),
                                                                           acc[a][b], 0, 0, 0);
                    else
                        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[b], fx[a], acc[a][b], 0, 0, 0);
                }
        }
    };

    const int KT = K / BK;
    gload(0);
    lstore(0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < KT) gload(kt + 1);
        compute(cur);
        if (kt + 1 < KT) lstore(cur ^ 1);
        __syncthreads();
    }

#pragma unroll
    for (int a = 0; a < TM; ++a) {
        const int j = m0 + wm * WTM + a * 32 + (lane & 31);
        if (j >= M) continue;
#pragma unroll
        for (int b = 0; b < TN; ++b) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int ch = n0 + wn * WTN + b * 32 + g * 8 + (lane >> 5) * 4;
                if (ch >= N) continue;
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = p.s_ch[ch + e] * acc[a][b][g * 4 + e];
                *reinterpret_cast<v2u*>(p.c + (int64_t)j * p.ldc + ch) =
                    v2u{pack16x2<F16>(v[0], v[1]), pack16x2<F16>(v[2], v[3])};
            }
        }
    }
}

template <int BM, int BN, int BK, int WM, int WN, int GM, bool F16>
inline hipError_t launch_w8a16(const W8A16Args& p, hipStream_t stream) {
    const int nbm = (p.M + BM - 1) / BM, nbn = (p.N + BN - 1) / BN;
    hipLaunchKernelGGL((w8a16_kernel<BM, BN, BK, WM, WN, GM, F16>), dim3(nbm * nbn), dim3(WM * WN * 64),
                       0, stream, p);
    return hipGetLastError();
}

}  // namespace q8
