// norm_quant.hpp -- residual add + RMSNorm + per-token INT8 quantization in
// one pass, the step that feeds a W8A8 linear layer.
//
// In the model the smoothing divisor of the W8A8 layer is folded into the
// weight of the norm before it ("Qwen3.8-27B -- SmoothQuant + activation-
// aware GPTQ, W8A8 INT8 (v3)", section "Recipe"; "Qwen3.8-27B -- FP8 block +
// AWQ", section "Recipe"), and serving stacks fuse the residual add, the
// RMSNorm and the INT8 quantization into one output step
// ("Qwen3.8-27B-GPTQ-INT8-W8A8-GS128", section "Serving (vLLM, gfx908
// fork)").  Fusing saves the normalized row's round trip through HBM: the
// row is read once (plus the residual), and only codes and one scale are
// written.
//
// Arithmetic, per row (K a multiple of 8):
//   h = bf16_rne(x + res) and res := h   (or h = x without a residual)
//   ss: the sum of the squares h[k]^2 (each exact in fp32), added in fp32:
//       64 running partial sums, lane l over its 8-element chunks l,
//       l + 64, ..., then a xor butterfly over the lanes.  The summation
//       tree has depth n_d = 8 * ceil(K / 512) + 6, so ss is within
//       n_d * 2^-24 (1 + n_d * 2^-24) of the exact sum, relative
//   rstd = 1 / sqrtf(ss / K + eps)        (correctly rounded)
//   y = bf16_rne((h * rstd) * gamma)
//   codes and scale of y exactly as the per-token quantizer.
// One wave per row, the row in registers (K <= 8192), 4 rows per workgroup.
#pragma once

#include "quant.hpp"

namespace q8 {

constexpr int NORM_MAX_K = 8192;

__device__ __forceinline__ u32 add_bf16x2(u32 a, u32 b) {
    return pack_bf16x2(bf16_lo(a) + bf16_lo(b), bf16_hi(a) + bf16_hi(b));
}

template <int NC, bool RES>
__global__ __launch_bounds__(256) void rmsnorm_quant_kernel(
    const uint16_t* x, int64_t ldx, uint16_t* res, int64_t ldr,
    const uint16_t* __restrict__ gamma, float eps, int8_t* __restrict__ xq, int64_t ldxq,
    float* __restrict__ s_tok, int M, int K) {
    const int lane = threadIdx.x & 63;
    const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (m >= M) return;
    const int nch = K >> 3;
    const v4u* xr = reinterpret_cast<const v4u*>(x + (int64_t)m * ldx);
    v4u* rr = reinterpret_cast<v4u*>(res + (int64_t)m * ldr);
    v4u h[NC];
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
        const int c = lane + 64 * i;
        if (c < nch) {
            v4u v = xr[c];
            if constexpr (RES) {
                const v4u r = rr[c];
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = add_bf16x2(v[e], r[e]);
                rr[c] = v;
            }
            h[i] = v;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float lo = bf16_lo(v[e]), hi = bf16_hi(v[e]);
                ss = ss + lo * lo;
                ss = ss + hi * hi;
            }
        }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) ss = ss + __shfl_xor(ss, o, 64);
    const float rstd = 1.0f / __builtin_sqrtf(ss / (float)K + eps);

    const v4u* gr = reinterpret_cast<const v4u*>(gamma);
    v2h mx = v2h{0, 0};
#pragma unroll
    for (int i = 0; i < NC; ++i) {
        const int c = lane + 64 * i;
        if (c < nch) {
            const v4u g = gr[c];
            v4u y;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                y[e] = pack_bf16x2((bf16_lo(h[i][e]) * rstd) * bf16_lo(g[e]),
                                   (bf16_hi(h[i][e]) * rstd) * bf16_hi(g[e]));
            h[i] = y;
            mx = mag_max8(mx, y);
        }
    }
    const RowScale q = row_scale(wave_max(mag_to_f32(mx)));
    if (lane == 0) s_tok[m] = q.s;
    v2u* qr = reinterpret_cast<v2u*>(xq + (int64_t)m * ldxq);
#pragma unroll
    for (int i = 0; i < NC; ++i) {
        const int c = lane + 64 * i;
        if (c < nch) qr[c] = codes8(h[i], q);
    }
}

template <bool RES>
inline hipError_t launch_rmsnorm_quant_r(const uint16_t* x, int64_t ldx, uint16_t* res, int64_t ldr,
                                         const uint16_t* gamma, float eps, int8_t* xq, int64_t ldxq,
                                         float* s, int M, int K, hipStream_t stream) {
    const dim3 grid((M + 3) / 4), block(256);
    const int nc = (K / 8 + 63) / 64;
#define Q8_NQ(n) hipLaunchKernelGGL((rmsnorm_quant_kernel<n, RES>), grid, block, 0, stream, x, ldx, res, \
                                    ldr, gamma, eps, xq, ldxq, s, M, K)
    if (nc <= 1) Q8_NQ(1);
    else if (nc <= 2) Q8_NQ(2);
    else if (nc <= 4) Q8_NQ(4);
    else if (nc <= 6) Q8_NQ(6);
    else if (nc <= 8) Q8_NQ(8);
    else if (nc <= 10) Q8_NQ(10);
    else if (nc <= 12) Q8_NQ(12);
    else Q8_NQ(16);
#undef Q8_NQ
    return hipGetLastError();
}

inline hipError_t launch_rmsnorm_quant(const uint16_t* x, int64_t ldx, uint16_t* res, int64_t ldr,
                                       const uint16_t* gamma, float eps, int8_t* xq, int64_t ldxq,
                                       float* s, int M, int K, hipStream_t stream) {
    return res ? launch_rmsnorm_quant_r<true>(x, ldx, res, ldr, gamma, eps, xq, ldxq, s, M, K, stream)
               : launch_rmsnorm_quant_r<false>(x, ldx, res, ldr, gamma, eps, xq, ldxq, s, M, K, stream);
}

}  // namespace q8
