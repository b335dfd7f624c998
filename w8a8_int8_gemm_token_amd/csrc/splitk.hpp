// splitk.hpp -- split-K for the tiled GEMMs when the output has too few
// tiles to fill the chip (roughly 65-512 tokens): each output tile is
// computed by ks workgroups, each over a contiguous range of K, writing raw
// partial sums to planes of a caller-supplied workspace; splitk_reduce then
// adds the planes and applies the epilogue.
//
// W8A8 ("Qwen3.8-27B -- SmoothQuant + activation-aware GPTQ, W8A8 INT8
// (v3)", "Recipe" and "Serving"): the planes hold exact int32 partial sums
// and are added in int32, which is exact and order-free, so the sum equals
// the unsplit acc[m,n] and the epilogue bf16_rne(((float)acc * s_tok[m]) *
// s_ch[n]) gives the same bits as the unsplit kernel.
// W8A16 ("lued/Qwen3.8-27B-INT8-W8A16-MTP", "Why W8A16 on Ampere"): the
// planes hold fp32 partial sums of the bf16 (fp16) products, added in fp32
// in plane order; the summation order is the hardware's either way, and the
// result stays within the same fp32 accumulation bound.
//
// Workspace: ks planes of [M][N] 4-byte values (dense, leading dimension
// N), ks * M * N * 4 bytes, every element of every plane written before it
// is read, so the workspace needs no clearing and holds nothing between
// calls.
#pragma once

#include "gemm_i8.hpp"

namespace q8 {

// MODE: 0 int32 planes -> per-channel epilogue; 1 fp32 planes -> W8A16
// epilogue.  F16: fp16 outputs instead of bf16.
template <int MODE, bool F16>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const int32_t* __restrict__ ws, int ks,
                                                            int64_t plane, const float* __restrict__ s_tok,
                                                            const float* __restrict__ s_ch, uint16_t* c,
                                                            int64_t ldc, int M, int N) {
    const int nq = N >> 2;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)M * nq) return;
    const int m = (int)(idx / nq), n = (int)(idx - (int64_t)m * nq) * 4;
    const v4i* src = reinterpret_cast<const v4i*>(ws + (int64_t)m * N + n);
    const int64_t pq = plane >> 2;  // plane stride in 16-byte units
    float v[4];
    if constexpr (MODE == 0) {
        v4i a = __builtin_nontemporal_load(src);
        for (int z = 1; z < ks; ++z) a += __builtin_nontemporal_load(src + z * pq);
        const float st = s_tok[m];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float t = (float)a[e] * st;
            v[e] = t * s_ch[n + e];
        }
    } else {
        v4f a = __builtin_bit_cast(v4f, __builtin_nontemporal_load(src));
        for (int z = 1; z < ks; ++z) {
            const v4f b = __builtin_bit_cast(v4f, __builtin_nontemporal_load(src + z * pq));
#pragma unroll
            for (int e = 0; e < 4; ++e) a[e] = a[e] + b[e];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = s_ch[n + e] * a[e];
    }
    v2u o;
    o[0] = pack16x2<F16>(v[0], v[1]);
    o[1] = pack16x2<F16>(v[2], v[3]);
    *reinterpret_cast<v2u*>(c + (int64_t)m * ldc + n) = o;
}

template <int MODE, bool F16>
inline hipError_t launch_splitk_reduce(const int32_t* ws, int ks, int64_t plane, const float* s_tok,
                                       const float* s_ch, uint16_t* c, int64_t ldc, int M, int N,
                                       hipStream_t stream) {
    const int64_t quads = (int64_t)M * (N / 4);
    hipLaunchKernelGGL((splitk_reduce_kernel<MODE, F16>), dim3((unsigned)((quads + 255) / 256)), dim3(256), 0,
                       stream, ws, ks, plane, s_tok, s_ch, c, ldc, M, N);
    return hipGetLastError();
}

}  // namespace q8
