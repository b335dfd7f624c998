// decode.hpp -- fused per-token quantization + INT8 GEMM for decode-sized
// batches (M <= 16 tokens), one launch.
//
// The decode regime streams the whole weight matrix once per call and is
// bound by HBM bandwidth ("Qwen3.8-27B-INT8-W8A8", section "Throughput":
// decode is weight-bandwidth-bound).  The activation side is tiny (M rows of
// K bf16), so every workgroup quantizes it itself instead of waiting for a
// separate quantization kernel:
//   * 4*CG "weight" waves each own 16 output channels x one quarter of K.
//     They issue all their 16-byte weight loads at once (the weight bytes of
//     the whole call are in flight together) and keep them in registers as
//     MFMA A fragments (v_mfma_i32_16x16x64_i8).
//   * 4 "activation" waves meanwhile quantize the M rows (row absmax ->
//     scale -> codes, exactly as the per-token kernel) into LDS.  Their loads
//     are tracked by their own wave's counters, so they never wait behind
//     the weight stream.
//   * After one barrier the weight waves read B fragments (16 tokens) from
//     LDS, run the MFMAs, and the K-quarters are summed in LDS (exact int32)
//     before the per-token x per-channel epilogue writes bf16.
// Workgroup 0 also writes the codes and scales to global memory.
#pragma once

#include "quant.hpp"

namespace q8 {

struct DecodeArgs {
    const uint16_t* x;  // [M, ldx] bf16
    int64_t ldx;
    const int8_t* w;  // [N, ldw]
    int64_t ldw;
    const float* s_ch;  // [N]
    uint16_t* c;        // [M, ldc] bf16
    int64_t ldc;
    int8_t* xq;    // [M, K] codes out (dense)
    float* s_tok;  // [M] out
    int M, N, K;
};

constexpr int DECODE_MAX_M = 16;
constexpr int DECODE_MAX_K = 8192;  // activation row held in registers
constexpr int DECODE_WREG = 32;     // 64-wide K blocks per weight wave in registers

inline size_t decode_lds_bytes(int M, int K, int CG) {
    return (size_t)M * (K + 16) + (size_t)CG * 4 * 64 * 16 + 64 * sizeof(float);
}

template <int CG>
__global__ __launch_bounds__((4 * CG + 4) * 64) void decode_fused_kernel(DecodeArgs p) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int M = p.M, N = p.N, K = p.K;
    const int LQ = K + 16;  // padded code-row stride: rows land on distinct banks
    int8_t* lq = reinterpret_cast<int8_t*>(lds);
    v4i* red = reinterpret_cast<v4i*>(lds + (size_t)M * LQ);  // [4*CG][64]
    float* ls = reinterpret_cast<float*>(lds + (size_t)M * LQ + (size_t)CG * 4 * 64 * 16);

    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    constexpr int NWW = 4 * CG;  // weight waves
    const int nb = K >> 6;       // 64-wide K blocks

    if (wid >= NWW) {
        // ------------------------------------------- activation waves ----
        const int xw = wid - NWW;
        const int nch = K >> 3;
        for (int m = xw; m < M; m += 4) {
            const v4u* xr = reinterpret_cast<const v4u*>(p.x + (int64_t)m * p.ldx);
            v4u v[DECODE_MAX_K / 512];
            float a = 0.0f;
#pragma unroll
            for (int i = 0; i < DECODE_MAX_K / 512; ++i) {
                const int c = lane + 64 * i;
                if (c < nch) {
                    v[i] = xr[c];
                    a = __builtin_fmaxf(a, absmax8(v[i]));
                }
            }
            a = wave_max(a);
            const float s = a / 127.0f;
            if (lane == 0) {
                ls[m] = s;
                if (blockIdx.x == 0) p.s_tok[m] = s;
            }
#pragma unroll
            for (int i = 0; i < DECODE_MAX_K / 512; ++i) {
                const int c = lane + 64 * i;
                if (c < nch) {
                    const v2u q = codes8(v[i], s);
                    *reinterpret_cast<v2u*>(lq + m * LQ + c * 8) = q;
                    if (blockIdx.x == 0)
                        *reinterpret_cast<v2u*>(p.xq + (int64_t)m * K + c * 8) = q;
                }
            }
        }
        __syncthreads();  // codes ready
        __syncthreads();  // partial sums ready
        return;
    }

    // ------------------------------------------------- weight waves ------
    const int cg = wid % CG, ks = wid / CG;
    const int n0 = (blockIdx.x * CG + cg) * 16;
    const int row = lane & 15, kg = lane >> 4;
    const int8_t* wrow = p.w + (int64_t)min(n0 + row, N - 1) * p.ldw + kg * 16;
    const int b0 = ks * nb / 4, b1 = (ks + 1) * nb / 4;

    v4i acc = v4i{};
    v4i wr[DECODE_WREG];
#pragma unroll
    for (int i = 0; i < DECODE_WREG; ++i)
        if (b0 + i < b1) wr[i] = *reinterpret_cast<const v4i*>(wrow + (int64_t)(b0 + i) * 64);
    __syncthreads();  // codes ready

    const int tok = lane & 15;
    const int8_t* qrow = lq + tok * LQ + kg * 16;
#pragma unroll
    for (int i = 0; i < DECODE_WREG; ++i) {
        if (b0 + i < b1) {
            const v4i bx = tok < M ? *reinterpret_cast<const v4i*>(qrow + (b0 + i) * 64) : v4i{};
            acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(wr[i], bx, acc, 0, 0, 0);
        }
    }
    // K blocks beyond the register window (K > 4 * 64 * DECODE_WREG)
    for (int b = b0 + DECODE_WREG; b < b1; ++b) {
        const v4i a = *reinterpret_cast<const v4i*>(wrow + (int64_t)b * 64);
        const v4i bx = tok < M ? *reinterpret_cast<const v4i*>(qrow + b * 64) : v4i{};
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, bx, acc, 0, 0, 0);
    }
    red[wid * 64 + lane] = acc;
    __syncthreads();  // partial sums ready
    if (ks != 0) return;
    v4i t = acc;
#pragma unroll
    for (int s = 1; s < 4; ++s) t += red[(s * CG + cg) * 64 + lane];
    // lane holds channels n0 + 4*kg + e (e = 0..3) of token `tok`
    const int ch = n0 + 4 * kg;
    if (tok >= M || ch >= N) return;
    const float st = ls[tok];
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float u = (float)t[e] * st;
        v[e] = u * p.s_ch[ch + e];
    }
    v2u o;
    o[0] = pack_bf16x2(v[0], v[1]);
    o[1] = pack_bf16x2(v[2], v[3]);
    *reinterpret_cast<v2u*>(p.c + (int64_t)tok * p.ldc + ch) = o;
}

template <int CG>
inline hipError_t launch_decode(const DecodeArgs& p, hipStream_t stream) {
    const int groups = (p.N + 16 * CG - 1) / (16 * CG);
    const size_t lds = decode_lds_bytes(p.M, p.K, CG);
    // allow the largest dynamic LDS this kernel can ask for (M=16, K=8192)
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&decode_fused_kernel<CG>),
        hipFuncAttributeMaxDynamicSharedMemorySize,
        (int)decode_lds_bytes(DECODE_MAX_M, DECODE_MAX_K, CG));
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((decode_fused_kernel<CG>), dim3(groups), dim3((4 * CG + 4) * 64), lds,
                       stream, p);
    return hipGetLastError();
}

}  // namespace q8
