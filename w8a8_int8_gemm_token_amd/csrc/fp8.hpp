// fp8.hpp -- FP8 (E4M3) block-scaled quantization for the FP8 W8A8 layer:
// dynamic per-token-per-128-group activations and offline [128,128] block
// weights ("Qwen3.8-27B -- FP8 block + AWQ", section "Recipe": FP8
// block-scaled [128,128] weights with dynamic per-group activations, every
// quantized dimension a multiple of 128; the same page's "KV cache" section
// scales E4M3 by amax/448).
//
// E4M3 is the OCP 8-bit float: sign, 4 exponent bits (bias 7), 3 mantissa
// bits, largest finite value 448 (S.1111.110; S.1111.111 is NaN), subnormal
// quantum 2^-9.  A block scale is s = fl32(absmax / 448) (one IEEE division;
// 0 for an all-zero block, whose codes are +0), and a code is the E4M3 value
// nearest to the correctly rounded quotient fl32(x / s), ties to the even
// mantissa, magnitudes from 448 up saturating to 448, sign kept.
#pragma once

#include "quant.hpp"

namespace q8 {

constexpr u32 E4M3_MIN_NORMAL_BITS = 121u << 23;  // 2^-6 as fp32 bits

// E4M3 code (7 magnitude bits) of a non-negative fp32 bit pattern a >= 2^-6:
// round to nearest even at fp32 mantissa bit 20 (E4M3 keeps 3 of the 23
// mantissa bits), rebias the exponent (127 -> 7), saturate at 0x7E.  Exact
// for every finite a in that range (inf also saturates).
__device__ __forceinline__ u32 e4m3_code_normal(u32 a) {
    const u32 r = (a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20;  // (exponent << 3 | mantissa), rounded
    const u32 c = r - (120u << 3);
    return c < 0x7Eu ? c : 0x7Eu;
}

// E4M3 code of any finite fp32 value q (the reference route, used for the
// quotient computed by division).
__device__ __forceinline__ u32 e4m3_code_exact(float q) {
    const u32 u = __float_as_uint(q);
    const u32 a = u & 0x7FFFFFFFu;
    u32 c;
    if (a >= E4M3_MIN_NORMAL_BITS)
        c = e4m3_code_normal(a);
    else  // subnormal range: quantum 2^-9, |q| * 512 is exact
        c = (u32)__builtin_rintf(__uint_as_float(a) * 512.0f);
    return ((u >> 24) & 0x80u) | c;
}

// E4M3 code of x under block scale s, by IEEE division.
__device__ __forceinline__ u32 e4m3_code_of(float x, float s) {
    if (s == 0.0f) return 0u;
    return e4m3_code_exact(x / s);
}

// Per-block constants: s = absmax / 448, r = fl(1/s).
struct BlockScale8 {
    float s, r;
    bool fast;  // s normal: the reciprocal route applies
};
__device__ __forceinline__ BlockScale8 block_scale8(float absmax) {
    BlockScale8 q;
    q.s = absmax / 448.0f;
    q.fast = q.s >= 0x1p-125f;
    q.r = q.fast ? 1.0f / q.s : 0.0f;
    return q;
}

// The 8 codes of the 8 bf16 values in v, packed little-endian, bit-identical
// to e4m3_code_of.  Fast route: t = fl(x * r), r = fl(1/s), converted by the
// hardware (v_cvt_pk_fp8_f32: OCP E4M3, round to nearest even; |t| <= 448
// (1 + 2^-22) here, so nothing saturates).  t differs from x/s by at most
// |x/s| * (2^-23 + 2^-48), and the correctly rounded quotient from x/s by
// half an ulp, so their distance is under 3 ulps of t.  E4M3 rounding of a
// normal-range t looks only at fp32 mantissa bits 19..0: when those lie
// more than 7 ulps from the halfway pattern 0x80000, the quotient rounds the
// same way (crossing a power of two keeps the grid point).  Any other
// element (a near-halfway t, about 1 element in 30,000, or a nonzero t
// below 2^-6, the E4M3 subnormal range) is recomputed by division.
__device__ __forceinline__ v2u e4m3_codes8(v4u v, const BlockScale8& q) {
    float t[8];
    bool redo = false;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float x = (e & 1) ? bf16_hi(v[e >> 1]) : bf16_lo(v[e >> 1]);
        t[e] = x * q.r;
        const u32 a = __float_as_uint(t[e]) & 0x7FFFFFFFu;
        redo |= (a - 1u) < (E4M3_MIN_NORMAL_BITS - 1u);       // 0 < |t| < 2^-6
        redo |= ((a + 8u) & 0xFFFF0u) == 0x80000u;             // near halfway
    }
    v2u r;
    r[0] = (u32)__builtin_amdgcn_cvt_pk_fp8_f32(t[0], t[1], 0, false);
    r[0] = (u32)__builtin_amdgcn_cvt_pk_fp8_f32(t[2], t[3], (int)r[0], true);
    r[1] = (u32)__builtin_amdgcn_cvt_pk_fp8_f32(t[4], t[5], 0, false);
    r[1] = (u32)__builtin_amdgcn_cvt_pk_fp8_f32(t[6], t[7], (int)r[1], true);
    if (!q.fast || redo) {  // rare: redo by division
        u32 c[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float x = (e & 1) ? bf16_hi(v[e >> 1]) : bf16_lo(v[e >> 1]);
            c[e] = e4m3_code_of(x, q.s);
        }
        r[0] = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
        r[1] = c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24);
    }
    return r;
}

// Dynamic per-token-per-group FP8 activations: one scale per (row, 128-wide
// K block).  One wave per 512-value span of a row: lane l holds chunk l (8
// values), lanes 16g .. 16g+15 form block g of the span (one DPP row), whose
// absmax takes four row rotations.  K % 128 == 0; 16-byte aligned x rows,
// 8-byte aligned xq rows; s [M, K/128] dense.
__global__ __launch_bounds__(256) void quant_fp8_per_group128_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, uint8_t* __restrict__ xq, int64_t ldxq,
    float* __restrict__ s, int M, int K) {
    const int lane = threadIdx.x & 63;
    const int spans = (K + 511) >> 9;
    const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int m = wave / spans, sp = wave - m * spans;
    if (m >= M) return;
    const int c = sp * 64 + lane;
    const bool ok = c < (K >> 3);
    v4u v = v4u{};
    if (ok) v = reinterpret_cast<const v4u*>(x + (int64_t)m * ldx)[c];
    const float a = row16_max(mag_to_f32(mag_max8(v2h{0, 0}, v)));
    const BlockScale8 q = block_scale8(a);
    if (!ok) return;
    reinterpret_cast<v2u*>(xq + (int64_t)m * ldxq)[c] = e4m3_codes8(v, q);
    if ((lane & 15) == 0) s[(int64_t)m * (K >> 7) + (c >> 4)] = q.s;
}

// Offline FP8 block weights: one 256-thread workgroup per [128,128] block of
// the fp32 weight (block (nb, g) = rows 128nb.., columns 128g..): absmax over
// the block, s = absmax / 448 into s_w[nb * G + g], codes by division.
__global__ __launch_bounds__(256) void quant_weight_fp8_block_kernel(
    const float* __restrict__ w, int64_t ldw, uint8_t* __restrict__ wq, int64_t ldwq,
    float* __restrict__ s_w, int G) {
    __shared__ float red[4];
    const int nb = blockIdx.x / G, g = blockIdx.x % G;
    const float* src = w + (int64_t)nb * 128 * ldw + (int64_t)g * 128;
    uint8_t* dst = wq + (int64_t)nb * 128 * ldwq + (int64_t)g * 128;
    const int col = threadIdx.x & 127, r0 = threadIdx.x >> 7;
    float a = 0.0f;
    for (int r = r0; r < 128; r += 2) a = __builtin_fmaxf(a, __builtin_fabsf(src[(int64_t)r * ldw + col]));
    a = wave_max(a);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = a;
    __syncthreads();
    a = __builtin_fmaxf(__builtin_fmaxf(red[0], red[1]), __builtin_fmaxf(red[2], red[3]));
    const float sc = a / 448.0f;
    if (threadIdx.x == 0) s_w[blockIdx.x] = sc;
    for (int r = r0; r < 128; r += 2)
        dst[(int64_t)r * ldwq + col] = (uint8_t)e4m3_code_of(src[(int64_t)r * ldw + col], sc);
}

}  // namespace q8
