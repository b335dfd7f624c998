// quant.hpp -- per-token activation quantization, offline weight quantization
// and the smoothing fold, for gfx950.
//
// Per-token dynamic symmetric INT8 ("Qwen3.8-27B -- SmoothQuant +
// activation-aware GPTQ, W8A8 INT8 (v3)", section "Recipe";
// "Qwen3.8-27B-INT8-W8A8", section "Quantization"): per row, scale =
// absmax/127 (one correctly rounded division), code = clamp(rne(x/scale),
// -127, 127).  HBM-bound: one read of the bf16 row, one write of the codes.
// The kernels take bf16 rows, or fp16 rows with F16 = true (the fp16
// variant: "Qwen3.8-27B-GPTQ-INT8-W8A8-GS128", "Serving (vLLM, gfx908
// fork)", where the model runs in half precision).
#pragma once

#include "q8_device.hpp"

namespace q8 {

// Running max of |x| over bf16 (or fp16) values, kept as two 16-bit
// magnitudes: for finite values the magnitude bits (sign cleared) order the
// same way as |x|,
// so a packed unsigned max gives the exact absmax at one VALU op per value.
typedef unsigned short v2h __attribute__((ext_vector_type(2)));
__device__ __forceinline__ v2h mag_max8(v2h acc, v4u v) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
        acc = __builtin_elementwise_max(acc, __builtin_bit_cast(v2h, v[e] & 0x7FFF7FFFu));
    return acc;
}
template <bool F16 = false>
__device__ __forceinline__ float mag_to_f32(v2h acc) {
    const u32 m = acc[0] > acc[1] ? acc[0] : acc[1];
    return h16_to_f32<F16>((uint16_t)m);
}

// Maximum of a non-negative float over the 16 lanes of each DPP row (lanes
// 16g .. 16g+15): rotations by 8, 4, 2 and 1 within the row leave every lane
// with the row's maximum, without a trip through the LDS crossbar.
__device__ __forceinline__ float row16_max(float a) {
    a = __builtin_fmaxf(a, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a), 0x128, 0xF, 0xF, false)));
    a = __builtin_fmaxf(a, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a), 0x124, 0xF, 0xF, false)));
    a = __builtin_fmaxf(a, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a), 0x122, 0xF, 0xF, false)));
    a = __builtin_fmaxf(a, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a), 0x121, 0xF, 0xF, false)));
    return a;
}

// The 8 codes of the 8 bf16 (or fp16) values in v, packed little-endian, each with a
// full IEEE division (the reference route).
template <bool F16 = false>
__device__ __forceinline__ v2u codes8_div(v4u v, float s) {
    v2u r;
    r[0] = pack_i8x4(code_of(h16_lo<F16>(v[0]), s), code_of(h16_hi<F16>(v[0]), s),
                    code_of(h16_lo<F16>(v[1]), s), code_of(h16_hi<F16>(v[1]), s));
    r[1] = pack_i8x4(code_of(h16_lo<F16>(v[2]), s), code_of(h16_hi<F16>(v[2]), s),
                    code_of(h16_lo<F16>(v[3]), s), code_of(h16_hi<F16>(v[3]), s));
    return r;
}

// Per-row constants of the code computation.
struct RowScale {
    float s;     // absmax / 127 (correctly rounded)
    float r;     // fl(1 / s)
    bool fast;   // s normal and 1/s finite: the reciprocal route applies
};
__device__ __forceinline__ RowScale row_scale(float absmax) {
    RowScale q;
    q.s = absmax / 127.0f;
    q.fast = q.s >= 0x1p-125f;
    q.r = q.fast ? 1.0f / q.s : 0.0f;
    return q;
}

// Codes without a division per element, bit-identical to codes8_div.
// With r = fl(1/s) = (1/s)(1 + e), |e| <= 2^-24: m = fl(x*r + 1.5*2^23) (one
// fused rounding) holds n = rint(x*r) in its low bits (ulp 1 in [2^23, 2^24);
// its low byte is the int8 code, two's complement), and d = fl(x*r - n)
// (fused again) is the distance of the exact product from that integer.
// x*r differs from x/s by |x/s| * |e| <= 127.0000076 * 2^-24 < 7.6e-6, fl(x/s)
// from x/s by at most half an ulp (< 3.9e-6 below 128), and d from x*r - n
// by at most 2^-25.  So when |d| <= 0.5 - 2^-16 the correctly rounded
// quotient fl(x/s) lies strictly within 0.5 of n and rounds to n.  Any other
// element (a near-tie, about one in 30000) is recomputed by division on its
// own.  |x*r| < 127.5 on the fast route, so no clamp is needed there.
template <bool F16 = false>
__device__ __forceinline__ v2u codes8(v4u v, const RowScale& q) {
    if (!q.fast) return codes8_div<F16>(v, q.s);
    constexpr float MAGIC = 12582912.0f;  // 1.5 * 2^23
    constexpr float TIE_LO = 0.5f - 0x1p-16f;
    u32 b[8];
    float d[8];
    float dmax = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float x = (e & 1) ? h16_hi<F16>(v[e >> 1]) : h16_lo<F16>(v[e >> 1]);
        const float m = __builtin_fmaf(x, q.r, MAGIC);
        d[e] = __builtin_fmaf(x, q.r, MAGIC - m);  // MAGIC - m = -n exactly
        dmax = __builtin_fmaxf(dmax, __builtin_fabsf(d[e]));
        b[e] = __float_as_uint(m);
    }
    v2u r;
    r[0] = __builtin_amdgcn_perm(b[1], b[0], 0x0c0c0400u) | (__builtin_amdgcn_perm(b[3], b[2], 0x0c0c0400u) << 16);
    r[1] = __builtin_amdgcn_perm(b[5], b[4], 0x0c0c0400u) | (__builtin_amdgcn_perm(b[7], b[6], 0x0c0c0400u) << 16);
    if (dmax > TIE_LO) {  // rare: redo only the near-tie elements by division
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            if (__builtin_fabsf(d[e]) > TIE_LO) {
                const float x = (e & 1) ? h16_hi<F16>(v[e >> 1]) : h16_lo<F16>(v[e >> 1]);
                const u32 sh = 8 * (e & 3);
                r[e >> 2] = (r[e >> 2] & ~(0xFFu << sh)) | ((u32)(code_of(x, q.s) & 0xFF) << sh);
            }
        }
    }
    return r;
}

// Per-token-per-group activations: one scale per (row, 128-wide K block),
// every block quantized like a row of 128 values.  One wave per 512-value
// span of a row: lane l holds chunk l (8 values), lanes 16g .. 16g+15 form
// block g of the span (one DPP row), whose absmax takes four row rotations.
// K % 128 == 0; 16-byte aligned x rows, 8-byte aligned xq rows; s [M, K/128]
// dense.
template <bool F16 = false>
__global__ __launch_bounds__(256) void quant_per_group128_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, int8_t* __restrict__ xq, int64_t ldxq,
    float* __restrict__ s, int M, int K) {
    const int lane = threadIdx.x & 63;
    const int spans = (K + 511) >> 9;
    const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int m = wave / spans, sp = wave - m * spans;
    if (m >= M) return;
    const int c = sp * 64 + lane;  // chunk of 8 values in the row
    const bool ok = c < (K >> 3);
    v4u v = v4u{};
    if (ok) v = reinterpret_cast<const v4u*>(x + (int64_t)m * ldx)[c];
    const float a = row16_max(mag_to_f32<F16>(mag_max8(v2h{0, 0}, v)));
    const RowScale q = row_scale(a);
    if (!ok) return;
    reinterpret_cast<v2u*>(xq + (int64_t)m * ldxq)[c] = codes8<F16>(v, q);
    if ((lane & 15) == 0) s[(int64_t)m * (K >> 7) + (c >> 4)] = q.s;
}

// One wave per row; the row stays in registers (NC 16-byte chunks per lane,
// K <= NC * 512).  Needs K % 8 == 0, 16-byte aligned x rows and 8-byte
// aligned xq rows.  4 rows per 256-thread workgroup.
template <int NC, bool F16 = false>
__global__ __launch_bounds__(256) void quant_per_token_reg(
    const uint16_t* __restrict__ x, int64_t ldx, int8_t* __restrict__ xq, int64_t ldxq,
    float* __restrict__ s_tok, int M, int K) {
    const int lane = threadIdx.x & 63;
    const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (m >= M) return;
    const v4u* xr = reinterpret_cast<const v4u*>(x + (int64_t)m * ldx);
    const int nch = K >> 3;
    v4u v[NC];
    v2h mx = v2h{0, 0};
#pragma unroll
    for (int i = 0; i < NC; ++i) {
        // Chunks past the row end load the row's last chunk again: its
        // values are in the row, so the absmax is unchanged, and the loop
        // has no branch (a conditional load made the compiler copy the
        // whole register array at every step in the fp16 instances: 246
        // registers instead of 59 at NC = 8).
        const int c = min(lane + 64 * i, nch - 1);
        // Streaming (non-temporal) load: the row is read once.  With X in
        // HBM (as after a large GEMM) this quantizer takes 33 us instead
        // of 43 at 8192 x 5120; with X still in the last-level cache it
        // takes 31 instead of 27, since these loads do not keep it there.
        v[i] = __builtin_nontemporal_load(&xr[c]);
        mx = mag_max8(mx, v[i]);
    }
    const float a = wave_max(mag_to_f32<F16>(mx));
    const RowScale q = row_scale(a);
    if (lane == 0) s_tok[m] = q.s;
    v2u* qr = reinterpret_cast<v2u*>(xq + (int64_t)m * ldxq);
#pragma unroll
    for (int i = 0; i < NC; ++i) {
        const int c = lane + 64 * i;
        if (c < nch) qr[c] = codes8<F16>(v[i], q);
    }
}

// One workgroup (NT threads) per row, CPT 16-byte chunks per thread held in
// registers (K <= 8 * NT * CPT): for few rows, where spreading each row over
// a whole workgroup is what shortens the call.
template <int NT, int CPT, bool F16 = false>
__global__ __launch_bounds__(NT) void quant_per_token_wg(
    const uint16_t* __restrict__ x, int64_t ldx, int8_t* __restrict__ xq, int64_t ldxq,
    float* __restrict__ s_tok, int K) {
    __shared__ float red[NT / 64];
    const int m = blockIdx.x;
    const v4u* xr = reinterpret_cast<const v4u*>(x + (int64_t)m * ldx);
    const int nch = K >> 3;
    v4u v[CPT];
    v2h mx = v2h{0, 0};
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        const int c = threadIdx.x + NT * i;
        if (c < nch) {
            v[i] = xr[c];
            mx = mag_max8(mx, v[i]);
        }
    }
    float a = wave_max(mag_to_f32<F16>(mx));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = a;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) a = __builtin_fmaxf(a, red[w]);
    const RowScale q = row_scale(a);
    if (threadIdx.x == 0) s_tok[m] = q.s;
    v2u* qr = reinterpret_cast<v2u*>(xq + (int64_t)m * ldxq);
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        const int c = threadIdx.x + NT * i;
        if (c < nch) qr[c] = codes8<F16>(v[i], q);
    }
}

// Any K, any alignment: one wave per row, two passes over the row.
template <bool F16 = false>
__global__ __launch_bounds__(256) void quant_per_token_any(
    const uint16_t* __restrict__ x, int64_t ldx, int8_t* __restrict__ xq, int64_t ldxq,
    float* __restrict__ s_tok, int M, int K) {
    const int lane = threadIdx.x & 63;
    const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (m >= M) return;
    const uint16_t* xr = x + (int64_t)m * ldx;
    float a = 0.0f;
    for (int k = lane; k < K; k += 64) a = __builtin_fmaxf(a, __builtin_fabsf(h16_to_f32<F16>(xr[k])));
    a = wave_max(a);
    const float s = a / 127.0f;
    if (lane == 0) s_tok[m] = s;
    int8_t* qr = xq + (int64_t)m * ldxq;
    for (int k = lane; k < K; k += 64) qr[k] = (int8_t)code_of(h16_to_f32<F16>(xr[k]), s);
}

// Offline weight quantization: one workgroup per (row, span of G columns).
__global__ __launch_bounds__(256) void quant_weight_span(
    const float* __restrict__ w, int64_t ldw, int8_t* __restrict__ wq, int64_t ldwq,
    float* __restrict__ scale, int G, int spans_per_row) {
    __shared__ float red[4];
    const int row = blockIdx.x / spans_per_row;
    const int g = blockIdx.x % spans_per_row;
    const float* src = w + (int64_t)row * ldw + (int64_t)g * G;
    int8_t* dst = wq + (int64_t)row * ldwq + (int64_t)g * G;
    float a = 0.0f;
    for (int k = threadIdx.x; k < G; k += 256) a = __builtin_fmaxf(a, __builtin_fabsf(src[k]));
    a = wave_max(a);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = a;
    __syncthreads();
    a = __builtin_fmaxf(__builtin_fmaxf(red[0], red[1]), __builtin_fmaxf(red[2], red[3]));
    const float s = a / 127.0f;
    if (threadIdx.x == 0) scale[blockIdx.x] = s;
    for (int k = threadIdx.x; k < G; k += 256) dst[k] = (int8_t)code_of(src[k], s);
}

// ---- smoothing fold ("...W8A8 INT8 (v3)", "Recipe": SmoothQuant folds with
// scales capped at 16; "Qwen3.8-27B -- FP8 block + AWQ", "Recipe": the fold
// is function-preserving) ------------------------------------------------

__global__ void fill_u32(u32* __restrict__ p, u32 v, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

// Column maximum of |x| over ROWS rows per workgroup, merged with an integer
// atomic max on the fp32 bit pattern (order-free for non-negative floats, so
// the result is exact and deterministic).
__global__ __launch_bounds__(256) void colmax_bf16(const uint16_t* __restrict__ x, int64_t ldx,
                                                   u32* __restrict__ cmax, int M, int K,
                                                   int rows) {
    const int j = blockIdx.x * 256 + threadIdx.x;
    if (j >= K) return;
    const int m0 = blockIdx.y * rows;
    const int m1 = min(M, m0 + rows);
    float a = 0.0f;
    for (int m = m0; m < m1; ++m) a = __builtin_fmaxf(a, __builtin_fabsf(bf16_to_f32(x[(int64_t)m * ldx + j])));
    atomicMax(cmax + j, __float_as_uint(a));
}

__global__ void smooth_finalize(float* __restrict__ s, float cap, int K) {
    const int j = blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= K) return;
    const float r = __builtin_sqrtf(s[j]);  // correctly rounded (no fast-math)
    s[j] = r > cap ? cap : r;
}

// x and xo may alias (in-place fold): each element is read, then written, by
// the same thread.
__global__ __launch_bounds__(256) void fold_x_bf16(const uint16_t* x, int64_t ldx,
                                                   const float* __restrict__ s,
                                                   uint16_t* xo, int64_t ldxo, int M,
                                                   int K) {
    const int j = blockIdx.x * 256 + threadIdx.x;
    if (j >= K) return;
    const float sj = s[j];
    for (int m = blockIdx.y; m < M; m += gridDim.y)
        xo[(int64_t)m * ldxo + j] = f32_to_bf16(bf16_to_f32(x[(int64_t)m * ldx + j]) / sj);
}

__global__ __launch_bounds__(256) void fold_w_f32(const float* w, int64_t ldw,
                                                  const float* __restrict__ s,
                                                  float* wo, int64_t ldwo, int N,
                                                  int K) {
    const int j = blockIdx.x * 256 + threadIdx.x;
    if (j >= K) return;
    const float sj = s[j];
    for (int n = blockIdx.y; n < N; n += gridDim.y)
        wo[(int64_t)n * ldwo + j] = w[(int64_t)n * ldw + j] * sj;
}

}  // namespace q8
