// small_fused.hpp -- the whole W8A8 layer in one kernel for small layers: up
// to 16 tokens and a weight matrix of a few MB at most (K <= 1024), where the
// two-kernel route (row quantizer, then a GEMM) pays two launches for a few
// microseconds of work.
//
// Same arithmetic as q8_quant_scaled_mm ("Qwen3.8-27B -- SmoothQuant +
// activation-aware GPTQ, W8A8 INT8 (v3)", section "Recipe": per-token
// dynamic INT8 activations, per-channel INT8 weights, bf16 out):
// s_tok[m] = fl32(absmax_m / 127), codes clamp(rne(x / s_tok), -127, 127)
// (quant.hpp), acc = exact int32 sum, y = bf16_rne(((float)acc * s_tok[m]) *
// s_ch[n]) (fp16 with F16).
//
// Workgroup b (16 waves) owns channels 64 b .. 64 b + 63:
//  * waves 0..3 first issue the loads of their 16 channels' weight fragments
//    (wave w: channels 64 b + 16 w ..) straight into registers (the A
//    operand of v_mfma_i32_16x16x64_i8: lane (r, kg) holds bytes
//    64 j + 16 kg .. + 15 of row r for every 64-deep K block j), through a
//    buffer resource over the weight matrix, so rows past N read as zero;
//  * wave w quantizes token row w (if below M) into a code tile in LDS,
//    [16][K] with 16-byte unit u of row r at u ^ (r & mask) so the fragment
//    reads are free of bank conflicts, and its scale; workgroup 0 also
//    writes the codes and scales out (one row per wave: four rows a wave in
//    turn cost 1.2 us more per call at 16 tokens);
//  * after one barrier waves 0..3 run K / 64 MFMAs over their 16 channels
//    and the 16 token columns (rows of the tile past M hold whatever the LDS
//    held: their products land in output columns that are never stored),
//    then apply the epilogue to their lanes' tokens below M.
#pragma once

#include "gemm_i8.hpp"
#include "quant.hpp"

namespace q8 {

constexpr int SMALL_MAX_M = 16;
constexpr int SMALL_MAX_K = 1024;

struct SmallArgs {
    const uint16_t* x;  // [M, ldx] bf16 (fp16) activations
    int64_t ldx;
    const int8_t* w;  // [N, ldw] int8 weight codes
    int64_t ldw;
    const float* s_ch;  // [N]
    uint16_t* c;        // [M, ldc] bf16 (fp16) out
    int64_t ldc;
    int8_t* xq;    // [M, K] codes out (dense), written by workgroup 0
    float* s_tok;  // [M] scales out, written by workgroup 0
    int M, N, K;
};

// KB = K / 64 (2..16): 64-deep K blocks.  16 waves: wave w quantizes token
// row w; waves 0..3 also load and multiply the workgroup's 64 channels.
template <int KB, bool F16>
__global__ __launch_bounds__(1024) void small_fused_kernel(SmallArgs p) {
    constexpr int K = KB * 64;
    constexpr int U = K / 16;                   // 16-byte units per code row
    constexpr int MASK = U % 16 == 0 ? 15 : 7;  // swizzle mask: u ^ MASK stays below U (U % 8 == 0)
    constexpr int NCH = K / 8;                  // 8-value chunks per activation row
    constexpr int CPL = (NCH + 63) / 64;        // chunks per lane
    __shared__ __attribute__((aligned(16))) int8_t ct[SMALL_MAX_M * K];
    __shared__ float ts[SMALL_MAX_M];

    const int M = p.M;
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int tok = lane & 15, kg = lane >> 4;
    const bool mul = wid < 4;                   // a multiplying wave
    const int n0 = blockIdx.x * 64 + 16 * (wid & 3);  // its first channel

    // ---- weight fragments of rows n0 + tok (zero past N)
    v4i a[KB];
    if (mul) {
        const __amdgpu_buffer_rsrc_t wr = make_rsrc(p.w, operand_extent(p.N, p.ldw, K));
#pragma unroll
        for (int j = 0; j < KB; ++j)
            a[j] = __builtin_bit_cast(
                v4i, __builtin_amdgcn_raw_buffer_load_b128(wr, (n0 + tok) * (int)p.ldw + 64 * j + 16 * kg, 0, 0));
    }
    // epilogue operands: channels n0 + 4 kg + e
    const int ch = n0 + 4 * kg;
    const bool writer = mul && tok < M && ch < p.N;
    v4f sc = v4f{};
    if (writer) {
#pragma unroll
        for (int e = 0; e < 4; ++e) sc[e] = p.s_ch[ch + e];  // 4-byte aligned scales
    }

    // ---- token row m = wid into the code tile
    const int m = wid;
    if (m < M) {
        const v4u* xr = reinterpret_cast<const v4u*>(p.x + (int64_t)m * p.ldx);
        v4u v[CPL];
        v2h mx = v2h{0, 0};
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            v[i] = xr[min(lane + 64 * i, NCH - 1)];  // past the row end: its last chunk again
            mx = mag_max8(mx, v[i]);
        }
        const RowScale q = row_scale(wave_max(mag_to_f32<F16>(mx)));
        if (lane == 0) {
            ts[m] = q.s;
            if (blockIdx.x == 0) p.s_tok[m] = q.s;
        }
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int c = lane + 64 * i;  // 8-code piece c: unit c / 2, half c % 2
            if (c < NCH) {
                const v2u cd = codes8<F16>(v[i], q);
                *reinterpret_cast<v2u*>(ct + m * K + (((c >> 1) ^ (m & MASK)) << 4) + ((c & 1) << 3)) = cd;
                if (blockIdx.x == 0) *reinterpret_cast<v2u*>(p.xq + (int64_t)m * K + 8 * c) = cd;
            }
        }
    }
    __syncthreads();
    if (!mul) return;

    // ---- 16 channels x 16 tokens over K
    v4i acc = v4i{};
    const int8_t* bp = ct + tok * K;
#pragma unroll
    for (int j = 0; j < KB; ++j) {
        const int u = 4 * j + kg;
        const v4i b = *reinterpret_cast<const v4i*>(bp + ((u ^ (tok & MASK)) << 4));
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[j], b, acc, 0, 0, 0);
    }
    if (!writer) return;
    const float st = ts[tok];
    float y[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float t = (float)acc[e] * st;
        y[e] = t * sc[e];
    }
    v2u o;
    o[0] = pack16x2<F16>(y[0], y[1]);
    o[1] = pack16x2<F16>(y[2], y[3]);
    *reinterpret_cast<v2u*>(p.c + (int64_t)tok * p.ldc + ch) = o;
}

template <bool F16>
inline hipError_t launch_small(const SmallArgs& p, hipStream_t stream) {
    const dim3 grid((p.N + 63) / 64), block(1024);
    switch (p.K / 64) {
#define Q8_S(kb) case kb: hipLaunchKernelGGL((small_fused_kernel<kb, F16>), grid, block, 0, stream, p); break;
        Q8_S(2) Q8_S(4) Q8_S(6) Q8_S(8) Q8_S(10) Q8_S(12) Q8_S(14) Q8_S(16)
#undef Q8_S
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// Where the one-call layer takes this kernel (the fused decode kernel,
// when it applies, comes first): K a multiple of 128 up to 1024 (1024 only
// up to 8 tokens), at most 16 MB of weights, and the weight operand within
// 32-bit buffer offsets.  Per call in a graph on rotating weight copies,
// against the row quantizer + GEMM it replaces (N x K from 128 x 256 to
// 16384 x 896, 1-16 tokens): 2.6-6.9 against 5.1-9.8 us, every shape
// measured; the tiny workload (16 x 256 -> 128) 3.75 against 5.47 us.  At
// K = 1024 and 12-16 tokens the repeated quantization (every workgroup
// quantizes all M rows) made it 3-5% slower at N = 4096.
inline bool small_fits(int M, int N, int K, int64_t ldw) {
    if (M < 1 || M > SMALL_MAX_M || K % 128 != 0 || K > SMALL_MAX_K) return false;
    if (K == SMALL_MAX_K && M > 8) return false;
    if ((int64_t)N * K > ((int64_t)16 << 20)) return false;
    return (int64_t)(N + 64) * ldw < ((int64_t)1 << 31);  // rows up to the last workgroup's end
}

}  // namespace q8
