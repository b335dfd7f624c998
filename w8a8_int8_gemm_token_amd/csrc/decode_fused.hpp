// decode_fused.hpp -- the whole W8A8 layer for decode-sized batches in one
// kernel: per-token quantization of X (M <= 8 rows) and the INT8 GEMM with
// the per-token x per-channel epilogue.
//
// Decode streams the whole weight matrix once per call and is bound by HBM
// bandwidth ("Qwen3.8-27B-INT8-W8A8", section "Throughput": decode is
// weight-bandwidth-bound); per-token dynamic INT8 activations with per-channel
// INT8 weights ("Qwen3.8-27B -- SmoothQuant + activation-aware GPTQ, W8A8
// INT8 (v3)", section "Recipe").  One workgroup of 16 waves per CU:
//  * workgroup b owns R consecutive output channels (R a multiple of 4, at
//    most 32): for N up to 256 * 32 the grid is ~256 workgroups, one per
//    CU, which streams the matrix at the rate of a plain coalesced read (a
//    grid that is not a whole number of workgroups per CU leaves a
//    straggler tail); larger N runs in whole waves of 256 (decode_rows);
//  * waves 0..7 quantize: wave m loads token row m (1 KB per instruction),
//    takes its absmax with a wave reduction and writes the exact codes of
//    quant.hpp into an M x K code tile in LDS.  Every workgroup does this for
//    itself: redundant VALU work that runs while the weights stream, and no
//    communication between workgroups;
//  * waves 8..15 move the workgroup's R x K weight tile to LDS with
//    buffer_load_dwordx4 ... lds (1 KB of one row per instruction, each wave
//    a contiguous eighth of the tile).  A CU
//    accepts only so many loads at a time, so a wave issuing the tile stalls
//    at issue until earlier loads drain; keeping the quantizing waves free of
//    weight loads is what lets the two overlap.  The quantizing waves run at
//    a raised wave priority so that their activation loads are issued ahead
//    of the weight stream;
//  * after one barrier, wave w multiplies its K range of both 16-row tiles
//    with v_mfma_i32_16x16x64_i8 (channels = A operand, tokens = B); rows and
//    tokens past the ends repeat the last valid one (broadcast LDS reads, and
//    their outputs are never stored), so the phase has no branches and its
//    LDS reads can be issued ahead of the MFMAs.  The 16 partial int32 tiles
//    are summed in LDS (exact), and waves 0..1 apply
//    y = bf16_rne(((float)acc * s_tok[m]) * s_ch[n]).
// LDS layout (both tiles row-major with row stride K): 16-byte unit u of row
// r is stored at unit u ^ (r & 15), so the fragment reads (16 rows, one unit
// each) are free of bank conflicts.  Workgroup 0 also writes the codes and
// the token scales to the caller's buffers.
#pragma once

#include "gemm_i8.hpp"
#include "quant.hpp"

namespace q8 {

constexpr int DECODE_MAX_M = 8;
constexpr int DECODE_MAX_ROWS = 32;
constexpr int DECODE_LDS_BYTES = 160 * 1024;

struct DecodeArgs {
    const uint16_t* x;  // [M, ldx] bf16 (fp16) activations
    int64_t ldx;
    const int8_t* w;  // [N, ldw] int8 weight codes
    int64_t ldw;
    const float* s_ch;  // [N]
    uint16_t* c;        // [M, ldc] bf16 out
    int64_t ldc;
    int8_t* xq;     // [M, K] codes out (dense), written by workgroup 0
    float* s_tok;   // [M] scales out, written by workgroup 0
    int M, N, K;
    int rows;       // R: channels per workgroup (multiple of 4)
};


// LDS: weight tile (or, after the MFMA phase, the 16 waves' partial tiles),
// code tile [8][K], token scales.
__host__ __device__ inline size_t decode_wt_bytes(int K, int rows) {
    const size_t red = (size_t)2 * 16 * 64 * 16;
    const size_t wt = (size_t)rows * K;
    return wt > red ? wt : red;
}
__host__ __device__ inline size_t decode_lds_bytes(int K, int rows) {
    return decode_wt_bytes(K, rows) + (size_t)DECODE_MAX_M * K + 256;
}

// LDS accesses done; vector memory loads may stay in flight.
__device__ __forceinline__ void wait_lgkm0() {
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));  // vmcnt 63, expcnt 7, lgkmcnt 0
}

// NC = K / 1024.  F16: fp16 activations and outputs instead of bf16.
template <int NC, bool F16>
__global__ __launch_bounds__(1024) void decode_fused_kernel(DecodeArgs p) {
    constexpr int K = NC * 1024;
    constexpr int NQ = 2 * NC;  // 16-byte activation chunks per lane (one row per wave)
    constexpr int KBW = NC;     // 64-deep K blocks per wave in the MFMA phase
    extern __shared__ __attribute__((aligned(1024))) int8_t lds[];

    const int M = p.M;
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int R = p.rows;
    const int n0 = blockIdx.x * R;
    const int rows = min(R, p.N - n0);
    int8_t* wt = lds;                                         // [R][K] weight tile
    int8_t* ct = lds + decode_wt_bytes(K, R);                 // [8][K] code tile
    float* row_scale_s = reinterpret_cast<float*>(ct + DECODE_MAX_M * K);  // [8] token scales

    // ---- epilogue operands of the output waves (wave t < 2, lane l: token
    // l % 16, channels n0 + 16t + 4(l / 16) + e), fetched first
    const int tok = lane & 15, kg = lane >> 4;
    const int ch = n0 + 16 * wid + 4 * kg;
    const bool writer = wid < 2 && tok < M && 16 * wid + 4 * kg < rows;
    v4f sc = v4f{};
    if (writer) {
#pragma unroll
        for (int e = 0; e < 4; ++e) sc[e] = p.s_ch[ch + e];
    }

    if (wid < 8) {
        // ---- quantizing wave: token row m = wid; chunk c = lane + 64 i
        __builtin_amdgcn_s_setprio(3);
        const int m = wid;
        const bool has_row = m < M;
        v4u v[NQ];
        if (has_row) {
            const v4u* xr = reinterpret_cast<const v4u*>(p.x + (int64_t)m * p.ldx);
#pragma unroll
            for (int i = 0; i < NQ; ++i) v[i] = xr[lane + 64 * i];
        }
        if (has_row) {
            v2h mx = v2h{0, 0};
#pragma unroll
            for (int i = 0; i < NQ; ++i) mx = mag_max8(mx, v[i]);
            const RowScale q = row_scale(wave_max(mag_to_f32<F16>(mx)));
            if (lane == 0) {
                row_scale_s[m] = q.s;
                if (blockIdx.x == 0) p.s_tok[m] = q.s;
            }
#pragma unroll
            for (int i = 0; i < NQ; ++i) {
                const v2u cd = codes8<F16>(v[i], q);
                const int c8 = lane + 64 * i;  // 8-byte code piece
                const int uu = c8 >> 1;
                *reinterpret_cast<v2u*>(ct + m * K + ((uu ^ m) << 4) + ((c8 & 1) << 3)) = cd;
                if (blockIdx.x == 0) *reinterpret_cast<v2u*>(p.xq + (int64_t)m * K + 8 * c8) = cd;
            }
        }
        wait_lgkm0();  // code tile written (the global stores may stay in flight)
        __builtin_amdgcn_s_setprio(0);
    } else {
        // ---- loading wave d: 1 KB blocks [d * per, (d + 1) * per) of the
        // row-major tile (a contiguous run of the weight matrix); lane l
        // moves global unit l ^ (r & 15) of a block of row r to LDS unit l
        const int d = wid - 8;
        const __amdgpu_buffer_rsrc_t wr = make_rsrc(p.w + (int64_t)n0 * p.ldw,
                                                    (uint32_t)((int64_t)rows * p.ldw));
        const int nblk = rows * NC;
        const int per = (nblk + 7) / 8;
        const int b1 = min(nblk, (d + 1) * per);
        for (int i = d * per; i < b1; ++i) {
            const int r = i / NC, u = i - r * NC;
            const int voff = r * (int)p.ldw + u * 1024 + ((lane ^ (r & 15)) << 4);
            // cache policy 2 = non-temporal: every weight byte is read once
            // per call (measured 0.4-0.6 us faster per call at N = K = 5120)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (Q8_LDS void*)(wt + r * K + u * 1024), 16,
                                                     voff, 0, 0, 2);
        }
        wait_vm_lgkm0<0>();  // this wave's part of the tile landed
    }
    block_barrier();  // weight tile and code tile complete

    // ---- MFMA: wave wid takes K blocks [wid * KBW, +KBW) of both tiles
    const int tc = min(tok, M - 1);          // token row of the B fragment
    const int r0 = min(tok, rows - 1);       // weight rows of the A fragments
    const int r1 = min(16 + tok, rows - 1);
    const int8_t* bp = ct + tc * K;
    const int8_t* a0p = wt + r0 * K;
    const int8_t* a1p = wt + r1 * K;
    v4i acc0 = v4i{}, acc1 = v4i{};
#pragma unroll
    for (int j = 0; j < KBW; ++j) {
        const int u = 4 * (wid * KBW + j) + kg;  // 16-byte unit of K
        const v4i b = *reinterpret_cast<const v4i*>(bp + ((u ^ tc) << 4));
        const v4i a0 = *reinterpret_cast<const v4i*>(a0p + ((u ^ (r0 & 15)) << 4));
        const v4i a1 = *reinterpret_cast<const v4i*>(a1p + ((u ^ (r1 & 15)) << 4));
        acc0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, b, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, b, acc1, 0, 0, 0);
    }

    // ---- sum the 16 waves' partial tiles (exact int32), epilogue
    block_barrier();  // every wave is done reading the weight tile
    v4i* red = reinterpret_cast<v4i*>(lds);
    red[wid * 64 + lane] = acc0;
    red[(16 + wid) * 64 + lane] = acc1;
    wait_lgkm0();
    block_barrier();
    if (!writer) return;
    v4i s = v4i{};
#pragma unroll
    for (int w = 0; w < 16; ++w) s += red[(wid * 16 + w) * 64 + lane];
    const float st = row_scale_s[tok];
    float y[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float u = (float)s[e] * st;
        y[e] = u * sc[e];
    }
    v2u o;
    o[0] = pack16x2<F16>(y[0], y[1]);
    o[1] = pack16x2<F16>(y[2], y[3]);
    *reinterpret_cast<v2u*>(p.c + (int64_t)tok * p.ldc + ch) = o;
}

template <int NC, bool F16>
inline hipError_t launch_decode_t(const DecodeArgs& p, hipStream_t stream) {
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&decode_fused_kernel<NC, F16>),
        hipFuncAttributeMaxDynamicSharedMemorySize, DECODE_LDS_BYTES);
    if (attr != hipSuccess) return attr;
    const int grid = (p.N + p.rows - 1) / p.rows;
    hipLaunchKernelGGL((decode_fused_kernel<NC, F16>), dim3(grid), dim3(1024),
                       decode_lds_bytes(p.K, p.rows), stream, p);
    return hipGetLastError();
}

template <bool F16>
inline hipError_t launch_decode(const DecodeArgs& p, hipStream_t stream) {
    switch (p.K / 1024) {
        case 1: return launch_decode_t<1, F16>(p, stream);
        case 2: return launch_decode_t<2, F16>(p, stream);
        case 3: return launch_decode_t<3, F16>(p, stream);
        case 4: return launch_decode_t<4, F16>(p, stream);
        case 5: return launch_decode_t<5, F16>(p, stream);
        case 6: return launch_decode_t<6, F16>(p, stream);
        case 7: return launch_decode_t<7, F16>(p, stream);
        case 8: return launch_decode_t<8, F16>(p, stream);
    }
    return hipErrorInvalidValue;
}

// M <= 8 tokens, K a multiple of 1024 up to 8192, ~N/256 channels per
// workgroup (at most 32) whose tile and the code tile fit in LDS, and 32-bit
// buffer offsets.
// Channels per workgroup (a multiple of 4), or 0 if no size fits LDS.  Up
// to 256 * 32 channels, one workgroup per CU: R = N / 256 rounded up.
// Beyond that the CUs take several workgroups in turn, and R (at least 16,
// so the per-workgroup quantization stays small next to its weight stream)
// minimizes the channels the busiest CU streams: ceil(ceil(N/R) / 256) * R.
inline int decode_rows(int N, int K) {
    int rmax = DECODE_MAX_ROWS;
    while (rmax >= 4 && decode_lds_bytes(K, rmax) > (size_t)DECODE_LDS_BYTES) rmax -= 4;
    if (rmax < 4) return 0;
    const int r1 = (((N + 255) / 256) + 3) & ~3;
    if (r1 <= rmax) return r1;
    int best = 0;
    int64_t cost = INT64_MAX;
    for (int r = rmax; r >= 16 && r >= 4; r -= 4) {
        const int64_t c = (int64_t)((((int64_t)N + r - 1) / r + 255) / 256) * r;
        if (c < cost) cost = c, best = r;
    }
    return best;
}

inline bool decode_fits(int M, int N, int K, int64_t ldw) {
    if (M < 1 || M > DECODE_MAX_M || K % 1024 != 0 || K > 8192) return false;
    const int R = decode_rows(N, K);
    if (R < 4) return false;
    return (int64_t)R * ldw < ((int64_t)1 << 31);
}

}  // namespace q8
