// decode_fused.hpp -- the whole W8A8 layer for decode-sized batches in one
// kernel: per-token quantization of X (M <= 8 rows, K a multiple of 128 up
// to 8192) and the INT8 GEMM with the per-token x per-channel epilogue.
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
//    buffer_load_dwordx4 ... lds (1 KB of one row per instruction; wave d
//    rows d, d + 8, ...), all of it issued at once, K segment (1024) by K
//    segment; as each segment of its rows lands (vmcnt) a wave increments
//    that segment's LDS counter.  A CU accepts only so many loads at a
//    time, so a wave issuing the tile stalls at issue until earlier loads
//    drain; keeping the quantizing waves free of weight loads is what lets
//    the two overlap.  The quantizing waves run at a raised wave priority
//    so that their activation loads are issued ahead of the weight stream;
//  * once the code tile is complete, waves 0..7 multiply segment by segment
//    as the segments land (wave w: K blocks 16 s + 2w and 16 s + 2w + 1 of
//    segment s), both 16-row tiles with v_mfma_i32_16x16x64_i8 (channels =
//    A operand, tokens = B), so that only the last segment's products
//    remain when the weight stream ends; rows and tokens past the ends
//    repeat the last valid one (broadcast LDS reads, and their outputs are
//    never stored).  The 8 partial int32 tiles are summed in LDS (exact),
//    and waves 0..1 apply y = bf16_rne(((float)acc * s_tok[m]) * s_ch[n]).
//    The waits on the counters are bounded (lds_sync.hpp).
// LDS layout (both tiles row-major with row stride K): 16-byte unit u of row
// r is stored at unit u ^ (r & 15), so the fragment reads (16 rows, one unit
// each) are free of bank conflicts.  Workgroup 0 also writes the token
// scales to the caller's buffer; the codes go out in 1 KB pieces spread over
// the first workgroups.
// decode_pre_kernel (below) runs the same weight stream and per-segment
// multiply on activations that are already int8 codes, up to 16 tokens.
#pragma once

#include "gemm_i8.hpp"
#include "lds_sync.hpp"
#include "quant.hpp"

namespace q8 {

constexpr int DECODE_MAX_M = 8;
constexpr int DECODE_MAX_ROWS = 32;
// dynamic LDS limit: 160 KB less the kernel's static counters, the dynamic
// array starting at the next 1024-byte boundary
constexpr int DECODE_LDS_BYTES = 160 * 1024 - 1024;

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
// codes: the fused kernel's 8 x K code tile and token scales (none for the
// pre-quantized kernel)
__host__ __device__ inline size_t decode_lds_bytes(int K, int rows, bool codes = true) {
    return decode_wt_bytes(K, rows) + (codes ? (size_t)DECODE_MAX_M * K + 256 : 0);
}

// LDS accesses done; vector memory loads may stay in flight.
__device__ __forceinline__ void wait_lgkm0() {
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));  // vmcnt 63, expcnt 7, lgkmcnt 0
}

// Loading wave d (0..7) of a decode workgroup: rows d, d + 8, ... of the
// workgroup's weight tile (rows x K, row stride KP = 1024 NC in LDS),
// segment by segment, 1 KB of one row per instruction (lane l moves global
// unit l ^ (r & 15) of the row's block to LDS unit l; a unit past K gets an
// offset beyond the buffer resource and lands as zeros); once its rows of
// segment s landed (vmcnt) the wave increments ready[s].
template <int NC, bool PK>
__device__ __forceinline__ void decode_load_tile(const int8_t* w, int64_t ldw, int rows, int K, int8_t* wt,
                                                 int* ready, int d, int lane, uint64_t t_start) {
    constexpr int KP = NC * 1024;
    if constexpr (!PK) K = KP;  // whole segments: no unit is past K
    const int cnt = rows > d ? (rows - d + 7) / 8 : 0;
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(w, (uint32_t)((int64_t)rows * ldw));
#pragma unroll
    for (int sg = 0; sg < NC; ++sg) {
        for (int j = 0; j < cnt; ++j) {
            const int r = d + 8 * j;
            const int ku = sg * 1024 + ((lane ^ (r & 15)) << 4);  // K byte of this lane's unit
            // past K: offset 2^31, beyond any resource here (decode_fits keeps
            // rows * ldw below 2^31), which reads as zero
            const int voff = !PK || ku < K ? r * (int)ldw + ku : INT32_MIN;
            // cache policy 2 = non-temporal: every weight byte is read once
            // per call (measured 0.4-0.6 us faster per call at N = K = 5120)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (Q8_LDS void*)(wt + r * KP + sg * 1024), 16, voff, 0, 0,
                                                     2);
        }
    }
#pragma unroll
    for (int sg = 0; sg < NC; ++sg) {
        sg_wait_vm((NC - 1 - sg) * cnt);  // segments 0..sg landed
        if (lane == 0) sg_signal(&ready[sg]);
    }
    if (__builtin_amdgcn_s_memrealtime() - t_start > SG_WAVE_LIMIT_TICKS && lane == 0)
        atomicAdd(&sg_wait_timeouts, 1u);
}

// Output lane of a decode workgroup (wave t < 2, lane l: token l % 16,
// channels n0 + 16 t + 4 (l / 16) + e): the sum of the 8 multiplying
// waves' partial tiles (exact int32), then y = ((float)acc * st) * sc[e].
template <bool F16>
__device__ __forceinline__ void decode_write(const v4i* red, int wid, int lane, float st, v4f sc, uint16_t* out) {
    v4i s = v4i{};
#pragma unroll
    for (int w = 0; w < 8; ++w) s += red[(wid * 8 + w) * 64 + lane];
    float y[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float u = (float)s[e] * st;
        y[e] = u * sc[e];
    }
    v2u o;
    o[0] = pack16x2<F16>(y[0], y[1]);
    o[1] = pack16x2<F16>(y[2], y[3]);
    *reinterpret_cast<v2u*>(out) = o;
}

// NC = ceil(K / 1024), K a multiple of 128.  PK: the last K segment is
// partial (its weights past K land as zeros, and whatever the code tile
// holds past K multiplies them); without it K = 1024 NC and the kernel
// carries none of the checks (they cost 0.25 us per call at 8 tokens,
// 5120 x 5120).  F16: fp16 activations and outputs instead of bf16.
template <int NC, bool PK, bool F16>
__global__ __launch_bounds__(1024) void decode_fused_kernel(DecodeArgs p) {
    constexpr int KP = NC * 1024;  // row stride of both LDS tiles
    constexpr int NQ = 2 * NC;     // 16-byte activation chunks per lane (one row per wave)
    const int K = PK ? p.K : KP;
    extern __shared__ __attribute__((aligned(1024))) int8_t lds[];
    __shared__ int ready[NC];  // loading waves whose rows of K segment s landed (8 = all)
    __shared__ int qdone;      // quantizing waves done (8 = the code tile is complete)

    const int M = p.M;
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int R = p.rows;
    const int n0 = blockIdx.x * R;
    const int rows = min(R, p.N - n0);
    int8_t* wt = lds;                                         // [R][KP] weight tile
    int8_t* ct = lds + decode_wt_bytes(KP, R);                // [8][KP] code tile
    float* row_scale_s = reinterpret_cast<float*>(ct + DECODE_MAX_M * KP);  // [8] token scales

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
    if (threadIdx.x < NC) ready[threadIdx.x] = 0;
    if (threadIdx.x == 0) qdone = 0;
    wait_lgkm0();
    block_barrier();
    const uint64_t t_start = __builtin_amdgcn_s_memrealtime();

    if (wid < 8) {
        // ---- quantizing wave: token row m = wid; chunk c = lane + 64 i
        __builtin_amdgcn_s_setprio(3);
        const int m = wid;
        const bool has_row = m < M;
        v4u v[NQ];
        if (has_row) {
            const v4u* xr = reinterpret_cast<const v4u*>(p.x + (int64_t)m * p.ldx);
            const int last = K / 8 - 1;  // past the row end: its last chunk again
#pragma unroll
            for (int i = 0; i < NQ; ++i) v[i] = xr[PK ? min(lane + 64 * i, last) : lane + 64 * i];
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
                *reinterpret_cast<v2u*>(ct + m * KP + ((uu ^ m) << 4) + ((c8 & 1) << 3)) = cd;
            }
        }
        wait_lgkm0();  // this wave's codes are in the tile
        __builtin_amdgcn_s_setprio(0);
        if (lane == 0) sg_signal(&qdone);

        // ---- multiplying: segment s (K 1024 s .. + 1023) once its rows
        // landed; this wave takes K blocks 16 s + 2 wid and + 1 of both
        // 16-row tiles
        sg_wait_ge(&qdone, 8);
        const int tc = min(tok, M - 1);     // token row of the B fragment
        const int r0 = min(tok, rows - 1);  // weight rows of the A fragments
        const int r1 = min(16 + tok, rows - 1);
        const int8_t* bp = ct + tc * KP;
        const int8_t* a0p = wt + r0 * KP;
        const int8_t* a1p = wt + r1 * KP;
        v4i acc0 = v4i{}, acc1 = v4i{};
#pragma unroll
        for (int sg = 0; sg < NC; ++sg) {
            sg_wait_ge(&ready[sg], 8);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int u = 4 * (16 * sg + 2 * wid + j) + kg;  // 16-byte unit of K
                const v4i b = *reinterpret_cast<const v4i*>(bp + ((u ^ tc) << 4));
                const v4i a0 = *reinterpret_cast<const v4i*>(a0p + ((u ^ (r0 & 15)) << 4));
                const v4i a1 = *reinterpret_cast<const v4i*>(a1p + ((u ^ (r1 & 15)) << 4));
                acc0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, b, acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, b, acc1, 0, 0, 0);
            }
        }
        v4i* red = reinterpret_cast<v4i*>(lds);
        if (__builtin_amdgcn_s_memrealtime() - t_start > SG_WAVE_LIMIT_TICKS && lane == 0)
            atomicAdd(&sg_wait_timeouts, 1u);
        block_barrier();  // every wave is done reading the weight tile
        red[wid * 64 + lane] = acc0;
        red[(8 + wid) * 64 + lane] = acc1;
    } else {
        decode_load_tile<NC, PK>(p.w + (int64_t)n0 * p.ldw, p.ldw, rows, K, wt, ready, wid - 8, lane, t_start);
        block_barrier();  // every wave is done reading the weight tile
    }

    // ---- sum the 8 multiplying waves' partial tiles (exact int32),
    // epilogue; the codes out
    wait_lgkm0();
    block_barrier();
    if (wid == 2) {
        // 1 KB piece q (token q / NC, K units 64 (q % NC) .. + 63) goes out
        // from workgroup q (mod the grid), so that no workgroup carries all
        for (int q = blockIdx.x; q < M * NC; q += gridDim.x) {
            const int m = q / NC, u = 64 * (q - m * NC) + lane;
            if (!PK || 16 * u < K)
                *reinterpret_cast<v4u*>(p.xq + (int64_t)m * K + 16 * u) =
                    *reinterpret_cast<const v4u*>(ct + m * KP + ((u ^ m) << 4));
        }
    }
    if (writer)
        decode_write<F16>(reinterpret_cast<const v4i*>(lds), wid, lane, row_scale_s[tok], sc,
                          p.c + (int64_t)tok * p.ldc + ch);
}

// The same weight stream and per-segment multiply for activations that are
// already quantized (q8_scaled_mm's int8 codes with their token scales, and
// the one-call layer from 9 tokens on, behind the row quantizer): up to 16
// tokens, which one 16-column B operand holds.  The multiplying waves load
// their B fragments straight from the codes in global memory -- all 2 NC
// of them, issued before the first wait -- so LDS holds only the weight
// tile (a 16 x K code tile would not fit beside it).  Waves 0..7 multiply,
// waves 8..15 load, as in decode_fused_kernel.
struct DecodePreArgs {
    const int8_t* a;  // [M, lda] int8 activation codes (lda % 16 == 0, 16-byte aligned)
    int64_t lda;
    const float* s_tok;  // [M]
    const int8_t* w;     // [N, ldw] int8 weight codes
    int64_t ldw;
    const float* s_ch;  // [N]
    uint16_t* c;        // [M, ldc] bf16 (fp16) out
    int64_t ldc;
    int M, N, K;
    int rows;  // R: channels per workgroup (multiple of 4)
};

template <int NC, bool F16>
__global__ __launch_bounds__(1024) void decode_pre_kernel(DecodePreArgs p) {
    extern __shared__ __attribute__((aligned(1024))) int8_t lds[];
    __shared__ int ready[NC];  // loading waves whose rows of K segment s landed (8 = all)

    const int M = p.M;
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int R = p.rows;
    const int n0 = blockIdx.x * R;
    const int rows = min(R, p.N - n0);
    int8_t* wt = lds;  // [R][K] weight tile

    const int tok = lane & 15, kg = lane >> 4;
    const int ch = n0 + 16 * wid + 4 * kg;
    const bool writer = wid < 2 && tok < M && 16 * wid + 4 * kg < rows;
    v4f sc = v4f{};
    float st = 0.0f;
    if (writer) {
#pragma unroll
        for (int e = 0; e < 4; ++e) sc[e] = p.s_ch[ch + e];
        st = p.s_tok[tok];
    }
    if (threadIdx.x < NC) ready[threadIdx.x] = 0;
    wait_lgkm0();
    block_barrier();
    const uint64_t t_start = __builtin_amdgcn_s_memrealtime();

    if (wid < 8) {
        // ---- multiplying wave: K blocks 16 s + 2 wid and + 1 of segment s,
        // both 16-row tiles; lane (tok, kg) holds 16 codes of token tc
        const int tc = min(tok, M - 1);     // token row of the B fragment
        const int r0 = min(tok, rows - 1);  // weight rows of the A fragments
        const int r1 = min(16 + tok, rows - 1);
        const int8_t* bp = p.a + (int64_t)tc * p.lda;
        v4i b[NC][2];
        __builtin_amdgcn_s_setprio(3);  // ahead of the weight stream
#pragma unroll
        for (int sg = 0; sg < NC; ++sg)
#pragma unroll
            for (int j = 0; j < 2; ++j)
                b[sg][j] = *reinterpret_cast<const v4i*>(bp + 16 * (4 * (16 * sg + 2 * wid + j) + kg));
        __builtin_amdgcn_s_setprio(0);
        const int8_t* a0p = wt + r0 * (NC * 1024);
        const int8_t* a1p = wt + r1 * (NC * 1024);
        v4i acc0 = v4i{}, acc1 = v4i{};
#pragma unroll
        for (int sg = 0; sg < NC; ++sg) {
            sg_wait_ge(&ready[sg], 8);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int u = 4 * (16 * sg + 2 * wid + j) + kg;  // 16-byte unit of K
                const v4i a0 = *reinterpret_cast<const v4i*>(a0p + ((u ^ (r0 & 15)) << 4));
                const v4i a1 = *reinterpret_cast<const v4i*>(a1p + ((u ^ (r1 & 15)) << 4));
                acc0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, b[sg][j], acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, b[sg][j], acc1, 0, 0, 0);
            }
        }
        v4i* red = reinterpret_cast<v4i*>(lds);
        if (__builtin_amdgcn_s_memrealtime() - t_start > SG_WAVE_LIMIT_TICKS && lane == 0)
            atomicAdd(&sg_wait_timeouts, 1u);
        block_barrier();  // every wave is done reading the weight tile
        red[wid * 64 + lane] = acc0;
        red[(8 + wid) * 64 + lane] = acc1;
    } else {
        decode_load_tile<NC, false>(p.w + (int64_t)n0 * p.ldw, p.ldw, rows, NC * 1024, wt, ready, wid - 8, lane,
                                    t_start);
        block_barrier();  // every wave is done reading the weight tile
    }

    wait_lgkm0();
    block_barrier();
    if (writer)
        decode_write<F16>(reinterpret_cast<const v4i*>(lds), wid, lane, st, sc, p.c + (int64_t)tok * p.ldc + ch);
}

template <int NC, bool PK, bool F16>
inline hipError_t launch_decode_t(const DecodeArgs& p, hipStream_t stream) {
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&decode_fused_kernel<NC, PK, F16>),
        hipFuncAttributeMaxDynamicSharedMemorySize, DECODE_LDS_BYTES);
    if (attr != hipSuccess) return attr;
    const int grid = (p.N + p.rows - 1) / p.rows;
    hipLaunchKernelGGL((decode_fused_kernel<NC, PK, F16>), dim3(grid), dim3(1024),
                       decode_lds_bytes(NC * 1024, p.rows), stream, p);
    return hipGetLastError();
}

template <int NC, bool F16>
inline hipError_t launch_decode_nc(const DecodeArgs& p, hipStream_t stream) {
    return p.K == NC * 1024 ? launch_decode_t<NC, false, F16>(p, stream) : launch_decode_t<NC, true, F16>(p, stream);
}

template <bool F16>
inline hipError_t launch_decode(const DecodeArgs& p, hipStream_t stream) {
    switch ((p.K + 1023) / 1024) {
        case 1: return launch_decode_nc<1, F16>(p, stream);
        case 2: return launch_decode_nc<2, F16>(p, stream);
        case 3: return launch_decode_nc<3, F16>(p, stream);
        case 4: return launch_decode_nc<4, F16>(p, stream);
        case 5: return launch_decode_nc<5, F16>(p, stream);
        case 6: return launch_decode_nc<6, F16>(p, stream);
        case 7: return launch_decode_nc<7, F16>(p, stream);
        case 8: return launch_decode_nc<8, F16>(p, stream);
    }
    return hipErrorInvalidValue;
}

template <int NC, bool F16>
inline hipError_t launch_decode_pre_t(const DecodePreArgs& p, hipStream_t stream) {
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&decode_pre_kernel<NC, F16>),
        hipFuncAttributeMaxDynamicSharedMemorySize, DECODE_LDS_BYTES);
    if (attr != hipSuccess) return attr;
    const int grid = (p.N + p.rows - 1) / p.rows;
    hipLaunchKernelGGL((decode_pre_kernel<NC, F16>), dim3(grid), dim3(1024),
                       decode_lds_bytes(p.K, p.rows, false), stream, p);
    return hipGetLastError();
}

template <bool F16>
inline hipError_t launch_decode_pre(const DecodePreArgs& p, hipStream_t stream) {
    switch (p.K / 1024) {
        case 1: return launch_decode_pre_t<1, F16>(p, stream);
        case 2: return launch_decode_pre_t<2, F16>(p, stream);
        case 3: return launch_decode_pre_t<3, F16>(p, stream);
        case 4: return launch_decode_pre_t<4, F16>(p, stream);
        case 5: return launch_decode_pre_t<5, F16>(p, stream);
        case 6: return launch_decode_pre_t<6, F16>(p, stream);
        case 7: return launch_decode_pre_t<7, F16>(p, stream);
        case 8: return launch_decode_pre_t<8, F16>(p, stream);
    }
    return hipErrorInvalidValue;
}

// M <= 8 tokens, K a multiple of 128 up to 8192, ~N/256 channels per
// workgroup (at most 32) whose tile and the code tile fit in LDS (rows
// padded to whole 1024-wide segments), and 32-bit buffer offsets.
// Channels per workgroup (a multiple of 4), or 0 if no size fits LDS.  Up
// to 256 * 32 channels, one workgroup per CU: R = N / 256 rounded up.
// Beyond that the CUs take several workgroups in turn, and R (at least 16,
// so the per-workgroup quantization stays small next to its weight stream)
// minimizes the channels the busiest CU streams: ceil(ceil(N/R) / 256) * R.
inline int decode_rows(int N, int K, bool codes = true) {
    const int KP = (K + 1023) / 1024 * 1024;
    int rmax = DECODE_MAX_ROWS;
    while (rmax >= 4 && decode_lds_bytes(KP, rmax, codes) > (size_t)DECODE_LDS_BYTES) rmax -= 4;
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
    if (M < 1 || M > DECODE_MAX_M || K % 128 != 0 || K > 8192) return false;
    const int R = decode_rows(N, K);
    if (R < 4) return false;
    return (int64_t)R * ldw < ((int64_t)1 << 31);
}

// The pre-quantized kernel: M <= 16 tokens, codes with lda % 16 == 0 (the
// GEMM entry points' rule), otherwise as decode_fits without the code tile.
constexpr int DECODE_PRE_MAX_M = 16;
inline bool decode_pre_fits(int M, int N, int K, int64_t ldw) {
    if (M < 1 || M > DECODE_PRE_MAX_M || K % 1024 != 0 || K > 8192) return false;
    const int R = decode_rows(N, K, false);
    if (R < 4) return false;
    return (int64_t)R * ldw < ((int64_t)1 << 31);
}

}  // namespace q8
