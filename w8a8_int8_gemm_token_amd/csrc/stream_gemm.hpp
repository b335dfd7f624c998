// stream_gemm.hpp -- GEMMs for a few tokens (M <= 64), which stream the
// weight matrix once and are bound by HBM bandwidth:
//   I8 (W8A8):  y[m,n] = bf16_rne(((float)sum_k xq[m,k]*w[n,k] * s_tok[m]) * s_ch[n])
//               (or fp16_rne: the fp16 variant of the layer)
//               exact int32 sums of the per-token codes
//   bf16 (W8A16): y[m,n] = bf16_rne(s_ch[n] * sum_k x[m,k] * bf16(w[n,k]))
// "Qwen3.8-27B -- SmoothQuant + activation-aware GPTQ, W8A8 INT8 (v3)",
// sections "Recipe" (the W8A8 and W8A16 module groups) and "Results"
// (single-stream decode); "Qwen3.8-27B-INT8-W8A8", section "Throughput"
// (decode is weight-bandwidth-bound); "lued/Qwen3.8-27B-INT8-W8A16-MTP",
// section "Why W8A16 on Ampere" (weights rebuilt in 16 bits).
//
// One 16-wave workgroup per CU owns R consecutive channels and all of K:
//  * waves 8..15 load: rows d, d+8, ... of the tile, K segment by K segment
//    (1 KB of one row per buffer_load_dwordx4 ... lds), into a ring of 3
//    segment slots in LDS; after each
//    segment lands (vmcnt) a wave increments that segment's `ready`
//    counter, and before reusing a slot it waits until all 8 multiplying
//    waves have released it (`freed`);
//  * waves 0..7 multiply: wave c takes its share of the K blocks of every
//    segment, reads the activation fragments (codes or bf16) straight from
//    global memory (the M x K block stays in L2) for MG groups of 16 tokens,
//    and runs 16x16 MFMAs (v_mfma_i32_16x16x64_i8, or
//    v_mfma_f32_16x16x32_bf16 on weights converted to bf16 as they are read:
//    exact, |q| <= 128) on both 16-row tiles;
//  * the 8 partial tiles are summed in LDS (exact int32 for I8), and waves
//    0 .. 2*MG-1 apply the epilogue.
// Progress: a loading wave signals segment s before it waits on any
// counter, and a multiplying wave releases segment s before it waits on
// segment s+1, so every wait is on an event that needs no further waiting;
// the polls are bounded all the same.  Rows and tokens past the ends repeat
// the last valid one; their outputs are never stored.
// Segment slot layout: [R][1024] bytes, 16-byte unit u of row r stored at
// unit u ^ (r & 15), so the fragment reads of 16 rows are conflict-free.
// K is a multiple of 128; when it is not one of 1024 the last segment is
// partial: its weight loads past K read nothing (an out-of-range offset
// returns zero), and the multiplying waves' K blocks past K pair those zeros
// with the last valid block's activations, adding exact zeros.
#pragma once

#include <type_traits>

#include "decode_fused.hpp"
#include "gemm_i8.hpp"
#include "lds_sync.hpp"
#include "w8a16.hpp"

namespace q8 {

constexpr int SG_MAX_M = 64;
constexpr int SG_SEG = 1024;       // K per segment
constexpr int SG_MAX_SEG = 128;    // K <= 131072
constexpr int SG_MAX_ROWS = 32;
constexpr int SG_RING_BYTES = 150 * 1024;
constexpr int SG_NBUF = 3;

typedef __bf16 v8bf16 __attribute__((ext_vector_type(8)));

struct StreamArgs {
    const void* x;  // [M, ldx]: int8 codes (I8), bf16, or fp16 (W8A16 with out_f16)
    int64_t ldx;
    const int8_t* w;  // [N, ldw] int8
    int64_t ldw;
    const float* s_tok;  // [M] (I8 only)
    const float* s_ch;   // [N]
    uint16_t* c;         // [M, ldc] bf16, or fp16 when out_f16
    int64_t ldc;
    int M, N, K;
    int rows;  // channels per workgroup (multiple of 4, <= 32)
    int nbuf;  // segment slots in the ring
    int out_f16;  // fp16 outputs (RNE) instead of bf16 (and, W8A16, fp16 activations)
};

// Three slots: a deeper ring issues most of a short K at once, and the
// loading waves then stall at issue the way a whole-tile load does
// (measured slower for K = 5120; no faster for K = 17408).
inline int sg_nbuf(int rows) {
    const int n = SG_RING_BYTES / (rows * SG_SEG);
    return n < SG_NBUF ? n : SG_NBUF;
}
__host__ __device__ inline size_t sg_lds_bytes(int rows, int nbuf, int mg) {
    const size_t ring = (size_t)nbuf * rows * SG_SEG;
    const size_t red = (size_t)2 * mg * 8 * 64 * 16;  // partial tiles of the 8 multiplying waves
    return ring > red ? ring : red;
}

__device__ __forceinline__ v8h i8x8_to_f16x8(v2u raw) {
    const v2u lo = i8x4_to_f16x4(raw[0]), hi = i8x4_to_f16x4(raw[1]);
    return __builtin_bit_cast(v8h, v4u{lo[0], lo[1], hi[0], hi[1]});
}
__device__ __forceinline__ v8bf16 i8x8_to_bf16x8(v2u raw) {
    const v2u lo = i8x4_to_bf16x4(raw[0]), hi = i8x4_to_bf16x4(raw[1]);
    return __builtin_bit_cast(v8bf16, v4u{lo[0], lo[1], hi[0], hi[1]});
}

// F16 (W8A16 only): fp16 activations, v_mfma_f32_16x16x32_f16.
// Up to 32 tokens (I8) or 16 (bf16) a workgroup fits in 64 registers per
// lane, so two workgroups share a CU when the tile is small (large N); the
// second launch-bounds argument (waves per SIMD) keeps it there.
template <bool I8, int MG>
constexpr int sg_waves_per_simd() { return (I8 ? MG <= 2 : MG == 1) ? 8 : 4; }

template <bool I8, int MG, bool F16 = false>
__global__ __launch_bounds__(1024, (sg_waves_per_simd<I8, MG>())) void stream_gemm_kernel(StreamArgs p) {
    // K blocks per MFMA: 64 (int8) or 32 (bf16); per segment and wave
    constexpr int KB = I8 ? 64 : 32;
    constexpr int BPW = SG_SEG / KB / 8;
    typedef typename std::conditional<I8, v4i, v4f>::type acc_t;
    extern __shared__ __attribute__((aligned(1024))) int8_t lds[];
    __shared__ int ready[SG_MAX_SEG];  // loading waves done with segment s (8 = landed)
    __shared__ int freed[SG_MAX_SEG];  // multiplying waves done with segment s (8 = free)

    const int M = p.M, K = p.K, nseg = (K + SG_SEG - 1) / SG_SEG, nbuf = p.nbuf;
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int R = p.rows;
    const int n0 = blockIdx.x * R;
    const int rows = min(R, p.N - n0);
    const int tok = lane & 15, kg = lane >> 4;
    const int slot_bytes = R * SG_SEG;

    // epilogue operands: wave w < 2*MG writes tile t = w / MG, token group
    // g = w % MG: token 16g + tok, channels n0 + 16t + 4kg + e
    const int et = wid / MG, eg = wid % MG;
    const int em = 16 * eg + tok;
    const int ch = n0 + 16 * et + 4 * kg;
    const bool writer = wid < 2 * MG && em < M && 16 * et + 4 * kg < rows;
    v4f sc = v4f{};
    float st = 1.0f;
    if (writer) {
#pragma unroll
        for (int e = 0; e < 4; ++e) sc[e] = p.s_ch[ch + e];
        if constexpr (I8) st = p.s_tok[em];
    }
    for (int i = threadIdx.x; i < nseg; i += 1024) ready[i] = freed[i] = 0;
    wait_lgkm0();
    block_barrier();

    acc_t acc[2][MG];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int g = 0; g < MG; ++g) acc[t][g] = acc_t{};
    const uint64_t t_start = __builtin_amdgcn_s_memrealtime();
    if (wid < 8) {
        // ---- multiplying wave: K blocks BPW*wid .. BPW*wid + BPW-1 of
        // every segment
        const int r0 = min(tok, rows - 1), r1 = min(16 + tok, rows - 1);
        const int8_t* xb[MG];
#pragma unroll
        for (int g = 0; g < MG; ++g) {
            const int tc = min(16 * g + tok, M - 1);
            xb[g] = static_cast<const int8_t*>(p.x) + ((int64_t)tc * p.ldx + (I8 ? 16 : 8) * kg) * (I8 ? 1 : 2);
        }
        // activation fragments (16 bytes per lane: 16 codes or 8 bf16) are
        // loaded before the wait on the segment when they fit in registers
        constexpr bool PRE = BPW * MG <= 8;
        // A wave's K range in a segment is 128 wide and 128-aligned, so with
        // K % 128 == 0 it lies wholly below or past K.  Past K (in a partial
        // last segment) the wave re-reads the last valid range's
        // activations: finite values (non-finite inputs are out of
        // contract) that meet the zeros the loading waves left in the slot
        // there, so those products add exact zeros (an fp32 sum that starts
        // at +0 never becomes -0, so even the sign of zero is unchanged).
        static_assert(KB * BPW == 128, "one 128-deep K range per wave and segment");
        auto bload = [&](int kb, int j, int g) __attribute__((always_inline)) {
            return *reinterpret_cast<const v4u*>(xb[g] + (int64_t)(kb + KB * j) * (I8 ? 1 : 2));
        };
        for (int sg = 0; sg < nseg; ++sg) {
            const int kb = min(sg * SG_SEG + KB * BPW * wid, K - KB * BPW);
            v4u b[PRE ? BPW : 1][MG];
            if constexpr (PRE) {
#pragma unroll
                for (int j = 0; j < BPW; ++j)
#pragma unroll
                    for (int g = 0; g < MG; ++g) b[j][g] = bload(kb, j, g);
            }
            sg_wait_ge(&ready[sg], 8);
            const int8_t* slot = lds + (sg % nbuf) * slot_bytes;
#pragma unroll
            for (int jj = 0; jj < BPW; ++jj) {
                const int j = PRE ? jj : 0;
                if constexpr (!PRE) {
#pragma unroll
                    for (int g = 0; g < MG; ++g) b[0][g] = bload(kb, jj, g);
                }
                const int o = KB * (BPW * wid + jj) + (I8 ? 16 : 8) * kg;  // byte of K in the row
                const int u = o >> 4;
                if constexpr (I8) {
                    const v4i a0 = *reinterpret_cast<const v4i*>(slot + r0 * SG_SEG + ((u ^ (r0 & 15)) << 4));
                    const v4i a1 = *reinterpret_cast<const v4i*>(slot + r1 * SG_SEG + ((u ^ (r1 & 15)) << 4));
#pragma unroll
                    for (int g = 0; g < MG; ++g) {
                        const v4i bg = __builtin_bit_cast(v4i, b[j][g]);
                        acc[0][g] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, bg, acc[0][g], 0, 0, 0);
                        acc[1][g] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, bg, acc[1][g], 0, 0, 0);
                    }
                } else if constexpr (F16) {
                    const int h = (o >> 3) & 1;
                    const v8h a0 = i8x8_to_f16x8(
                        *reinterpret_cast<const v2u*>(slot + r0 * SG_SEG + ((u ^ (r0 & 15)) << 4) + (h << 3)));
                    const v8h a1 = i8x8_to_f16x8(
                        *reinterpret_cast<const v2u*>(slot + r1 * SG_SEG + ((u ^ (r1 & 15)) << 4) + (h << 3)));
#pragma unroll
                    for (int g = 0; g < MG; ++g) {
                        const v8h bg = __builtin_bit_cast(v8h, b[j][g]);
                        acc[0][g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, bg, acc[0][g], 0, 0, 0);
                        acc[1][g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, bg, acc[1][g], 0, 0, 0);
                    }
                } else {
                    const int h = (o >> 3) & 1;
                    const v8bf16 a0 = i8x8_to_bf16x8(
                        *reinterpret_cast<const v2u*>(slot + r0 * SG_SEG + ((u ^ (r0 & 15)) << 4) + (h << 3)));
                    const v8bf16 a1 = i8x8_to_bf16x8(
                        *reinterpret_cast<const v2u*>(slot + r1 * SG_SEG + ((u ^ (r1 & 15)) << 4) + (h << 3)));
#pragma unroll
                    for (int g = 0; g < MG; ++g) {
                        const v8bf16 bg = __builtin_bit_cast(v8bf16, b[j][g]);
                        acc[0][g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, bg, acc[0][g], 0, 0, 0);
                        acc[1][g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, bg, acc[1][g], 0, 0, 0);
                    }
                }
            }
            wait_lgkm0();  // this wave's reads of the slot are done
            if (lane == 0) sg_signal(&freed[sg]);
        }
    } else {
        // ---- loading wave d: rows d + 8 j, segment by segment
        const int d = wid - 8;
        const int cnt = rows > d ? (rows - d + 7) / 8 : 0;
        const __amdgpu_buffer_rsrc_t wr = make_rsrc(p.w + (int64_t)n0 * p.ldw,
                                                    (uint32_t)((int64_t)rows * p.ldw));
        auto issue = [&](int sg) __attribute__((always_inline)) {
            int8_t* slot = lds + (sg % nbuf) * slot_bytes;
            for (int j = 0; j < cnt; ++j) {
                const int r = d + 8 * j;
                const int ku = sg * SG_SEG + ((lane ^ (r & 15)) << 4);  // K byte of this lane's unit
                // past K: offset 2^31, beyond any resource here (sg_fits keeps
                // rows * ldw below 2^31), which reads as zero
                const int voff = ku < K ? r * (int)p.ldw + ku : INT32_MIN;
                // non-temporal (cache policy 2): the weights are read once
                __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (Q8_LDS void*)(slot + r * SG_SEG), 16, voff,
                                                         0, 0, 2);
            }
        };
        const int first = min(nbuf, nseg);
        for (int sg = 0; sg < first; ++sg) issue(sg);
        int issued = first;
        for (int sg = 0; sg < nseg; ++sg) {
            sg_wait_vm((issued - 1 - sg) * cnt);  // segments 0..sg landed
            if (lane == 0) sg_signal(&ready[sg]);
            if (issued < nseg) {
                sg_wait_ge(&freed[sg], 8);  // slot of sg free again
                issue(issued);
                ++issued;
            }
        }
    }

    // ---- sum the 8 multiplying waves' partial tiles, epilogue
    if (__builtin_amdgcn_s_memrealtime() - t_start > SG_WAVE_LIMIT_TICKS && lane == 0)
        atomicAdd(&sg_wait_timeouts, 1u);
    block_barrier();  // every wave is done with the ring
    acc_t* red = reinterpret_cast<acc_t*>(lds);
    if (wid < 8) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int g = 0; g < MG; ++g) red[((t * MG + g) * 8 + wid) * 64 + lane] = acc[t][g];
    }
    wait_lgkm0();
    block_barrier();
    if (!writer) return;
    acc_t s = acc_t{};
#pragma unroll
    for (int w = 0; w < 8; ++w) s += red[(wid * 8 + w) * 64 + lane];
    float y[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        if constexpr (I8) {
            const float u = (float)s[e] * st;
            y[e] = u * sc[e];
        } else {
            y[e] = s[e] * sc[e];
        }
    }
    v2u o;
    if (p.out_f16) {
        o[0] = pack_f16x2(y[0], y[1]);
        o[1] = pack_f16x2(y[2], y[3]);
    } else {
        o[0] = pack_bf16x2(y[0], y[1]);
        o[1] = pack_bf16x2(y[2], y[3]);
    }
    *reinterpret_cast<v2u*>(p.c + (int64_t)em * p.ldc + ch) = o;
}

// Channels per workgroup: N / 256 rounded up to a multiple of 4 when that is
// at most 32 (one workgroup per CU); otherwise the size in [16, 32] that
// minimizes the channels the busiest CU streams over whole waves of 256.
inline int sg_rows(int N) {
    const int r1 = (((N + 255) / 256) + 3) & ~3;
    if (r1 <= SG_MAX_ROWS) return r1;
    int best = SG_MAX_ROWS;
    int64_t cost = INT64_MAX;
    for (int r = SG_MAX_ROWS; r >= 16; r -= 4) {
        const int64_t c = (int64_t)((((int64_t)N + r - 1) / r + 255) / 256) * r;
        if (c < cost) cost = c, best = r;
    }
    return best;
}

// The one-call layer at up to 8 tokens: the fused decode kernel (every
// workgroup quantizes the rows for itself while its weights stream) unless
// its whole-tile LDS budget makes the busiest CU stream 32 KB or more of
// weights beyond what the row quantizer + streaming kernel would.  Per call
// in a graph on rotating weight copies, 1-8 tokens: at 17408 x 5120 (the
// fused kernel's 871 workgroups of 20 rows, 80 rows per CU, against 726 of
// 24, 72 rows) 21.1-23.7 us fused against 20.4-21.0 us; at 13824 x 5120
// (60 against 56 rows per CU) 16.5-18.4 us fused against 18.0-19.0.
inline bool decode_beats_stream(int N, int K) {
    const int rf = decode_rows(N, K), rs = sg_rows(N);
    if (rf < 4) return false;
    // more than three waves of workgroups: the repeated quantization shows
    // even at equal channels per CU (18944 x 3584, 948 workgroups of 20
    // rows on both routes: 18.6-20.8 us fused against 18.1-19.1)
    if ((((int64_t)N + rf - 1) / rf + 255) / 256 > 3) return false;
    const int64_t cf = (int64_t)((((int64_t)N + rf - 1) / rf + 255) / 256) * rf;
    const int64_t cs = (int64_t)((((int64_t)N + rs - 1) / rs + 255) / 256) * rs;
    return (cf - cs) * K < 32768;
}

// M <= max_m, K a multiple of 128, 32-bit buffer offsets for the tile.
inline bool sg_fits(int M, int N, int K, int64_t ldw, int max_m) {
    if (M < 1 || M > max_m || K % 128 != 0 || (K + SG_SEG - 1) / SG_SEG > SG_MAX_SEG) return false;
    return (int64_t)sg_rows(N) * ldw < ((int64_t)1 << 31);
}

template <bool I8, int MG, bool F16>
inline hipError_t launch_stream_t(const StreamArgs& p, hipStream_t stream) {
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&stream_gemm_kernel<I8, MG, F16>),
        hipFuncAttributeMaxDynamicSharedMemorySize, SG_RING_BYTES);
    if (attr != hipSuccess) return attr;
    const int grid = (p.N + p.rows - 1) / p.rows;
    hipLaunchKernelGGL((stream_gemm_kernel<I8, MG, F16>), dim3(grid), dim3(1024),
                       sg_lds_bytes(p.rows, p.nbuf, MG), stream, p);
    return hipGetLastError();
}

// Fills rows and nbuf from N, then launches for the token count.  F16 (W8A16
// only): fp16 activations and outputs.
template <bool I8, bool F16 = false>
inline hipError_t launch_stream(StreamArgs p, hipStream_t stream) {
    static_assert(!(I8 && F16), "fp16 activations are a W8A16 mode");
    p.rows = sg_rows(p.N);
    p.nbuf = sg_nbuf(p.rows);
    if (F16) p.out_f16 = 1;
    if (p.M <= 16) return launch_stream_t<I8, 1, F16>(p, stream);
    if (p.M <= 32) return launch_stream_t<I8, 2, F16>(p, stream);
    return launch_stream_t<I8, 4, F16>(p, stream);
}

}  // namespace q8
