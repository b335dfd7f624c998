// stream_group.hpp -- the group-128 W8A8 GEMMs for few tokens (M <= 64),
// streaming the weight matrix once.
//
// Same results as gemm_i8_kernel's EPI_GROUP / EPI_GROUP_ACT(_F16)
// ("Qwen3.8-27B-GPTQ-INT8-W8A8-GS128", section "Quantization details": one
// weight scale per 128-wide K block; the per-group activation form with one
// activation scale per token and block as well): for each 128-wide K block
// g in ascending order the exact int32 block sum p_g is folded as
// f = fmaf((float)p_g, s, f) from f = 0, s = s_w[n,g] (EPI_GROUP, then
// y = bf16_rne(f * s_tok[m])) or s = fl(s_x[m,g] * s_w[n,g]) (ACT, then
// y = bf16_rne(f), fp16 with F16).
//
// The tiled kernel takes one 32 x 128 tile per workgroup at these sizes:
// 40 workgroups at N = 5120, 37 us for 26 MB of weights.  Here, as in
// stream_gemm_kernel, one 16-wave workgroup per CU owns R consecutive
// channels and all of K:
//  * waves 8..15 load rows d, d + 8, ... of the R x K weight tile into a
//    ring of LDS segment slots (1 KB of one row per instruction), and with
//    each segment the block scales it needs: R x 8 weight scales (and, for
//    ACT, 16 MG x 8 activation scales), 4-byte direct loads into a small
//    scale slot beside the weight slot (scales of blocks past K, and rows
//    or tokens past the ends, land as zeros).  They announce each segment
//    on an LDS counter as it lands and reuse a slot once every multiplying
//    wave has released it;
//  * wave t < 2 MG owns one 16 x 16 output tile (channels 16 (t & 1) ..,
//    tokens 16 (t >> 1) ..) over all of K: for each 128-wide block of a
//    segment, in ascending order, two v_mfma_i32_16x16x64_i8 from zero give
//    the exact block sum, folded at once into the tile's fp32 sums -- the
//    fold order of the definition, with no hand-over between waves.  The
//    activation fragments come straight from global memory, a segment's 16
//    loads issued before its wait.
// A K that is not a multiple of 1024 ends with a partial segment: its
// weights past K read as zero, and so do the scales of its blocks past K,
// so those blocks fold fmaf(0, 0, f) = f.
#pragma once

#include "lds_sync.hpp"
#include "stream_gemm.hpp"

namespace q8 {

struct StreamGroupArgs {
    const int8_t* x;  // [M, ldx] int8 codes
    int64_t ldx;
    const int8_t* w;  // [N, ldw] int8
    int64_t ldw;
    const float* s_x;  // EPI_GROUP: [M] token scales; ACT: [M, G] block scales
    const float* s_w;  // [N, G] weight block scales
    uint16_t* c;       // [M, ldc] bf16 (fp16 with F16)
    int64_t ldc;
    int M, N, K;
    int rows;  // channels per workgroup (multiple of 4, <= 32)
    int nbuf;  // segment slots in the ring
};

constexpr int SGG_SCALE_SLOT = 8 * SG_MAX_ROWS + 8 * SG_MAX_M;  // floats per scale slot

__host__ __device__ inline size_t sgg_lds_bytes(int rows, int nbuf) {
    return (size_t)nbuf * rows * SG_SEG + (size_t)nbuf * SGG_SCALE_SLOT * 4;
}

template <int MG, bool ACT, bool F16>
__global__ __launch_bounds__(1024) void stream_group_kernel(StreamGroupArgs p) {
    static_assert(!F16 || ACT, "fp16 outputs are a mode of the per-group activation form");
    constexpr int TOK = 16 * MG;  // token columns of the workgroup
    extern __shared__ __attribute__((aligned(1024))) int8_t lds[];
    __shared__ int ready[SG_MAX_SEG];  // loading waves done with segment s (8 = landed)
    __shared__ int freed[SG_MAX_SEG];  // multiplying waves done with segment s (2 MG = free)

    const int M = p.M, K = p.K, G = K >> 7, nseg = (K + SG_SEG - 1) / SG_SEG, nbuf = p.nbuf;
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int R = p.rows;
    const int n0 = blockIdx.x * R;
    const int rows = min(R, p.N - n0);
    const int tok = lane & 15, kg = lane >> 4;
    const int slot_bytes = R * SG_SEG;
    // scale slot s: [8][R] weight scales (block j of the segment, row r at
    // j R + r), then, for ACT, [8][TOK] activation scales
    float* sslot0 = reinterpret_cast<float*>(lds + nbuf * slot_bytes);

    for (int i = threadIdx.x; i < nseg; i += 1024) ready[i] = freed[i] = 0;
    wait_lgkm0();
    block_barrier();
    const uint64_t t_start = __builtin_amdgcn_s_memrealtime();

    if (wid < 2 * MG) {
        // ---- wave t: channel rows 16 ct .., token columns 16 tg ..
        const int ct = wid & 1, tg = wid >> 1;
        const int r = min(16 * ct + tok, rows - 1);         // weight row of the A fragments
        const int m = 16 * tg + tok;                         // token of the B fragment / outputs
        const __amdgpu_buffer_rsrc_t xr = make_rsrc(p.x, operand_extent(M, p.ldx, K));
        const int xrow = min(m, M - 1) * (int)p.ldx + 16 * kg;
        float st = 0.0f;
        if (!ACT && m < M) st = p.s_x[m];
        v4f f = v4f{};
        for (int sg = 0; sg < nseg; ++sg) {
            // a segment's activation fragments: block j, halves h (K bytes
            // 128 j + 64 h + 16 kg ..); blocks past K re-read the last one
            v4i b[8][2];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int kb = min(8 * sg + j, G - 1);
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    b[j][h] = __builtin_bit_cast(
                        v4i, __builtin_amdgcn_raw_buffer_load_b128(xr, xrow + 128 * kb + 64 * h, 0, 0));
            }
            sg_wait_ge(&ready[sg], 8);
            const int8_t* slot = lds + (sg % nbuf) * slot_bytes;
            const float* ss = sslot0 + (sg % nbuf) * SGG_SCALE_SLOT;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                v4i pg = v4i{};
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int u = 8 * j + 4 * h + kg;  // 16-byte unit of the segment row
                    const v4i a = *reinterpret_cast<const v4i*>(slot + r * SG_SEG + ((u ^ (r & 15)) << 4));
                    pg = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b[j][h], pg, 0, 0, 0);
                }
                // lane holds channels 16 ct + 4 kg + e of token m
                const v4f sw = *reinterpret_cast<const v4f*>(ss + j * R + 16 * ct + 4 * kg);
                float sx = 1.0f;
                if constexpr (ACT) sx = ss[8 * SG_MAX_ROWS + j * TOK + m];
#pragma unroll
                for (int e = 0; e < 4; ++e) f[e] = __builtin_fmaf((float)pg[e], ACT ? sx * sw[e] : sw[e], f[e]);
            }
            wait_lgkm0();  // this wave's reads of the slot are done
            if (lane == 0) sg_signal(&freed[sg]);
        }
        if (__builtin_amdgcn_s_memrealtime() - t_start > SG_WAVE_LIMIT_TICKS && lane == 0)
            atomicAdd(&sg_wait_timeouts, 1u);
        // ---- epilogue: token m, channels n0 + 16 ct + 4 kg + e
        const int ch = 16 * ct + 4 * kg;
        if (m < M && ch < rows) {
            float y[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) y[e] = ACT ? f[e] : f[e] * st;
            v2u o;
            o[0] = pack16x2<F16>(y[0], y[1]);
            o[1] = pack16x2<F16>(y[2], y[3]);
            *reinterpret_cast<v2u*>(p.c + (int64_t)m * p.ldc + n0 + ch) = o;
        }
    } else if (wid >= 8) {
        // ---- loading wave d: rows d + 8 j, segment by segment; wave 8 also
        // moves the segment's block scales
        const int d = wid - 8;
        const int cnt = rows > d ? (rows - d + 7) / 8 : 0;
        const int nsw = d == 0 ? (8 * R + 63) / 64 : 0;                 // weight-scale loads
        const int nsx = d == 0 && ACT ? (8 * TOK + 63) / 64 : 0;        // activation-scale loads
        const int per = cnt + nsw + nsx;                                 // loads per segment
        const __amdgpu_buffer_rsrc_t wr = make_rsrc(p.w + (int64_t)n0 * p.ldw,
                                                    (uint32_t)((int64_t)rows * p.ldw));
        const __amdgpu_buffer_rsrc_t swr = make_rsrc(p.s_w, (uint32_t)((int64_t)p.N * G * 4));
        const __amdgpu_buffer_rsrc_t sxr = make_rsrc(p.s_x, ACT ? (uint32_t)((int64_t)M * G * 4) : 0u);
        auto issue = [&](int sg) __attribute__((always_inline)) {
            int8_t* slot = lds + (sg % nbuf) * slot_bytes;
            for (int j = 0; j < cnt; ++j) {
                const int rr = d + 8 * j;
                const int ku = sg * SG_SEG + ((lane ^ (rr & 15)) << 4);  // K byte of this lane's unit
                // past K: offset 2^31, beyond any resource here (the entry
                // point keeps rows * ldw below 2^31), which reads as zero
                const int voff = ku < K ? rr * (int)p.ldw + ku : INT32_MIN;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (Q8_LDS void*)(slot + rr * SG_SEG), 16, voff, 0, 0,
                                                         2);
            }
            float* ss = sslot0 + (sg % nbuf) * SGG_SCALE_SLOT;
            for (int q = 0; q < nsw; ++q) {
                const int i = 64 * q + lane, j = i / R, rr = i - j * R;  // scale of row rr, block 8 sg + j
                const int kb = 8 * sg + j;
                const int voff = j < 8 && rr < rows && kb < G ? ((n0 + rr) * G + kb) * 4 : INT32_MIN;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(swr, (Q8_LDS void*)(ss + 64 * q), 4, voff, 0, 0, 0);
            }
            for (int q = 0; q < nsx; ++q) {
                const int i = 64 * q + lane, j = i / TOK, mm = i - j * TOK;  // token mm, block 8 sg + j
                const int kb = 8 * sg + j;
                const int voff = j < 8 && mm < M && kb < G ? (mm * G + kb) * 4 : INT32_MIN;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(sxr, (Q8_LDS void*)(ss + 8 * SG_MAX_ROWS + 64 * q), 4,
                                                         voff, 0, 0, 0);
            }
        };
        const int first = min(nbuf, nseg);
        for (int sg = 0; sg < first; ++sg) issue(sg);
        int issued = first;
        for (int sg = 0; sg < nseg; ++sg) {
            sg_wait_vm((issued - 1 - sg) * per);  // segments 0..sg landed
            if (lane == 0) sg_signal(&ready[sg]);
            if (issued < nseg) {
                sg_wait_ge(&freed[sg], 2 * MG);  // slot of sg free again
                issue(issued);
                ++issued;
            }
        }
        if (__builtin_amdgcn_s_memrealtime() - t_start > SG_WAVE_LIMIT_TICKS && lane == 0)
            atomicAdd(&sg_wait_timeouts, 1u);
    }
}

// Where the group-scaled GEMMs stream: K a multiple of 128, 32-bit buffer
// offsets for the tile and the scales, and up to 16 tokens -- or up to 64
// when the grid is one wave of workgroups.  With several waves and more
// tokens the 2 MG multiplying waves of each workgroup fall behind the
// tiled kernel: per call in a graph on rotating weight copies, against
// the 32 x 128 tiles (bit-identical), 5120 x 5120 at 1 / 16 / 64 tokens
// 9.8 / 11.8 / 23.8 against 36.9-37.1 us, 5120 x 17408 27.7 / 32.9 / 71.3
// against 114-116 us, 15360 x 5120 (three waves) 26.5 / 32.6 against 39.6
// us but 43.2 / 68.6 against 39.7 / 39.3 us at 32 / 64 tokens.
inline bool sgg_fits(int M, int N, int K, int64_t ldx, int64_t ldw) {
    if (!sg_fits(M, N, K, ldw, SG_MAX_M)) return false;
    const int R = sg_rows(N);
    if (M > 16 && ((N + R - 1) / R + 255) / 256 > 1) return false;
    const int64_t lim = (int64_t)1 << 31;
    return (int64_t)(N + 64) * (K / 128) * 4 < lim && (int64_t)M * ldx + K < lim;
}

template <int MG, bool ACT, bool F16>
inline hipError_t launch_stream_group_t(const StreamGroupArgs& p, hipStream_t stream) {
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&stream_group_kernel<MG, ACT, F16>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)sgg_lds_bytes(SG_MAX_ROWS, SG_NBUF));
    if (attr != hipSuccess) return attr;
    const int grid = (p.N + p.rows - 1) / p.rows;
    hipLaunchKernelGGL((stream_group_kernel<MG, ACT, F16>), dim3(grid), dim3(1024),
                       sgg_lds_bytes(p.rows, p.nbuf), stream, p);
    return hipGetLastError();
}

// Fills rows and nbuf from N, then launches for the token count.
template <bool ACT, bool F16>
inline hipError_t launch_stream_group(StreamGroupArgs p, hipStream_t stream) {
    p.rows = sg_rows(p.N);
    p.nbuf = SG_NBUF;
    if (p.M <= 16) return launch_stream_group_t<1, ACT, F16>(p, stream);
    if (p.M <= 32) return launch_stream_group_t<2, ACT, F16>(p, stream);
    return launch_stream_group_t<4, ACT, F16>(p, stream);
}

}  // namespace q8
