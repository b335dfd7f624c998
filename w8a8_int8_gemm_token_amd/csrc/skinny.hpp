// skinny.hpp -- INT8 GEMM for decode-sized batches (M <= 16 tokens).
//
// Decode streams the whole weight matrix once per call and is bound by HBM
// bandwidth ("Qwen3.8-27B-INT8-W8A8", section "Throughput": decode is
// weight-bandwidth-bound), so this kernel is built around the weight stream:
//  * one workgroup per 8 output channels; wave w owns the K slice
//    [w*K/4, (w+1)*K/4) of the 8 x K weight tile and moves it straight to
//    its own LDS region with buffer_load_dwordx4 ... lds.  Each such wave
//    instruction covers 4 rows x 256 contiguous bytes; all of a wave's
//    instructions are issued up front, so the whole matrix is in flight at
//    once across the grid.
//  * the wave first loads the activation codes of its K slice with plain
//    coalesced loads (8 token rows x 128 bytes per instruction; every
//    workgroup reads the whole code matrix, so its layout in flight matters
//    as much as the weights'), then issues the weight stream, then consumes
//    the stream 256 bytes of K at a time as its own loads land (vmcnt): no
//    barrier is needed until the end, because a wave only reads the LDS it
//    filled.  The codes are moved into the MFMA B-operand layout (lane = token
//    + 16 * k-group) with ds_bpermute; v_mfma_i32_16x16x64_i8 accumulates
//    exact int32.
//  * inside a 4-row x 256-byte piece, chunk c of row r sits at slot
//    16*(r%4) + (c ^ (r & 15)), so the A-fragment reads (16 rows, one chunk
//    each) are conflict-free.
//  * the four K slices are summed in LDS (exact int32), then the epilogue
//    y = bf16_rne(((float)acc * s_tok[m]) * s_ch[n]).
// A workgroup owns 8 channels (the MFMA's rows 8..15 repeat them and are
// dropped): with K = 5120 its tile is 40 KB, four workgroups share a CU and
// all N/8 workgroups of a 5120-channel layer are resident at once.
#pragma once

#include "gemm_i8.hpp"

namespace q8 {

constexpr int SKINNY_MAX_M = 16;
constexpr int SKINNY_SEG = 256;  // bytes of K per weight-stream segment

struct SkinnyArgs {
    const int8_t* xq;  // [M, ldx] activation codes
    int64_t ldx;
    const int8_t* w;  // [N, ldw] weight codes
    int64_t ldw;
    const float* s_tok;  // [M]
    const float* s_ch;   // [N]
    uint16_t* c;         // [M, ldc] bf16
    int64_t ldc;
    int M, N, K;
};

// Each wave's K slice is a whole number of 256-byte segments: K % 1024 == 0.
// A workgroup owns ROWS (8 or 16) channels; with 8 the MFMA rows 8..15 repeat
// rows 0..7 and their results are dropped, which halves the LDS tile so that
// more workgroups stay resident per CU.
inline size_t skinny_lds_bytes(int K, int rows) { return (size_t)rows * K; }

// Lane `src` of a 64-lane wave, one dword (ds_bpermute takes a byte index).
__device__ __forceinline__ int lane_fetch(int src_byte, int v) {
    return __builtin_amdgcn_ds_bpermute(src_byte, v);
}

template <int NSEG, int ROWS, bool T16>  // K = 4 * 256 * NSEG; T16: 8 < M <= 16
__global__ __launch_bounds__(256) void skinny_gemm_kernel(SkinnyArgs p) {
    constexpr int RG = ROWS / 4;  // 4-row groups per segment
    extern __shared__ __attribute__((aligned(1024))) int8_t lds[];
    const int M = p.M, N = p.N;
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n0 = blockIdx.x * ROWS;
    const int k0 = wid * NSEG * SKINNY_SEG;       // this wave's K slice
    int8_t* lw = lds + wid * (NSEG * RG * 1024);  // this wave's LDS region
    const int tok = lane & 15, kg = lane >> 4;

    // ---- epilogue scales, fetched now so their latency is hidden by the
    // stream (wave 0 writes the outputs: token tok, channels n0 + 4kg + e)
    const int ch = n0 + 4 * kg;
    const bool writer = wid == 0 && tok < M && 4 * kg < ROWS && ch < N;
    float st = 0.0f;
    v4f sc = v4f{};
    if (writer) {
        st = p.s_tok[tok];
#pragma unroll
        for (int e = 0; e < 4; ++e) sc[e] = p.s_ch[ch + e];
    }

    // ---- activation codes of the slice, loaded first so they land before
    // the weight stream: piece j = K bytes [k0 + 128j, +128) of token rows
    // l/8 (xa) and 8 + l/8 (xb); lane l holds chunk l%8 of its row.
    constexpr int NJ = NSEG * 2;
    const int lt = lane >> 3, lc = lane & 7;
    v4i xa[NJ], xb[T16 ? NJ : 1];
    {
        const int8_t* ra = p.xq + (int64_t)lt * p.ldx + k0 + lc * 16;
#pragma unroll
        for (int j = 0; j < NJ; ++j) xa[j] = lt < M ? *reinterpret_cast<const v4i*>(ra + j * 128) : v4i{};
        if constexpr (T16) {
            const int8_t* rb = ra + 8 * p.ldx;
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                xb[j] = lt + 8 < M ? *reinterpret_cast<const v4i*>(rb + j * 128) : v4i{};
        }
    }
    // B fragment of block 2j + h for lane (tok, kg): chunk 4h + kg of token
    // tok, i.e. lane 8 * (tok % 8) + 4h + kg of piece j
    const int src = ((tok & 7) * 8 + kg) * 4;
    auto bfrag = [&](int j, int h) __attribute__((always_inline)) {
        v4i r;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int va = lane_fetch(src + h * 16, xa[j][e]);
            if constexpr (T16) {
                const int vb = lane_fetch(src + h * 16, xb[j][e]);
                r[e] = tok < 8 ? va : vb;
            } else {
                r[e] = tok < 8 ? va : 0;
            }
        }
        return r;
    };

    // ---- weight stream: piece (segment sg, row group rg) = rows 4rg..4rg+3
    // x bytes [k0 + 256 sg, +256); lane l writes slot l of the piece: row
    // 4rg + l/16, global chunk (l%16) ^ (row & 15) of the segment.
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(p.w, (uint32_t)((int64_t)N * p.ldw));
#pragma unroll
    for (int sg = 0; sg < NSEG; ++sg) {
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
            const int r = rg * 4 + (lane >> 4);
            const int voff = r * (int)p.ldw + (((lane & 15) ^ r) << 4);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                wr, (Q8_LDS void*)(lw + (sg * RG + rg) * 1024), 16, voff,
                n0 * (int)p.ldw + k0 + sg * SKINNY_SEG, 0, 0);
        }
    }

    // ---- consume segment by segment as this wave's loads land
    // A fragment of block (sg, j): row tok % ROWS, chunk 4j + kg of segment sg
    const int arow = tok % ROWS;
    const int aoff = (arow >> 2) * 1024 + (arow & 3) * 256;
    v4i acc0 = v4i{}, acc1 = v4i{};
#pragma unroll
    for (int sg = 0; sg < NSEG; ++sg) {
        // the codes and segments 0..sg are done once at most RG*(NSEG-1-sg)
        // loads remain in flight
        switch (NSEG - 1 - sg) {
#define Q8_WAIT_CASE(n) case n: wait_vm_lgkm0<RG * (n)>(); break;
            Q8_WAIT_CASE(0) Q8_WAIT_CASE(1) Q8_WAIT_CASE(2) Q8_WAIT_CASE(3)
            Q8_WAIT_CASE(4) Q8_WAIT_CASE(5) Q8_WAIT_CASE(6) Q8_WAIT_CASE(7)
            Q8_WAIT_CASE(8) Q8_WAIT_CASE(9) Q8_WAIT_CASE(10) Q8_WAIT_CASE(11)
            Q8_WAIT_CASE(12) Q8_WAIT_CASE(13) Q8_WAIT_CASE(14) Q8_WAIT_CASE(15)
#undef Q8_WAIT_CASE
        }
        const int8_t* seg = lw + sg * RG * 1024 + aoff;
        v4i a[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) a[j] = *reinterpret_cast<const v4i*>(seg + (((4 * j + kg) ^ arow) << 4));
        acc0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[0], bfrag(2 * sg, 0), acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[1], bfrag(2 * sg, 1), acc1, 0, 0, 0);
        acc0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[2], bfrag(2 * sg + 1, 0), acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[3], bfrag(2 * sg + 1, 1), acc1, 0, 0, 0);
    }
    v4i acc = acc0 + acc1;

    // ---- sum the four K slices (exact int32)
    block_barrier();  // every wave is done with its LDS region
    v4i* red = reinterpret_cast<v4i*>(lds);
    if (wid != 0) red[(wid - 1) * 64 + lane] = acc;
    wait_vm_lgkm0<0>();
    block_barrier();
    if (wid != 0) return;
    acc += red[lane] + red[64 + lane] + red[128 + lane];
    if (!writer) return;
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float u = (float)acc[e] * st;
        v[e] = u * sc[e];
    }
    v2u o;
    o[0] = pack_bf16x2(v[0], v[1]);
    o[1] = pack_bf16x2(v[2], v[3]);
    *reinterpret_cast<v2u*>(p.c + (int64_t)tok * p.ldc + ch) = o;
}

template <int NSEG, int ROWS, bool T16>
inline hipError_t launch_skinny_t(const SkinnyArgs& p, hipStream_t stream) {
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&skinny_gemm_kernel<NSEG, ROWS, T16>),
        hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((skinny_gemm_kernel<NSEG, ROWS, T16>), dim3((p.N + ROWS - 1) / ROWS), dim3(256),
                       skinny_lds_bytes(p.K, ROWS), stream, p);
    return hipGetLastError();
}

template <int NSEG, int ROWS = 8>
inline hipError_t launch_skinny_n(const SkinnyArgs& p, hipStream_t stream) {
    return p.M > 8 ? launch_skinny_t<NSEG, ROWS, true>(p, stream)
                   : launch_skinny_t<NSEG, ROWS, false>(p, stream);
}

inline hipError_t launch_skinny(const SkinnyArgs& p, hipStream_t stream) {
    switch (p.K / 1024) {
        case 1: return launch_skinny_n<1>(p, stream);
        case 2: return launch_skinny_n<2>(p, stream);
        case 3: return launch_skinny_n<3>(p, stream);
        case 4: return launch_skinny_n<4>(p, stream);
        case 5: return launch_skinny_n<5>(p, stream);
        case 6: return launch_skinny_n<6>(p, stream);
        case 7: return launch_skinny_n<7>(p, stream);
        case 8: return launch_skinny_n<8>(p, stream);
        case 9: return launch_skinny_n<9>(p, stream);
        case 10: return launch_skinny_n<10>(p, stream);
    }
    return hipErrorInvalidValue;
}

// K a multiple of 1024 up to 10240 (the tile fits in LDS), 32-bit offsets.
inline bool skinny_fits(const SkinnyArgs& p) {
    return p.M <= SKINNY_MAX_M && p.K % 1024 == 0 && p.K <= 10240 &&
           ((int64_t)p.N + 16) * p.ldw < ((int64_t)1 << 31);
}

}  // namespace q8
