// gemm_big.hpp -- the large-problem INT8 GEMM with the per-channel (or raw
// int32) epilogue on 256-token x 384-channel tiles.
//
// It computes exactly gemm_i8_kernel's EPI_CHANNEL / EPI_I32 result
// ("Qwen3.8-27B -- SmoothQuant + activation-aware GPTQ, W8A8 INT8 (v3)",
// sections "Recipe" and "Serving": INT8 x INT8 with per-token x per-channel
// scales, bf16 out): acc[m,n] = sum_k x[m,k] w[n,k] in int32, then
// y = bf16_rne(((float)acc * s_tok[m]) * s_ch[n]) (fp16 for EPI_CHANNEL_F16).
//
// Why this tile: a compute unit moves operands from L2 into LDS at a fixed
// rate (about 37 bytes per clock measured, the same with 32 or 256 units
// busy), and a 256 x 256 tile's loads take most of its MFMA time.  A
// 256 x 384 tile loads 17% fewer bytes per product and reads 7 fragments per
// 12 MFMAs instead of 6 per 8; at 8192 x 15360 it also splits into 1,280
// tiles, five per unit with no partly filled last wave.  Two 128-deep
// stages of (256 + 384) rows x 128 bytes fill the 160 KB of LDS.  Eight
// waves (two per SIMD) each own 128 tokens x 96 channels: 12 accumulator
// blocks, 192 registers, so a wave keeps one fragment register set and the
// other wave on its SIMD runs while it waits for a read.
//
// Data movement and layout are those of gemm_i8_kernel: direct
// buffer_load_dwordx4 ... lds of 8 rows x 128 bytes per wave instruction,
// rows past the edge read as zero, chunk c of LDS row r at slot
// c ^ (r & 7) ^ ((r >> 3) & 1).  Schedule of a stage (four 32-deep
// sub-steps): the next stage's loads go out behind the MFMAs of sub-step 0;
// each sub-step's fragments are read behind the previous sub-step's MFMAs as
// they release the registers; after sub-step 3 the wave waits for its loads
// of the next stage, and one barrier publishes that stage and frees this
// one.
#pragma once

#include "gemm_i8.hpp"

namespace q8 {

constexpr int BIG_BM = 256, BIG_BN = 384;

template <int EPI_>
__global__ __launch_bounds__(512) void gemm_big_kernel(GemmArgs p) {
    constexpr int EPI = epi_base(EPI_);
    constexpr bool OUT_F16 = EPI_ != EPI;
    static_assert(EPI == EPI_CHANNEL || EPI == EPI_I32, "per-channel or raw int32 epilogue");
    constexpr int BM = BIG_BM, BN = BIG_BN, WM = 2, WN = 4, NW = WM * WN, GM = 8, BK = 128;
    constexpr int WTM = BM / WM, WTN = BN / WN;  // tokens x channels per wave
    constexpr int TM = WTM / 32, TN = WTN / 32;
    constexpr int XIW = BM / 8 / NW, WIW = BN / 8 / NW;  // 8-row direct loads per wave and stage
    constexpr int LPS = XIW + WIW;
    constexpr int NR = TM + TN;  // fragment reads per sub-step
    constexpr int NM = TM * TN;  // MFMAs per sub-step

    __shared__ __attribute__((aligned(1024))) int8_t lx0[BM * BK];
    __shared__ __attribute__((aligned(1024))) int8_t lx1[BM * BK];
    __shared__ __attribute__((aligned(1024))) int8_t lw0[BN * BK];
    __shared__ __attribute__((aligned(1024))) int8_t lw1[BN * BK];

    const int M = p.M, N = p.N, K = p.K;
    const int nbm = (M + BM - 1) / BM, nbn = (N + BN - 1) / BN;
    const int id = xcd_remap(blockIdx.x, nbm * nbn);
    const int per_group = GM * nbn;
    const int first_m = (id / per_group) * GM;
    const int gsz = min(nbm - first_m, GM);
    const int tile_m = first_m + (id % per_group) % gsz;
    const int tile_n = (id % per_group) / gsz;
    const int m0 = tile_m * BM, n0 = tile_n * BN;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wid % WM, wn = wid / WM;
    const int hi = lane >> 5;

    // ---- direct loads: instruction i of wave wid fills rows 8 (wid XIW + i)
    // .. + 7; lane l writes slot l % 8 of row l / 8 of that group from global
    // chunk (l % 8) ^ (l / 8) ^ (parity of the 8-row group)
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(p.x, (uint32_t)((int64_t)M * p.ldx));
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(p.w, (uint32_t)((int64_t)N * p.ldw));
    const int lrow = lane >> 3, lslot = lane & 7;
    const int xv[2] = {lrow * (int)p.ldx + ((lslot ^ lrow) << 4), lrow * (int)p.ldx + ((lslot ^ lrow ^ 1) << 4)};
    const int wv[2] = {lrow * (int)p.ldw + ((lslot ^ lrow) << 4), lrow * (int)p.ldw + ((lslot ^ lrow ^ 1) << 4)};
    const int xs0 = (m0 + wid * XIW * 8) * (int)p.ldx;  // scalar row offsets
    const int ws0 = (n0 + wid * WIW * 8) * (int)p.ldw;

    auto issue = [&](int kt, int8_t* bx, int8_t* bw) __attribute__((always_inline)) {
        const int koff = kt * BK;
#pragma unroll
        for (int i = 0; i < XIW; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                xr, (Q8_LDS void*)(bx + (wid * XIW + i) * 1024), 16, xv[(wid * XIW + i) & 1],
                xs0 + i * 8 * (int)p.ldx + koff, 0, 0);
#pragma unroll
        for (int i = 0; i < WIW; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                wr, (Q8_LDS void*)(bw + (wid * WIW + i) * 1024), 16, wv[(wid * WIW + i) & 1],
                ws0 + i * 8 * (int)p.ldw + koff, 0, 0);
    };

    // ---- fragment reads: sub-step kk takes chunk 2 kk + hi of the lane's
    // row; the 32-row block b is b * 32 * BK further on (same slot pattern)
    int wbase[4], xbase[4];
    {
        const int rw0 = wn * WTN + (lane & 31), rx0 = wm * WTM + (lane & 31);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int ch = 2 * kk + hi;
            wbase[kk] = rw0 * BK + ((ch ^ lds_swizzle(rw0)) << 4);
            xbase[kk] = rx0 * BK + ((ch ^ lds_swizzle(rx0)) << 4);
        }
    }

    v16i acc[TM][TN];
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int b = 0; b < TN; ++b) acc[a][b] = v16i{};
    v4i fw[TN], fx[TM];

    auto read = [&](int kk, const int8_t* bx, const int8_t* bw) __attribute__((always_inline)) {
#pragma unroll
        for (int a = 0; a < TM; ++a) fx[a] = *reinterpret_cast<const v4i*>(bx + xbase[kk] + a * 32 * BK);
#pragma unroll
        for (int b = 0; b < TN; ++b) fw[b] = *reinterpret_cast<const v4i*>(bw + wbase[kk] + b * 32 * BK);
    };
    // token block a outer: fx[a] is free again after the TN MFMAs that use it
    auto mfma = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < NM; ++t) {
            const int a = t / TN, b = t % TN;
            acc[a][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fw[b], fx[a], acc[a][b], 0, 0, 0);
        }
    };

    auto stage = [&](int kt, const int8_t* cx, const int8_t* cw, int8_t* nx, int8_t* nw)
                     __attribute__((always_inline)) {
        issue(kt + 1, nx, nw);
        mfma();
        read(1, cx, cw);
        interleave<NM, NR, LPS>();
        __builtin_amdgcn_sched_barrier(0);
        mfma();
        read(2, cx, cw);
        interleave<NM, NR, 0>();
        __builtin_amdgcn_sched_barrier(0);
        mfma();
        read(3, cx, cw);
        interleave<NM, NR, 0>();
        __builtin_amdgcn_sched_barrier(0);
        mfma();
        __builtin_amdgcn_sched_barrier(0);
        wait_vm_lgkm0<0>();
        block_barrier();
        read(0, nx, nw);
        __builtin_amdgcn_sched_barrier(0);
    };

    const int KT = K / BK;
    issue(0, lx0, lw0);
    wait_vm_lgkm0<0>();
    block_barrier();
    read(0, lx0, lw0);
    int kt = 0;
    for (; kt + 2 <= KT; kt += 2) {
        stage(kt, lx0, lw0, lx1, lw1);
        stage(kt + 1, lx1, lw1, lx0, lw0);
    }
    if (kt < KT) stage(kt, lx0, lw0, lx1, lw1);
    // the last stage's loads (one stage past K, never read) have landed:
    // the hand-over waited for them

    // ---------------------------------------------------------- epilogue --
#pragma unroll
    for (int a = 0; a < TM; ++a) {
        const int j = m0 + wm * WTM + a * 32 + (lane & 31);  // token
        if (j >= M) continue;
        const float st = EPI == EPI_CHANNEL ? p.s_tok[j] : 0.0f;
#pragma unroll
        for (int b = 0; b < TN; ++b) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int ch = n0 + wn * WTN + b * 32 + g * 8 + hi * 4;
                if (ch >= N) continue;
                if constexpr (EPI == EPI_I32) {
                    const v4i o = {acc[a][b][g * 4 + 0], acc[a][b][g * 4 + 1], acc[a][b][g * 4 + 2],
                                   acc[a][b][g * 4 + 3]};
                    *reinterpret_cast<v4i*>(static_cast<int32_t*>(p.c) + (int64_t)j * p.ldc + ch) = o;
                } else {
                    float v[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float t = (float)acc[a][b][g * 4 + e] * st;
                        v[e] = t * p.s_w[ch + e];
                    }
                    v2u o;
                    o[0] = pack16x2<OUT_F16>(v[0], v[1]);
                    o[1] = pack16x2<OUT_F16>(v[2], v[3]);
                    *reinterpret_cast<v2u*>(static_cast<uint16_t*>(p.c) + (int64_t)j * p.ldc + ch) = o;
                }
            }
        }
    }
}

// 32-bit buffer offsets: channel rows reach n0 + 383 < N + 383, token rows
// m0 + 255, and the loads run one stage past K.
inline bool gemm_big_offsets_fit(const GemmArgs& p) {
    const int64_t lim = (int64_t)1 << 31;
    return ((int64_t)p.M + 256) * p.ldx + 256 < lim && ((int64_t)p.N + 384) * p.ldw + 256 < lim;
}

template <int EPI>
inline hipError_t launch_gemm_big(const GemmArgs& p, hipStream_t stream) {
    const int nbm = (p.M + BIG_BM - 1) / BIG_BM, nbn = (p.N + BIG_BN - 1) / BIG_BN;
    hipLaunchKernelGGL((gemm_big_kernel<EPI>), dim3(nbm * nbn), dim3(512), 0, stream, p);
    return hipGetLastError();
}

}  // namespace q8
