// gemm_i8.hpp -- tiled INT8 x INT8 -> INT32 GEMM on CDNA4 int8 MFMA
// (v_mfma_i32_32x32x32_i8), with the scale epilogues of the W8A8 layer.
//
//   acc[m,n] = sum_k x[m,k] * w[n,k]          exact int32
//   EPI_CHANNEL: y = bf16_rne(((float)acc * s_tok[m]) * s_ch[n])
//   EPI_GROUP:   per 128-wide K block g (ascending), acc_g exact int32 and
//                f = fmaf((float)acc_g, s_grp[n,g], f); y = bf16_rne(f*s_tok[m])
//   EPI_I32:     raw int32 acc
// "Qwen3.8-27B -- SmoothQuant + activation-aware GPTQ, W8A8 INT8 (v3)",
// sections "Recipe" and "Serving" (INT8 x INT8 with per-token x per-channel
// scales, bf16 out); "Qwen3.8-27B-GPTQ-INT8-W8A8-GS128", "Quantization
// details" (one weight scale per 128-wide K block).
//
// Design (gfx950): a workgroup owns a BM (tokens) x BN (channels) output
// tile; WM x WN waves each own a (BM/WM) x (BN/WN) register tile of 32x32
// MFMA blocks.  The weight tile feeds the MFMA A operand (32 channels) and
// the activation tile the B operand (32 tokens), so a lane's accumulators
// hold four consecutive channels of one token: the epilogue stores 8-byte
// bf16 quads along N.  K advances BK bytes per stage through a double-
// buffered LDS tile (rows padded by 16 bytes so the 16-byte fragment reads of
// 32 rows hit distinct banks); the next stage's global loads are in flight
// in registers while the current stage's MFMAs run.  Because an integer sum
// is order-free, the K order inside one MFMA only has to agree between the
// two operands: lane l of both fragments carries the 16 bytes at
// k = 32*kk + 16*(l/32) of its row.
#pragma once

#include "q8_device.hpp"

namespace q8 {

enum { EPI_I32 = 0, EPI_CHANNEL = 1, EPI_GROUP = 2 };

struct GemmArgs {
    const int8_t* x;  // activations (tokens) [M, ldx]
    int64_t ldx;
    const int8_t* w;  // weights (channels) [N, ldw]
    int64_t ldw;
    const float* s_tok;  // [M]
    const float* s_w;    // [N] per channel, or [N, K/128] per group
    void* c;             // [M, ldc] bf16 bits, or int32
    int64_t ldc;
    int M, N, K;
};

template <int BM, int BN, int BK, int WM, int WN, int EPI, int GM>
__global__ __launch_bounds__(WM* WN * 64) void gemm_i8_kernel(GemmArgs p) {
    constexpr int NT = WM * WN * 64;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int TM = WTM / 32, TN = WTN / 32;
    constexpr int LDSW = BK + 16;  // padded row stride (bytes)
    constexpr int CPR = BK / 16;   // 16-byte chunks per row and stage
    constexpr int XCH = BM * CPR / NT;
    constexpr int WCH = BN * CPR / NT;
    constexpr int KK = BK / 32;
    static_assert(TM * 32 * WM == BM && TN * 32 * WN == BN, "tile shape");
    static_assert(XCH * NT == BM * CPR && WCH * NT == BN * CPR, "load split");
    static_assert(EPI != EPI_GROUP || (BK == 128 && BN <= NT), "group tiles");

    __shared__ __attribute__((aligned(16))) int8_t lx[2][BM * LDSW];
    __shared__ __attribute__((aligned(16))) int8_t lw[2][BN * LDSW];
    __shared__ __attribute__((aligned(16))) float lsg[2][EPI == EPI_GROUP ? BN : 4];

    const int M = p.M, N = p.N, K = p.K;
    const int nbm = (M + BM - 1) / BM, nbn = (N + BN - 1) / BN;
    const int id = xcd_remap(blockIdx.x, nbm * nbn);
    const int per_group = GM * nbn;
    const int first_m = (id / per_group) * GM;
    const int gsz = min(nbm - first_m, GM);
    const int tile_m = first_m + (id % per_group) % gsz;
    const int tile_n = (id % per_group) / gsz;
    const int m0 = tile_m * BM, n0 = tile_n * BN;

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int wm = wid % WM, wn = wid / WM;

    // This thread's global chunks: rows past the matrix edge are clamped to
    // the last row (their products are computed and never stored).
    const int8_t* xs[XCH];
    int xo[XCH];
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
        const int cidx = tid + i * NT, r = cidx / CPR, q = cidx % CPR;
        xs[i] = p.x + (int64_t)min(m0 + r, M - 1) * p.ldx + q * 16;
        xo[i] = r * LDSW + q * 16;
    }
    const int8_t* ws[WCH];
    int wo[WCH];
#pragma unroll
    for (int i = 0; i < WCH; ++i) {
        const int cidx = tid + i * NT, r = cidx / CPR, q = cidx % CPR;
        ws[i] = p.w + (int64_t)min(n0 + r, N - 1) * p.ldw + q * 16;
        wo[i] = r * LDSW + q * 16;
    }
    const int G = K >> 7;
    const float* sg_src = p.s_w + (int64_t)min(n0 + tid, N - 1) * G;

    uint4 rx[XCH], rw[WCH];
    float rsg = 0.0f;

    v16i acc[TM][TN];
    v16f facc[EPI == EPI_GROUP ? TM : 1][EPI == EPI_GROUP ? TN : 1];
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int b = 0; b < TN; ++b) acc[a][b] = v16i{};
    if constexpr (EPI == EPI_GROUP) {
#pragma unroll
        for (int a = 0; a < TM; ++a)
#pragma unroll
            for (int b = 0; b < TN; ++b) facc[a][b] = v16f{};
    }

    auto gload = [&](int kt) {
        const int64_t koff = (int64_t)kt * BK;
#pragma unroll
        for (int i = 0; i < XCH; ++i) rx[i] = *reinterpret_cast<const uint4*>(xs[i] + koff);
#pragma unroll
        for (int i = 0; i < WCH; ++i) rw[i] = *reinterpret_cast<const uint4*>(ws[i] + koff);
        if constexpr (EPI == EPI_GROUP) {
            if (tid < BN) rsg = sg_src[kt];
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < XCH; ++i) *reinterpret_cast<uint4*>(&lx[buf][xo[i]]) = rx[i];
#pragma unroll
        for (int i = 0; i < WCH; ++i) *reinterpret_cast<uint4*>(&lw[buf][wo[i]]) = rw[i];
        if constexpr (EPI == EPI_GROUP) {
            if (tid < BN) lsg[buf][tid] = rsg;
        }
    };

    const int frow = lane & 31, fk = (lane >> 5) * 16;
    auto compute = [&](int buf) {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            v4i fw[TN], fx[TM];
#pragma unroll
            for (int b = 0; b < TN; ++b)
                fw[b] = *reinterpret_cast<const v4i*>(
                    &lw[buf][(wn * WTN + b * 32 + frow) * LDSW + kk * 32 + fk]);
#pragma unroll
            for (int a = 0; a < TM; ++a)
                fx[a] = *reinterpret_cast<const v4i*>(
                    &lx[buf][(wm * WTM + a * 32 + frow) * LDSW + kk * 32 + fk]);
#pragma unroll
            for (int a = 0; a < TM; ++a)
#pragma unroll
                for (int b = 0; b < TN; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fw[b], fx[a], acc[a][b], 0, 0, 0);
        }
        if constexpr (EPI == EPI_GROUP) {
            // fold this 128-wide group into the fp32 accumulators, ascending g
#pragma unroll
            for (int b = 0; b < TN; ++b) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const v4f sc = *reinterpret_cast<const v4f*>(
                        &lsg[buf][wn * WTN + b * 32 + g * 8 + (lane >> 5) * 4]);
#pragma unroll
                    for (int a = 0; a < TM; ++a)
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            facc[a][b][g * 4 + e] = __builtin_fmaf(
                                (float)acc[a][b][g * 4 + e], sc[e], facc[a][b][g * 4 + e]);
                }
#pragma unroll
                for (int a = 0; a < TM; ++a) acc[a][b] = v16i{};
            }
        }
    };

    const int KT = K / BK;
    gload(0);
    lstore(0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < KT) gload(kt + 1);
        compute(cur);
        if (kt + 1 < KT) lstore(cur ^ 1);
        __syncthreads();
    }

    // ---------------------------------------------------------- epilogue --
#pragma unroll
    for (int a = 0; a < TM; ++a) {
        const int j = m0 + wm * WTM + a * 32 + (lane & 31);  // token
        if (j >= M) continue;
        const float st = (EPI == EPI_I32) ? 0.0f : p.s_tok[j];
#pragma unroll
        for (int b = 0; b < TN; ++b) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int ch = n0 + wn * WTN + b * 32 + g * 8 + (lane >> 5) * 4;
                if (ch >= N) continue;
                if constexpr (EPI == EPI_I32) {
                    int4 o;
                    o.x = acc[a][b][g * 4 + 0];
                    o.y = acc[a][b][g * 4 + 1];
                    o.z = acc[a][b][g * 4 + 2];
                    o.w = acc[a][b][g * 4 + 3];
                    *reinterpret_cast<int4*>(static_cast<int32_t*>(p.c) + (int64_t)j * p.ldc + ch) = o;
                } else {
                    float v[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        if constexpr (EPI == EPI_CHANNEL) {
                            float t = (float)acc[a][b][g * 4 + e] * st;
                            v[e] = t * p.s_w[ch + e];
                        } else {
                            v[e] = facc[a][b][g * 4 + e] * st;
                        }
                    }
                    uint2 o;
                    o.x = pack_bf16x2(v[0], v[1]);
                    o.y = pack_bf16x2(v[2], v[3]);
                    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.c) + (int64_t)j * p.ldc + ch) = o;
                }
            }
        }
    }
}

template <int BM, int BN, int BK, int WM, int WN, int EPI, int GM>
inline hipError_t launch_gemm_i8(const GemmArgs& p, hipStream_t stream) {
    const int nbm = (p.M + BM - 1) / BM, nbn = (p.N + BN - 1) / BN;
    hipLaunchKernelGGL((gemm_i8_kernel<BM, BN, BK, WM, WN, EPI, GM>), dim3(nbm * nbn),
                       dim3(WM * WN * 64), 0, stream, p);
    return hipGetLastError();
}

}  // namespace q8
