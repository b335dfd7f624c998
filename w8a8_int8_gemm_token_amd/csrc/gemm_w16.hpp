// gemm_w16.hpp -- the large-problem weight-only INT8 GEMM (W8A16) on
// 256-token x 320-channel tiles.
//
// It computes what gemm_i8_kernel's EPI_W8A16 / EPI_W8A16_F16 modes compute
// ("Qwen3.8-27B -- SmoothQuant + activation-aware GPTQ, W8A8 INT8 (v3)",
// section "Recipe": INT8 per-channel weights with 16-bit activations;
// "lued/Qwen3.8-27B-INT8-W8A16-MTP", section "Why W8A16 on Ampere": the
// weights are rebuilt for a 16-bit GEMM): y = rne16(s_ch[n] * acc), acc the
// fp32 MFMA sum of x[m,k] * w16(w[n,k]), w16 the exact bf16 (or fp16) value
// of the int8 code.
//
// Why this tile: a compute unit moves operands from L2 into LDS at about 37
// bytes per clock, and a 256 x 128 tile's loads (512 bytes of activations
// plus 128 of weights per K step) take longer than its bf16 MFMAs.  A
// 256 x 320 tile loads 48% fewer bytes per product; at 8192 x 5120 it gives
// 512 tiles, two whole waves of 256.  Two 64-deep stages of 256 x 128-byte
// activation rows and 320 x 128-byte 16-bit weight rows take 144 KB of LDS.
// Eight waves (two per SIMD) of 64 tokens x 160 channels keep 160 fp32
// accumulators and one fragment register set.
//
// Data movement: activations go straight to LDS (buffer_load_dwordx4 ...
// lds, 8 rows x 128 bytes per wave instruction); the int8 weights (320 rows x
// 64 bytes per stage) come through registers, 16-byte loads issued before
// the activation loads so that waiting for them leaves those in flight, and
// are converted exactly to 16-bit into the same swizzled layout (chunk c of
// row r at slot c ^ (r & 7) ^ ((r >> 3) & 1)).  A stage has four 16-deep
// sub-steps; each sub-step's fragments are read behind the previous one's
// MFMAs; at the hand-over the wave converts its weight loads into the next
// stage's slot, waits for its activation loads, and one barrier publishes
// that stage and frees this one.
#pragma once

#include "gemm_i8.hpp"

namespace q8 {

constexpr int W16B_BM = 256, W16B_BN = 320;

template <bool F16>
__global__ __launch_bounds__(512) void gemm_w16_kernel(GemmArgs p) {
    constexpr int BM = W16B_BM, BN = W16B_BN, WM = 4, WN = 2, NW = WM * WN, GM = 8;
    constexpr int BK = 128;  // LDS row bytes: 64 K elements of 16 bits
    constexpr int KS = 64;   // K elements per stage
    constexpr int WTM = BM / WM, WTN = BN / WN;  // 64 tokens x 160 channels per wave
    constexpr int TM = WTM / 32, TN = WTN / 32;
    constexpr int XIW = BM / 8 / NW;              // 8-row activation loads per wave and stage
    constexpr int WCH = BN * 4;                   // 16-byte weight chunks per stage (64 bytes a row)
    constexpr int WLC = (WCH + NW * 64 - 1) / (NW * 64);  // per thread (the last partly)
    constexpr int NR = TM + TN;
    constexpr int NM = TM * TN;
    static_assert(XIW * 8 * NW == BM, "load split");

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

    // ---- activation loads (p.x is addressed in bytes, ldx in bytes)
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(p.x, operand_extent(M, p.ldx, 2 * K));
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(p.w, operand_extent(N, p.ldw, K));
    const int lrow = lane >> 3, lslot = lane & 7;
    const int xv[2] = {lrow * (int)p.ldx + ((lslot ^ lrow) << 4), lrow * (int)p.ldx + ((lslot ^ lrow ^ 1) << 4)};
    const int xs0 = (m0 + wid * XIW * 8) * (int)p.ldx;

    v4i wreg[WLC];
    auto issue = [&](int kt, int8_t* bx) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < WLC; ++i) {
            const int c = tid + i * NW * 64, r = c >> 2, q = c & 3;
            if (i + 1 < WLC || c < WCH)
                wreg[i] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(
                                                      wr, lane_offset((n0 + r) * (int)p.ldw + q * 16, kt * KS), 0, 0));
        }
#pragma unroll
        for (int i = 0; i < XIW; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                xr, (Q8_LDS void*)(bx + (wid * XIW + i) * 1024), 16, lane_offset(xv[(wid * XIW + i) & 1],
                xs0 + i * 8 * (int)p.ldx + kt * BK), 0, 0, 0);
    };
    // the staged weights -> exact 16-bit values: 16 codes of row r, chunk q,
    // become the 16-bit chunks 2q and 2q + 1 of that row
    auto wstore = [&](int8_t* bw) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < WLC; ++i) {
            const int c = tid + i * NW * 64, r = c >> 2, q = c & 3;
            if (i + 1 < WLC || c < WCH) {
                const v2u a0 = i8x4_to_h16x4<F16>((u32)wreg[i][0]);
                const v2u a1 = i8x4_to_h16x4<F16>((u32)wreg[i][1]);
                const v2u a2 = i8x4_to_h16x4<F16>((u32)wreg[i][2]);
                const v2u a3 = i8x4_to_h16x4<F16>((u32)wreg[i][3]);
                const int f = lds_swizzle(r);
                *reinterpret_cast<v4u*>(bw + r * BK + (((2 * q) ^ f) << 4)) = v4u{a0[0], a0[1], a1[0], a1[1]};
                *reinterpret_cast<v4u*>(bw + r * BK + (((2 * q + 1) ^ f) << 4)) = v4u{a2[0], a2[1], a3[0], a3[1]};
            }
        }
    };

    // ---- fragments: sub-step kk takes chunk 2 kk + hi (8 values at
    // k = 16 kk + 8 hi) of the lane's row
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
    v16f acc[TM][TN];
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int b = 0; b < TN; ++b) acc[a][b] = v16f{};
    v4i fw[TN], fx[TM];
    // token blocks [a0, a1) of sub-step kk
    auto read_x = [&](int kk, const int8_t* bx, int a0, int a1) __attribute__((always_inline)) {
#pragma unroll
        for (int a = a0; a < a1; ++a) fx[a] = *reinterpret_cast<const v4i*>(bx + xbase[kk] + a * 32 * BK);
    };
    auto read = [&](int kk, const int8_t* bx, const int8_t* bw) __attribute__((always_inline)) {
        read_x(kk, bx, 0, TM);
#pragma unroll
        for (int b = 0; b < TN; ++b) fw[b] = *reinterpret_cast<const v4i*>(bw + wbase[kk] + b * 32 * BK);
    };
    // MFMAs [t0, t1) of a sub-step, token block a outer
    auto mfma = [&](int t0 = 0, int t1 = NM) __attribute__((always_inline)) {
#pragma unroll
        for (int t = t0; t < t1; ++t) {
            const int a = t / TN, b = t % TN;
            if constexpr (F16)
                acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, fw[b]),
                                                                   __builtin_bit_cast(v8h, fx[a]), acc[a][b], 0, 0, 0);
            else
                acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, fw[b]),
                                                                    __builtin_bit_cast(v8bf, fx[a]), acc[a][b], 0, 0, 0);
        }
    };

    auto stage = [&](int kt, const int8_t* cx, const int8_t* cw, int8_t* nx, int8_t* nw)
                     __attribute__((always_inline)) {
        issue(kt + 1, nx);
        mfma();
        read(1, cx, cw);
        interleave<NM, NR, WLC + XIW>();
        __builtin_amdgcn_sched_barrier(0);
        mfma();
        read(2, cx, cw);
        interleave<NM, NR, 0>();
        __builtin_amdgcn_sched_barrier(0);
        mfma();
        read(3, cx, cw);
        interleave<NM, NR, 0>();
        __builtin_amdgcn_sched_barrier(0);
        // sub-step 3 in two halves around the hand-over (as in
        // gemm_big_kernel): token block 0, the weight conversion and the
        // barrier, then the next stage's block-0 fragments behind the MFMAs
        // of token block 1, then the rest
        mfma(0, NM / 2);
        __builtin_amdgcn_sched_barrier(0);
        wait_vm_lgkm0<XIW>();  // this thread's weight loads landed (issued first)
        wstore(nw);
        wait_vm_lgkm0<0>();
        block_barrier();
        read_x(0, nx, 0, TM / 2);
        mfma(NM / 2, NM);
        read_x(0, nx, TM / 2, TM);
#pragma unroll
        for (int b = 0; b < TN; ++b) fw[b] = *reinterpret_cast<const v4i*>(nw + wbase[0] + b * 32 * BK);
        __builtin_amdgcn_sched_barrier(0);
    };

    const int KT = K / KS;
    issue(0, lx0);
    wait_vm_lgkm0<0>();
    wstore(lw0);
    wait_vm_lgkm0<0>();
    block_barrier();
    read(0, lx0, lw0);
    int kt = 0;
    for (; kt + 2 <= KT; kt += 2) {
        stage(kt, lx0, lw0, lx1, lw1);
        stage(kt + 1, lx1, lw1, lx0, lw0);
    }
    if (kt < KT) stage(kt, lx0, lw0, lx1, lw1);

    // ---------------------------------------------------------- epilogue --
    // The outputs leave through LDS in whole 128-byte lines (stored straight
    // from the MFMA layout each instruction would write 16-byte pieces of 32
    // rows).  One pass per 32-token block a: the rows of wave rows 0-1 in one
    // weight stage buffer and those of wave rows 2-3 in the other (64 rows x
    // 320 channels, 40 KB each).  Same values and rounding as a direct
    // store.
    constexpr int RB = BN * 2;    // 640 bytes per staged row
    constexpr int CPR = RB / 16;  // 40 chunks of 16 bytes
    static_assert(64 * RB <= BN * BK && (RB / 8) % 16 == 0 && WM == 4, "staging layout");
    wait_vm_lgkm0<0>();
    block_barrier();  // every wave is done with the stage buffers
    int8_t* const wbuf = (wm >> 1) ? lw1 : lw0;
#pragma unroll
    for (int a = 0; a < TM; ++a) {
        const int r = (wm & 1) * 32 + (lane & 31);  // staged row
#pragma unroll
        for (int b = 0; b < TN; ++b) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int c8 = wn * (WTN / 4) + b * 8 + g * 2 + hi;  // 8-byte unit in the row
                const int ch = min(n0 + 4 * c8, N - 4);
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = p.s_w[ch + e] * acc[a][b][g * 4 + e];
                v2u o;
                o[0] = pack16x2<F16>(v[0], v[1]);
                o[1] = pack16x2<F16>(v[2], v[3]);
                // unit c8 of row r at c8 ^ ((r >> 1) & 15) (rows of 160
                // dwords alternate between the two bank halves): the 32 rows
                // a write instruction touches fall in distinct banks
                *reinterpret_cast<v2u*>(wbuf + r * RB + ((c8 ^ ((r >> 1) & 15)) << 3)) = o;
            }
        }
        wait_vm_lgkm0<63>();  // LDS writes done (stores still in flight)
        block_barrier();
#pragma unroll
        for (int i = 0; i < 2 * 64 * CPR / (NW * 64); ++i) {
            const int idx = i * NW * 64 + tid;
            const int h = idx / (64 * CPR);
            const int rr = (idx / CPR) % 64, q = idx % CPR;
            const int sw = (rr >> 1) & 15;
            const int base = (2 * q) ^ (sw & ~1);
            v4u d = *reinterpret_cast<const v4u*>((h ? lw1 : lw0) + rr * RB + (base << 3));
            if (sw & 1) d = v4u{d[2], d[3], d[0], d[1]};
            const int jj = m0 + (2 * h + (rr >> 5)) * WTM + a * 32 + (rr & 31);
            const int cc = n0 + q * 8;
            if (jj < M && cc < N)
                __builtin_nontemporal_store(d, reinterpret_cast<v4u*>(static_cast<uint16_t*>(p.c) +
                                                                       (int64_t)jj * p.ldc + cc));
        }
        if (a + 1 < TM) {
            wait_vm_lgkm0<63>();
            block_barrier();  // the reads are done before the next pass writes
        }
    }
}

// 32-bit buffer offsets: weight rows reach n0 + 319 < N + 319, activation
// rows m0 + 255, and the loads run one stage past K.
inline bool gemm_w16_offsets_fit(const GemmArgs& p) {
    const int64_t lim = (int64_t)1 << 31;
    return ((int64_t)p.M + 256) * p.ldx + 256 < lim && ((int64_t)p.N + 320) * p.ldw + 256 < lim;
}

template <bool F16>
inline hipError_t launch_gemm_w16(const GemmArgs& p, hipStream_t stream) {
    const int nbm = (p.M + W16B_BM - 1) / W16B_BM, nbn = (p.N + W16B_BN - 1) / W16B_BN;
    hipLaunchKernelGGL((gemm_w16_kernel<F16>), dim3(nbm * nbn), dim3(512), 0, stream, p);
    return hipGetLastError();
}

}  // namespace q8
