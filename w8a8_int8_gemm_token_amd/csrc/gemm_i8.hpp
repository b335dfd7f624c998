// gemm_i8.hpp -- INT8 x INT8 -> INT32 GEMM on CDNA4 int8 MFMA
// (v_mfma_i32_32x32x32_i8) with the scale epilogues of the W8A8 layer.
//
//   acc[m,n] = sum_k x[m,k] * w[n,k]                       exact int32
//   EPI_CHANNEL: y = bf16_rne(((float)acc * s_tok[m]) * s_ch[n])
//   EPI_GROUP:   for each 128-wide K block g in ascending order, the exact
//                int32 block sum p_g is folded as f = fmaf((float)p_g,
//                s_grp[n,g], f); y = bf16_rne(f * s_tok[m])
//   EPI_GROUP_ACT: as EPI_GROUP with one activation scale per (token,
//                128-wide K block) as well: f = fmaf((float)p_g,
//                fl(s_x[m,g] * s_w[n,g]), f); y = bf16_rne(f)
//   EPI_FP8_BLOCK: FP8 (E4M3) operands on v_mfma_f32_32x32x64_f8f6f4, one
//                activation scale per (token, 128-wide K block) and one
//                weight scale per [128,128] block: each block's fp32 partial
//                P_g is folded as f = fmaf(P_g, fl(s_x[m,g] * s_w[n/128,g]),
//                f) in ascending g; y = bf16_rne(f)
//   EPI_CHANNEL_F16, EPI_GROUP_ACT_F16: as EPI_CHANNEL and EPI_GROUP_ACT
//                with fp16 (RNE) outputs
//   EPI_W8A16_F16: EPI_W8A16 with fp16 activations (v_mfma_f32_32x32x16_f16)
//                and fp16 outputs
//   EPI_W8A16:   bf16 activations (x, ldx in bytes) times int8 weights on
//                v_mfma_f32_32x32x16_bf16: y = bf16_rne(s_ch[n] * acc), acc
//                the fp32 MFMA sum of x[m,k] * bf16(w[n,k])
//   EPI_I32:     the raw int32 acc
//   EPI_W16_PART, EPI_W16_PART_F16: EPI_W8A16 (bf16 or fp16 activations)
//                without the scale: the raw fp32 acc
// Split K: with p.kz > 0, workgroup row blockIdx.y sums only K elements
// [blockIdx.y * kz, min(K, (blockIdx.y + 1) * kz)) and writes its raw
// partial (EPI_I32, EPI_W16_PART*) to plane blockIdx.y, p.plane elements
// after the previous one; a separate kernel sums the planes and applies the
// epilogue.  Only these raw epilogues split.
// "Qwen3.8-27B -- SmoothQuant + activation-aware GPTQ, W8A8 INT8 (v3)",
// sections "Recipe" and "Serving" (INT8 x INT8 with per-token x per-channel
// scales, bf16 out); "Qwen3.8-27B-GPTQ-INT8-W8A8-GS128", "Quantization
// details" (one weight scale per 128-wide K block); "Qwen3.8-27B -- FP8
// block + AWQ", "Recipe" (FP8 [128,128] block weights, dynamic per-group
// activations).
//
// Tiling: a workgroup owns a BM (tokens) x BN (channels) output tile; WM x WN
// waves each own a (BM/WM) x (BN/WN) register tile of 32x32 MFMA blocks.  The
// weight tile feeds the MFMA A operand (32 channels) and the activation tile
// the B operand (32 tokens), so a lane's accumulators hold four consecutive
// channels of one token and the epilogue stores 8-byte bf16 quads along N.
// Because an integer sum is order-free, the K order inside one MFMA only has
// to agree between the two operands: lane l of both fragments carries the 16
// bytes at k = 32*kk + 16*(l/32) of its row.
//
// Data movement (BK = 128 bytes of K per stage):
//  * global -> LDS with buffer_load_dwordx4 ... lds (direct to LDS, no VGPR
//    staging).  Every wave instruction moves 8 rows x 128 contiguous bytes
//    (whole 128-byte lines).  One buffer resource per operand, over exactly
//    the bytes the caller guarantees ((rows - 1) * ld + K); the whole offset
//    of every load is its vector offset, the part the hardware checks
//    against that range (a scalar offset is added after the check).  So a
//    row past the matrix edge, and the stage after K that the last stage
//    prefetches, read as zero without touching memory (their products are
//    never stored).  A lane keeps two vector offsets per operand and adds
//    the row/stage part, a wave-uniform value, per load.
//  * LDS rows are 128 bytes; the 16-byte chunk c of row r is stored at slot
//    c ^ f(r), f(r) = (r & 7) ^ ((r >> 3) & 1).  The MFMA fragment reads
//    (one 16-byte chunk per lane, 32 consecutive rows) are then free of bank
//    conflicts for 32- and 64-bank LDS, and since f ignores row bits >= 4 the
//    fragment of each further 32-row block is an immediate offset away.
//  * two LDS stages, held in distinct LDS objects so that the compiler can
//    tell the stage being filled from the one being read (it would otherwise
//    drain every in-flight direct load before each LDS read).
// Schedule of one stage (four 32-deep sub-steps, two fragment register
// sets): the fragments of sub-step s+1 are read while the MFMAs of sub-step
// s run (sched_group_barrier puts the LDS reads, and in sub-step 0 the next
// stage's direct loads, between the MFMAs); halfway through sub-step 3 the
// wave waits for its own direct loads of the next stage and all its LDS
// reads of this one, one barrier publishes the next stage and frees this
// one, and the first fragments of the next stage are read while the last
// MFMAs of this stage drain.  One barrier per stage.
#pragma once

#include <type_traits>

#include "q8_device.hpp"

#define Q8_LDS __attribute__((address_space(3)))

namespace q8 {

enum { EPI_I32 = 0, EPI_CHANNEL = 1, EPI_GROUP = 2, EPI_GROUP_ACT = 3, EPI_FP8_BLOCK = 4,
       EPI_CHANNEL_F16 = 5, EPI_GROUP_ACT_F16 = 6, EPI_W8A16 = 7, EPI_W8A16_F16 = 8,
       EPI_W16_PART = 9, EPI_W16_PART_F16 = 10 };

// The _F16 epilogues are EPI_CHANNEL, EPI_GROUP_ACT and EPI_W8A16 with fp16
// outputs (EPI_W8A16_F16: fp16 activations as well).
constexpr int epi_base(int e) {
    return e == EPI_CHANNEL_F16 ? EPI_CHANNEL
           : e == EPI_GROUP_ACT_F16 ? EPI_GROUP_ACT
           : e == EPI_W8A16_F16 ? EPI_W8A16
           : e == EPI_W16_PART_F16 ? EPI_W16_PART : e;
}

struct GemmArgs {
    const int8_t* x;  // activations (tokens) [M, ldx]
    int64_t ldx;
    const int8_t* w;  // weights (channels) [N, ldw]
    int64_t ldw;
    const float* s_tok;  // [M]; EPI_GROUP_ACT, EPI_FP8_BLOCK: [M, K/128] per (token, block)
    const float* s_w;    // [N] per channel, [N, K/128] per group, or [N/128, K/128] per block
    void* c;             // [M, ldc] bf16 (fp16 for the _F16 epilogues) bits, or int32
    int64_t ldc;
    int M, N, K;
    int kz;         // split K: K elements per workgroup row (blockIdx.y); 0 = all of K
    int64_t plane;  // split K: elements between two partial planes of c
};

// s_waitcnt with vmcnt = N and lgkmcnt = 0 (expcnt untouched).
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

// Workgroup barrier without the implicit release fence of __syncthreads
// (which would drain every in-flight global load); the empty asm statements
// keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void block_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// sched_group_barrier masks
constexpr int SG_MFMA = 0x008, SG_VMEM_RD = 0x020, SG_DS_RD = 0x100;

// Schedule of one region: N_MFMA MFMAs, with N_DS LDS reads and N_VM direct
// loads spread evenly behind them.
template <int N_MFMA, int N_DS, int N_VM, int I = 0>
__device__ __forceinline__ void interleave() {
    if constexpr (I < N_MFMA) {
        __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
        constexpr int v = N_VM * (I + 1) / N_MFMA - N_VM * I / N_MFMA;
        constexpr int d = N_DS * (I + 1) / N_MFMA - N_DS * I / N_MFMA;
        if constexpr (v > 0) __builtin_amdgcn_sched_group_barrier(SG_VMEM_RD, v, 0);
        if constexpr (d > 0) __builtin_amdgcn_sched_group_barrier(SG_DS_RD, d, 0);
        interleave<N_MFMA, N_DS, N_VM, I + 1>();
    }
}

__device__ __forceinline__ int lds_swizzle(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// Buffer resource over `bytes` bytes at p (raw buffer, no stride).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// Bytes of a row-major operand that the caller guarantees: rows - 1 full
// leading dimensions, then the last row's kbytes.  A resource over exactly
// this range turns every read past the last row's K-th byte -- the tile
// rows past the edge, and the prefetch of the stage after K on the last
// row -- into a zero read that touches no memory.  (rows * ld would not:
// for a view that starts inside its rows, such as a K slice at a column
// offset, rows * ld from that start runs past the end of the allocation.)
__device__ __forceinline__ uint32_t operand_extent(int rows, int64_t ld, int kbytes) {
    return rows > 0 ? (uint32_t)((int64_t)(rows - 1) * ld + kbytes) : 0u;
}

// Vector offset of one buffer load: the lane's part v plus a wave-uniform
// part u (row and stage).  The empty asm keeps u an opaque scalar here, so
// the compiler adds it right at the load instead of keeping one hoisted
// vector sum per load alive across the K loop.
__device__ __forceinline__ int lane_offset(int v, int u) {
    asm volatile("" : "+s"(u));
    return v + u;
}

template <int BM, int BN, int WM, int WN, int EPI_, int GM>
__global__ __launch_bounds__(WM* WN * 64) void gemm_i8_kernel(GemmArgs p) {
    constexpr int EPI = epi_base(EPI_);
    constexpr bool OUT_F16 = EPI_ != EPI;
    constexpr int BK = 128;
    constexpr int NW = WM * WN;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int TM = WTM / 32, TN = WTN / 32;
    constexpr bool W16 = EPI == EPI_W8A16 || EPI == EPI_W16_PART;
    constexpr bool RAW = EPI == EPI_I32 || EPI == EPI_W16_PART;  // raw partial sums out
    // K elements per stage: 128 bytes of LDS row hold 128 codes or 64 bf16
    constexpr int KS = W16 ? 64 : 128;
    constexpr int XIW = BM / 8 / NW;                // 8-row direct loads per wave and stage
    constexpr int WIW = W16 ? 0 : BN / 8 / NW;
    // W8A16: the int8 weight tile (BN rows x 64 bytes) comes through registers,
    // WLC 16-byte loads per thread, and is written to LDS as bf16
    constexpr int WLC = W16 ? BN * 4 / (NW * 64) : 0;
    constexpr bool F8 = EPI == EPI_FP8_BLOCK;
    constexpr bool GRP = EPI == EPI_GROUP || EPI == EPI_GROUP_ACT;
    constexpr bool FOLD = GRP || F8;                       // per-block fp32 fold
    constexpr bool ACT = EPI == EPI_GROUP_ACT || F8;       // per-(token, block) scales
    constexpr int SGI = GRP ? BN / 64 : 0;             // 64-scale weight loads per stage
    constexpr int SXI = ACT ? (BM + 63) / 64 : 0;      // 64-scale activation loads per stage
    constexpr int XOFF = GRP ? BN : 0;                 // activation scales in a stage's block
    constexpr int LPS = XIW + WIW + WLC + (SGI + NW - 1) / NW + (SXI + NW - 1) / NW;
    constexpr int LSN = FOLD ? XOFF + SXI * 64 : 4;    // scale floats per stage
    constexpr int NR = (F8 ? 2 : 1) * (TM + TN);  // fragment reads (16 bytes) per sub-step
    constexpr int NM = TM * TN;  // MFMAs per sub-step
    constexpr int NM0 = NM / 2;  // MFMAs of sub-step 3 before the hand-over
    static_assert(TM * 32 * WM == BM && TN * 32 * WN == BN, "tile shape");
    static_assert(XIW * 8 * NW == BM && (W16 ? WLC * NW * 64 == BN * 4 : WIW * 8 * NW == BN), "load split");
    static_assert(!GRP || BN % 64 == 0, "group scales load 64 at a time");
    static_assert(!F8 || (WTN <= 128 && 128 % WTN == 0), "a wave's channels share one weight block");
    using AccT = std::conditional_t<F8 || W16, v16f, v16i>;
    using FragT = std::conditional_t<F8, v8i, v4i>;

    __shared__ __attribute__((aligned(1024))) int8_t lx0[BM * BK];
    __shared__ __attribute__((aligned(1024))) int8_t lx1[BM * BK];
    __shared__ __attribute__((aligned(1024))) int8_t lw0[BN * BK];
    __shared__ __attribute__((aligned(1024))) int8_t lw1[BN * BK];
    // per stage: the tile's BN weight block scales, then (EPI_GROUP_ACT) its
    // activation block scales
    __shared__ __attribute__((aligned(16))) float ls0[LSN];
    __shared__ __attribute__((aligned(16))) float ls1[LSN];

    const int M = p.M, N = p.N, K = p.K;
    // this workgroup's K range (the whole of K unless K is split)
    const int kz = RAW && p.kz > 0 ? p.kz : K;
    const int kb = blockIdx.y * kz;
    const int kn = min(kz, K - kb);
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

    // ---- direct loads: instruction i of wave wid fills rows
    // (wid*XIW + i)*8 .. +8 of the tile; lane l writes LDS slot l%8 of row
    // l/8 of that group, i.e. global chunk (l%8) ^ f(row), and f(row)
    // = (l/8) ^ (parity of the instruction's 8-row group).
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(p.x, operand_extent(M, p.ldx, W16 ? 2 * K : K));
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(p.w, operand_extent(N, p.ldw, K));
    const int G = K >> 7;
    const __amdgpu_buffer_rsrc_t sr = make_rsrc(p.s_w, GRP ? (uint32_t)((int64_t)N * G * 4) : 0u);
    const int lrow = lane >> 3, lslot = lane & 7;
    const int xv[2] = {lrow * (int)p.ldx + ((lslot ^ lrow) << 4),
                       lrow * (int)p.ldx + ((lslot ^ lrow ^ 1) << 4)};
    const int wv[2] = {lrow * (int)p.ldw + ((lslot ^ lrow) << 4),
                       lrow * (int)p.ldw + ((lslot ^ lrow ^ 1) << 4)};
    const int xs0 = (m0 + wid * XIW * 8) * (int)p.ldx;  // scalar row offsets
    const int ws0 = (n0 + wid * WIW * 8) * (int)p.ldw;
    const int sv = (n0 + lane) * G * 4;  // group scales: channel n0 + 64*i + lane
    const __amdgpu_buffer_rsrc_t sxr = make_rsrc(p.s_tok, (uint32_t)((int64_t)M * G * 4));
    const int svx = (m0 + lane) * G * 4;  // activation block scales: token m0 + 64*i + lane

    v4i wreg[W16 ? WLC : 1];
    auto issue = [&](int kt, int8_t* bx, int8_t* bw, float* bs) __attribute__((always_inline)) {
        const int koff = kt * BK + (W16 ? 2 : 1) * kb;  // activation bytes
        const int kwoff = kt * BK + kb;                  // int8 weight bytes (direct loads)
        if constexpr (W16) {  // first, so that a wait for them can leave the tile loads in flight
#pragma unroll
            for (int i = 0; i < WLC; ++i) {
                const int c = (int)threadIdx.x + i * NW * 64, r = c >> 2, q = c & 3;
                wreg[i] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(
                                                      wr, lane_offset((n0 + r) * (int)p.ldw + q * 16, kt * 64 + kb), 0, 0));
            }
        }
#pragma unroll
        for (int i = 0; i < XIW; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                xr, (Q8_LDS void*)(bx + (wid * XIW + i) * 1024), 16, lane_offset(xv[(wid * XIW + i) & 1],
                xs0 + i * 8 * (int)p.ldx + koff), 0, 0, 0);
#pragma unroll
        for (int i = 0; i < WIW; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                wr, (Q8_LDS void*)(bw + (wid * WIW + i) * 1024), 16, lane_offset(wv[(wid * WIW + i) & 1],
                ws0 + i * 8 * (int)p.ldw + kwoff), 0, 0, 0);
        if constexpr (SGI > 0) {
#pragma unroll
            for (int i = 0; i < (SGI + NW - 1) / NW; ++i) {
                const int j = wid + i * NW;  // 64-channel block of this load
                if (j < SGI)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(sr, (Q8_LDS void*)(bs + j * 64), 4,
                                                             lane_offset(sv, j * 64 * G * 4 + kt * 4), 0, 0, 0);
            }
        }
        if constexpr (SXI > 0) {
#pragma unroll
            for (int i = 0; i < (SXI + NW - 1) / NW; ++i) {
                const int j = wid + i * NW;
                if (j < SXI)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(sxr, (Q8_LDS void*)(bs + XOFF + j * 64), 4,
                                                             lane_offset(svx, j * 64 * G * 4 + kt * 4), 0, 0, 0);
            }
        }
    };

    // W8A16: the staged int8 weights of a stage -> exact bf16 (|q| <= 128) in
    // the swizzled LDS layout: 16 codes of row r, K chunk q, become the bf16
    // chunks 2q and 2q + 1 of that row.
    auto wstore = [&](int8_t* bw) __attribute__((always_inline)) {
        if constexpr (W16) {
#pragma unroll
            for (int i = 0; i < WLC; ++i) {
                const int c = (int)threadIdx.x + i * NW * 64, r = c >> 2, q = c & 3;
                const v2u a0 = i8x4_to_h16x4<OUT_F16>((u32)wreg[i][0]);
                const v2u a1 = i8x4_to_h16x4<OUT_F16>((u32)wreg[i][1]);
                const v2u a2 = i8x4_to_h16x4<OUT_F16>((u32)wreg[i][2]);
                const v2u a3 = i8x4_to_h16x4<OUT_F16>((u32)wreg[i][3]);
                const int f = lds_swizzle(r);
                *reinterpret_cast<v4u*>(bw + r * BK + (((2 * q) ^ f) << 4)) = v4u{a0[0], a0[1], a1[0], a1[1]};
                *reinterpret_cast<v4u*>(bw + r * BK + (((2 * q + 1) ^ f) << 4)) = v4u{a2[0], a2[1], a3[0], a3[1]};
            }
        }
    };

    // ---- fragment reads: 16-byte read i of 32-row block b sits at
    // base[i] + b*32*BK (f is the same for rows r and r + 32b).  INT8: read
    // i is sub-step i's fragment, chunk 2i + hi of the row.  FP8: sub-step kk
    // takes 32 bytes per lane, chunks 4kk + 2hi and 4kk + 2hi + 1 (reads 2kk
    // and 2kk + 1); both operands use the same chunks, so every product
    // pairs equal k.
    int wbase[4], xbase[4];
    {
        const int rw0 = wn * WTN + (lane & 31), rx0 = wm * WTM + (lane & 31);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int ch = F8 ? (i >> 1) * 4 + hi * 2 + (i & 1) : i * 2 + hi;
            wbase[i] = rw0 * BK + ((ch ^ lds_swizzle(rw0)) << 4);
            xbase[i] = rx0 * BK + ((ch ^ lds_swizzle(rx0)) << 4);
        }
    }

    AccT acc[TM][TN];
    v16f facc[FOLD ? TM : 1][FOLD ? TN : 1];
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int b = 0; b < TN; ++b) acc[a][b] = AccT{};
    if constexpr (FOLD) {
#pragma unroll
        for (int a = 0; a < TM; ++a)
#pragma unroll
            for (int b = 0; b < TN; ++b) facc[a][b] = v16f{};
    }
    FragT fw[2][TN], fx[2][TM];

    auto read = [&](int set, int kk, const int8_t* bx, const int8_t* bw) __attribute__((always_inline)) {
        if constexpr (F8) {
#pragma unroll
            for (int b = 0; b < TN; ++b) {
                const v4i lo = *reinterpret_cast<const v4i*>(bw + wbase[2 * kk] + b * 32 * BK);
                const v4i hi8 = *reinterpret_cast<const v4i*>(bw + wbase[2 * kk + 1] + b * 32 * BK);
                fw[set][b] = v8i{lo[0], lo[1], lo[2], lo[3], hi8[0], hi8[1], hi8[2], hi8[3]};
            }
#pragma unroll
            for (int a = 0; a < TM; ++a) {
                const v4i lo = *reinterpret_cast<const v4i*>(bx + xbase[2 * kk] + a * 32 * BK);
                const v4i hi8 = *reinterpret_cast<const v4i*>(bx + xbase[2 * kk + 1] + a * 32 * BK);
                fx[set][a] = v8i{lo[0], lo[1], lo[2], lo[3], hi8[0], hi8[1], hi8[2], hi8[3]};
            }
        } else {
#pragma unroll
            for (int b = 0; b < TN; ++b)
                fw[set][b] = *reinterpret_cast<const v4i*>(bw + wbase[kk] + b * 32 * BK);
#pragma unroll
            for (int a = 0; a < TM; ++a)
                fx[set][a] = *reinterpret_cast<const v4i*>(bx + xbase[kk] + a * 32 * BK);
        }
    };
    // FP8: `fresh` starts a block's partial (C = 0) instead of adding to acc
    auto mfma = [&](int set, int from, int to, bool fresh = false) __attribute__((always_inline)) {
#pragma unroll
        for (int t = from; t < to; ++t) {
            const int a = t / TN, b = t % TN;
            if constexpr (F8)  // A and B in E4M3 (format 0), no block exponents
                acc[a][b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    fw[set][b], fx[set][a], fresh ? AccT{} : acc[a][b], 0, 0, 0, 0, 0, 0);
            else if constexpr (W16 && OUT_F16)
                acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, fw[set][b]),
                                                                   __builtin_bit_cast(v8h, fx[set][a]),
                                                                   acc[a][b], 0, 0, 0);
            else if constexpr (W16)
                acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, fw[set][b]),
                                                                    __builtin_bit_cast(v8bf, fx[set][a]),
                                                                    acc[a][b], 0, 0, 0);
            else
                acc[a][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fw[set][b], fx[set][a], fresh ? AccT{} : acc[a][b],
                                                                  0, 0, 0);
        }
    };
    // EPI_GROUP: fold the stage's 128-wide block sums into the fp32
    // accumulators (the stage is group kt; groups arrive in ascending order)
    auto fold = [&](const float* bs, int kt) __attribute__((always_inline)) {
        if constexpr (F8) {
            // a wave's WTN channels lie in one 128-channel weight block
            const float sw = p.s_w[(int64_t)((n0 + wn * WTN) >> 7) * G + kt];
            float f[TM];
#pragma unroll
            for (int a = 0; a < TM; ++a) f[a] = bs[wm * WTM + a * 32 + (lane & 31)] * sw;
#pragma unroll
            for (int a = 0; a < TM; ++a)
#pragma unroll
                for (int b = 0; b < TN; ++b) {
#pragma unroll
                    for (int e = 0; e < 16; ++e) facc[a][b][e] = __builtin_fmaf(acc[a][b][e], f[a], facc[a][b][e]);
                }
        } else if constexpr (GRP) {
            float sx[TM];  // EPI_GROUP_ACT: block scale of this lane's token in block a
#pragma unroll
            for (int a = 0; a < TM; ++a) sx[a] = ACT ? bs[BN + wm * WTM + a * 32 + (lane & 31)] : 1.0f;
#pragma unroll
            for (int b = 0; b < TN; ++b) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const v4f sc = *reinterpret_cast<const v4f*>(bs + wn * WTN + b * 32 + g * 8 + hi * 4);
#pragma unroll
                    for (int a = 0; a < TM; ++a)
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            facc[a][b][g * 4 + e] = __builtin_fmaf(
                                (float)acc[a][b][g * 4 + e], ACT ? sx[a] * sc[e] : sc[e],
                                facc[a][b][g * 4 + e]);
                }
            }
        }
    };

    // One stage held in (cx, cw, cs); the next stage goes to (nx, nw, ns).
    // The last stage also issues loads for a stage K..K+127 that is never
    // read: with buffer loads those offsets stay inside the operand's rows or
    // fall outside the resource and read as zero, so the loop needs no tail.
    auto stage = [&](int kt, const int8_t* cx, const int8_t* cw, const float* cs, int8_t* nx,
                     int8_t* nw, float* ns) __attribute__((always_inline)) {
        if constexpr (F8) {
            // two 64-deep sub-steps: MFMAs on set 0 with the next stage's
            // direct loads and set 1 <- kk 1 behind them; then set 1, the
            // fold of this stage's block, and the hand-over
            issue(kt + 1, nx, nw, ns);
            read(1, 1, cx, cw);
            mfma(0, 0, NM, true);
            interleave<NM, NR, LPS>();
            __builtin_amdgcn_sched_barrier(0);
            mfma(1, 0, NM);
            fold(cs, kt);
            __builtin_amdgcn_sched_barrier(0);
            wait_vm_lgkm0<0>();
            block_barrier();
            read(0, 0, nx, nw);
            __builtin_amdgcn_sched_barrier(0);
        } else {
            // sub-step 0: MFMAs on set 0 (a group's first: C = 0); next
            // stage's direct loads; set 1 <- kk 1
            issue(kt + 1, nx, nw, ns);
            read(1, 1, cx, cw);
            mfma(0, 0, NM, GRP);
            interleave<NM, NR, LPS>();
            __builtin_amdgcn_sched_barrier(0);
            // sub-step 1
            read(0, 2, cx, cw);
            mfma(1, 0, NM);
            interleave<NM, NR, 0>();
            __builtin_amdgcn_sched_barrier(0);
            // sub-step 2
            read(1, 3, cx, cw);
            mfma(0, 0, NM);
            interleave<NM, NR, 0>();
            __builtin_amdgcn_sched_barrier(0);
            // sub-step 3: part of the MFMAs, then the stage hand-over
            if constexpr (GRP) {
                // the group fold reads this stage's scales: do it before the
                // hand-over frees the stage
                mfma(1, 0, NM);
                fold(cs, kt);
                __builtin_amdgcn_sched_barrier(0);
                wait_vm_lgkm0<0>();
                block_barrier();
                read(0, 0, nx, nw);
                __builtin_amdgcn_sched_barrier(0);
            } else {
                mfma(1, 0, NM0);
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (W16) {  // this thread's weight loads landed: convert them into nw
                    wait_vm_lgkm0<XIW>();
                    wstore(nw);
                }
                wait_vm_lgkm0<0>();
                block_barrier();
                read(0, 0, nx, nw);
                mfma(1, NM0, NM);
                interleave<NM - NM0, NR, 0>();
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    const int KT = kn / KS;
    issue(0, lx0, lw0, ls0);
    wait_vm_lgkm0<0>();
    wstore(lw0);
    wait_vm_lgkm0<0>();
    block_barrier();
    read(0, 0, lx0, lw0);
    int kt = 0;
    for (; kt + 2 <= KT; kt += 2) {
        stage(kt, lx0, lw0, ls0, lx1, lw1, ls1);
        stage(kt + 1, lx1, lw1, ls1, lx0, lw0, ls0);
    }
    if (kt < KT) stage(kt, lx0, lw0, ls0, lx1, lw1, ls1);

    // ---------------------------------------------------------- epilogue --
    if constexpr (!RAW) {
        // 16-bit outputs leave through LDS in whole 128-byte lines (stored
        // straight from the MFMA layout each instruction would write 16-byte
        // pieces of 32 rows): one 32-token block of every wave row per pass,
        // WM*32 rows x BN channels, alternating between two stage buffers
        // that hold it.  Same values and rounding as a direct store.
        constexpr bool USE_W = WM * 32 * BN * 2 <= BN * BK;
        static_assert(USE_W || WM * 32 * BN * 2 <= BM * BK, "a pass fits a stage buffer");
        static_assert(BN % 128 == 0, "rows of whole 32-unit swizzle groups");
        constexpr int RB = BN * 2;    // bytes per staged row
        constexpr int CPR = RB / 16;  // 16-byte chunks per row
        wait_vm_lgkm0<0>();
        block_barrier();  // every wave is done with the stage buffers
#pragma unroll
        for (int a = 0; a < TM; ++a) {
            int8_t* buf = USE_W ? ((a & 1) ? lw1 : lw0) : ((a & 1) ? lx1 : lx0);
            const int r = wm * 32 + (lane & 31);  // staged row
            const int j = min(m0 + wm * WTM + a * 32 + (lane & 31), M - 1);
            const float st = (EPI == EPI_CHANNEL || EPI == EPI_GROUP) ? p.s_tok[j] : 0.0f;
#pragma unroll
            for (int b = 0; b < TN; ++b) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int c8 = wn * (WTN / 4) + b * 8 + g * 2 + hi;  // 8-byte unit in the row
                    const int ch = min(n0 + 4 * c8, N - 4);
                    float v[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        if constexpr (EPI == EPI_CHANNEL) {
                            float t = (float)acc[a][b][g * 4 + e] * st;
                            v[e] = t * p.s_w[ch + e];
                        } else if constexpr (EPI == EPI_GROUP) {
                            v[e] = facc[a][b][g * 4 + e] * st;
                        } else if constexpr (W16) {
                            v[e] = p.s_w[ch + e] * acc[a][b][g * 4 + e];
                        } else {
                            v[e] = facc[a][b][g * 4 + e];
                        }
                    }
                    v2u o;
                    o[0] = pack16x2<OUT_F16>(v[0], v[1]);
                    o[1] = pack16x2<OUT_F16>(v[2], v[3]);
                    // unit c8 of row r at c8 ^ (r & 31): conflict-free writes
                    *reinterpret_cast<v2u*>(buf + r * RB + ((c8 ^ (r & 31)) << 3)) = o;
                }
            }
            // LDS writes done; the previous pass's reads of the other buffer
            // were waited for before this barrier as well
            wait_vm_lgkm0<63>();
            block_barrier();
#pragma unroll
            for (int i = 0; i < WM * 32 * CPR / (NW * 64); ++i) {
                const int idx = i * NW * 64 + tid;
                const int rr = idx / CPR, q = idx % CPR;
                const int sw = rr & 31;
                const int base = (2 * q) ^ (sw & ~1);
                v4u d = *reinterpret_cast<const v4u*>(buf + rr * RB + (base << 3));
                if (sw & 1) d = v4u{d[2], d[3], d[0], d[1]};
                const int jj = m0 + (rr >> 5) * WTM + a * 32 + (rr & 31);
                const int cc = n0 + q * 8;
                if (jj < M && cc < N)
                    __builtin_nontemporal_store(d, reinterpret_cast<v4u*>(static_cast<uint16_t*>(p.c) +
                                                                           (int64_t)jj * p.ldc + cc));
            }
        }
        return;
    } else if constexpr (WM <= 2) {
        // Raw int32 (or fp32) sums, as a split-K plane or q8_mm_i32's
        // output, through LDS as well: one 32-row block per wave row and pass,
        // wave row i in stage buffer i (32 rows x BN x 4 bytes, BN x 128
        // bytes of LDS), 16-byte unit u of row r at u ^ (r & 31), then whole
        // lines out.
        constexpr int RB = BN * 4;    // bytes per staged row
        constexpr int CPR = RB / 16;  // 16-byte chunks per row
        static_assert(32 * RB <= BN * BK && CPR % 32 == 0, "staging layout");
        wait_vm_lgkm0<0>();
        block_barrier();  // every wave is done with the stage buffers
        int8_t* const wbuf = (wm & 1) ? lw1 : lw0;
#pragma unroll
        for (int a = 0; a < TM; ++a) {
            const int r = lane & 31;
#pragma unroll
            for (int b = 0; b < TN; ++b) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int u = wn * (WTN / 4) + b * 8 + g * 2 + hi;  // 16-byte unit in the row
                    v4i o;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        if constexpr (EPI == EPI_I32) o[e] = acc[a][b][g * 4 + e];
                        else o[e] = __float_as_int(acc[a][b][g * 4 + e]);
                    }
                    *reinterpret_cast<v4i*>(wbuf + r * RB + ((u ^ r) << 4)) = o;
                }
            }
            wait_vm_lgkm0<63>();  // LDS writes done (stores still in flight)
            block_barrier();
#pragma unroll
            for (int i = 0; i < WM * 32 * CPR / (NW * 64); ++i) {
                const int idx = i * NW * 64 + tid;
                const int h = idx / (32 * CPR);
                const int rr = (idx / CPR) % 32, q = idx % CPR;
                const v4i d = *reinterpret_cast<const v4i*>((h ? lw1 : lw0) + rr * RB + ((q ^ rr) << 4));
                const int jj = m0 + h * WTM + a * 32 + rr;
                const int cc = n0 + q * 4;
                if (jj < M && cc < N) {
                    v4i* dst = reinterpret_cast<v4i*>(static_cast<int32_t*>(p.c) + (int64_t)blockIdx.y * p.plane +
                                                      (int64_t)jj * p.ldc + cc);
                    *dst = d;  // plain store: the reduce reads the planes next
                }
            }
            if (a + 1 < TM) {
                wait_vm_lgkm0<63>();
                block_barrier();  // the reads are done before the next pass writes
            }
        }
        return;
    }
#pragma unroll
    for (int a = 0; a < TM; ++a) {
        const int j = m0 + wm * WTM + a * 32 + (lane & 31);  // token
        if (j >= M) continue;
        const float st = (EPI == EPI_CHANNEL || EPI == EPI_GROUP) ? p.s_tok[j] : 0.0f;
#pragma unroll
        for (int b = 0; b < TN; ++b) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int ch = n0 + wn * WTN + b * 32 + g * 8 + hi * 4;
                if (ch >= N) continue;
                if constexpr (RAW) {  // int32, or fp32 bits (EPI_W16_PART)
                    v4i o;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        if constexpr (EPI == EPI_I32) o[e] = acc[a][b][g * 4 + e];
                        else o[e] = __float_as_int(acc[a][b][g * 4 + e]);
                    }
                    *reinterpret_cast<v4i*>(static_cast<int32_t*>(p.c) + (int64_t)blockIdx.y * p.plane +
                                            (int64_t)j * p.ldc + ch) = o;
                } else {
                    float v[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        if constexpr (EPI == EPI_CHANNEL) {
                            float t = (float)acc[a][b][g * 4 + e] * st;
                            v[e] = t * p.s_w[ch + e];
                        } else if constexpr (EPI == EPI_GROUP) {
                            v[e] = facc[a][b][g * 4 + e] * st;
                        } else if constexpr (W16) {
                            v[e] = p.s_w[ch + e] * acc[a][b][g * 4 + e];
                        } else {
                            v[e] = facc[a][b][g * 4 + e];
                        }
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

// The kernel addresses operands with 32-bit buffer offsets: tiles past the
// edge form row offsets up to (rows + 255) * ld, plus one stage beyond K.
inline bool gemm_offsets_fit(const GemmArgs& p) {
    const int64_t lim = (int64_t)1 << 31;
    return ((int64_t)p.M + 256) * p.ldx + 256 < lim && ((int64_t)p.N + 256) * p.ldw + 256 < lim &&
           ((int64_t)p.N + 256) * (p.K / 128) * 4 + 256 < lim &&
           ((int64_t)p.M + 256) * (p.K / 128) * 4 + 256 < lim;
}

template <int BM, int BN, int WM, int WN, int EPI, int GM>
inline hipError_t launch_gemm_i8(const GemmArgs& p, hipStream_t stream) {
    const int nbm = (p.M + BM - 1) / BM, nbn = (p.N + BN - 1) / BN;
    const int ks = p.kz > 0 ? (p.K + p.kz - 1) / p.kz : 1;
    hipLaunchKernelGGL((gemm_i8_kernel<BM, BN, WM, WN, EPI, GM>), dim3(nbm * nbn, ks), dim3(WM * WN * 64),
                       0, stream, p);
    return hipGetLastError();
}

}  // namespace q8
