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
// the whole offset in the range-checked vector operand, so rows past the
// edge and the stage after K read as zero, chunk c of LDS row r at slot
// c ^ (r & 7) ^ ((r >> 3) & 1).  Schedule of a stage (four 32-deep
// sub-steps): the next stage's loads go out behind the MFMAs of sub-step 0;
// each sub-step's fragments are read behind the previous sub-step's MFMAs as
// they release the registers; halfway through sub-step 3 the wave waits for
// its loads of the next stage and one barrier publishes that stage and
// frees this one, and the second half of sub-step 3 runs behind the next
// stage's first fragment reads.
//
// Epilogue (16-bit outputs): written straight from the MFMA layout, each
// store instruction would put 16-byte pieces into 32 rows, and the 252 MB
// output of the prefill shape then cost about 80 us of the launch (the same
// kernel with the stores branched off: 472 against 551 us).  The values go
// through LDS instead and leave in whole 128-byte lines with non-temporal
// 16-byte stores: 558 -> 531 us, bit-identical.
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
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(p.x, operand_extent(M, p.ldx, K));
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(p.w, operand_extent(N, p.ldw, K));
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
                xr, (Q8_LDS void*)(bx + (wid * XIW + i) * 1024), 16, lane_offset(xv[(wid * XIW + i) & 1],
                xs0 + i * 8 * (int)p.ldx + koff), 0, 0, 0);
#pragma unroll
        for (int i = 0; i < WIW; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                wr, (Q8_LDS void*)(bw + (wid * WIW + i) * 1024), 16, lane_offset(wv[(wid * WIW + i) & 1],
                ws0 + i * 8 * (int)p.ldw + koff), 0, 0, 0);
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
    // MFMAs [t0, t1) of a sub-step, token block a outer: fx[a] is free again
    // after the TN MFMAs that use it
    auto mfma = [&](int t0 = 0, int t1 = NM) __attribute__((always_inline)) {
#pragma unroll
        for (int t = t0; t < t1; ++t) {
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
        // sub-step 3 in two halves around the hand-over: the MFMAs of token
        // blocks 0-1, the barrier, then the next stage's fragments of those
        // blocks (their registers free again) behind the MFMAs of blocks
        // 2-3, then the rest (3% faster than all 12 MFMAs before the
        // barrier: a stage's first reads no longer start with the matrix
        // pipe idle)
        mfma(0, NM / 2);
        __builtin_amdgcn_sched_barrier(0);
        wait_vm_lgkm0<0>();
        block_barrier();
        read_x(0, nx, 0, TM / 2);
        mfma(NM / 2, NM);
        read_x(0, nx, TM / 2, TM);
#pragma unroll
        for (int b = 0; b < TN; ++b) fw[b] = *reinterpret_cast<const v4i*>(nw + wbase[0] + b * 32 * BK);
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
    if constexpr (EPI == EPI_CHANNEL) {
        // 16-bit outputs leave through LDS, so that every store instruction
        // writes whole 128-byte lines: a lane of the MFMA layout holds four
        // channels of one token, and stored directly each instruction would
        // write 16-byte pieces of 32 rows.  Two passes, each of two 32-token
        // blocks of both wave rows (64 tokens x 384 channels, 48 KB, in the
        // two weight stage buffers).  The values and their rounding are the
        // direct form's; only the route to memory differs.
        wait_vm_lgkm0<0>();
        block_barrier();  // every wave is done with the stage buffers
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int a = 2 * pass + h;
                int8_t* buf = h ? lw1 : lw0;
                const int r = wm * 32 + (lane & 31);  // row of the 64-token block
                const int j = min(m0 + wm * WTM + a * 32 + (lane & 31), M - 1);
                const float st = p.s_tok[j];
#pragma unroll
                for (int b = 0; b < TN; ++b) {
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int c8 = wn * (WTN / 4) + b * 8 + g * 2 + hi;  // 8-byte unit in the row
                        const int ch = min(n0 + 4 * c8, N - 4);
                        float v[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float t = (float)acc[a][b][g * 4 + e] * st;
                            v[e] = t * p.s_w[ch + e];
                        }
                        v2u o;
                        o[0] = pack16x2<OUT_F16>(v[0], v[1]);
                        o[1] = pack16x2<OUT_F16>(v[2], v[3]);
                        // unit c8 of row r at c8 ^ (r & 31): the 32 rows a
                        // write instruction touches fall in distinct banks
                        *reinterpret_cast<v2u*>(buf + r * (BN * 2) + ((c8 ^ (r & 31)) << 3)) = o;
                    }
                }
            }
            wait_vm_lgkm0<63>();  // LDS writes done (stores still in flight)
            block_barrier();
            // 2 x 64 rows x 48 chunks of 16 bytes; lane-consecutive chunks
            // of a row, so eight lanes write one whole line
            constexpr int CPR = BN * 2 / 16;  // 16-byte chunks per row
#pragma unroll
            for (int i = 0; i < 2 * 64 * CPR / (NW * 64); ++i) {
                const int idx = i * NW * 64 + tid;
                const int h = idx / (64 * CPR);
                const int rr = (idx / CPR) % 64, q = idx % CPR;
                const int s = rr & 31;
                const int base = (2 * q) ^ (s & ~1);
                v4u d = *reinterpret_cast<const v4u*>((h ? lw1 : lw0) + rr * (BN * 2) + (base << 3));
                if (s & 1) d = v4u{d[2], d[3], d[0], d[1]};
                const int j = m0 + (rr >> 5) * WTM + (2 * pass + h) * 32 + (rr & 31);
                const int ch = n0 + q * 8;
                if (j < M && ch < N)
                    __builtin_nontemporal_store(d, reinterpret_cast<v4u*>(static_cast<uint16_t*>(p.c) +
                                                                           (int64_t)j * p.ldc + ch));
            }
            if (pass == 0) {
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

// gemm_big16_kernel: the per-channel (16-bit output) launches of this tile.
// Why a second form: under changing operands the board lowers its clock
// with the matrix cores' power, and the 16 x 16 x 64 instruction writes half
// the accumulators per product of the 32 x 32 x 32 one.  An MFMA-only loop
// on random int8 operands sustains 3,568 TOP/s with it against 3,135 (zero
// operands: 4,657 against 4,716); this kernel takes 473 us at 8192 x 15360
// x 5120 against 525 us for gemm_big_kernel on the same board, bit-identical.
// gemm_big_kernel keeps the raw int32 mode.
//
// The same tile, loads, LDS layout and epilogue on v_mfma_i32_16x16x64_i8:
// a wave's 128 tokens x 96 channels are 8 x 6 blocks of 16 x 16 (four int32
// sums per lane, four consecutive channels of one token), each 128-deep stage
// two 64-deep sub-steps.  A lane's fragment is 16 bytes of K (chunk 4 kk +
// lane / 16 of row lane % 16 of the 16-row block) for both operands, so the
// products pair equal k.  The six channel fragments stay for a whole
// sub-step; the token fragments are read one block ahead into two register
// slots.  Integer sums are order-free: bit-identical to gemm_big_kernel.
//
// Persistent: one workgroup per CU (each holds the CU's whole LDS) takes
// tiles b, b + grid, ... in turn.  Launched one tile per workgroup, a CU's
// matrix cores idle while its tile's 196 KB of output leave and until the
// next tile's first stage lands; here the next tile's stage 0 is issued into
// lx0 / lw0 right after the last stage, the epilogue stages through lw1 alone
// (four 64-row passes) with the scales in lx1, and the next tile starts as
// soon as its own loads landed: vmcnt retires in issue order, and every wave
// issues the same 24 output stores after them (a store outside C gets an
// offset past its buffer resource and is dropped), so a wait for all but 24
// operations is a wait for exactly the stage-0 loads.  The stores drain
// behind the next tile's first stage.  Same board, bit-identical: 456 against
// 481 us (random codes), 353 against 373 us (zero codes) at 8192 x 15360 x 5120.
template <int EPI_>
__global__ __launch_bounds__(512) void gemm_big16_kernel(GemmArgs p) {
    constexpr int EPI = epi_base(EPI_);
    constexpr bool OUT_F16 = EPI_ != EPI;
    static_assert(EPI == EPI_CHANNEL, "per-channel epilogue");
    constexpr int BM = BIG_BM, BN = BIG_BN, WM = 2, WN = 4, NW = WM * WN, GM = 8, BK = 128;
    constexpr int WTM = BM / WM, WTN = BN / WN;  // 128 tokens x 96 channels per wave
    constexpr int TT = WTM / 16, TC = WTN / 16;  // 8 token blocks, 6 channel blocks
    constexpr int XIW = BM / 8 / NW, WIW = BN / 8 / NW;

    __shared__ __attribute__((aligned(1024))) int8_t lx0[BM * BK];
    __shared__ __attribute__((aligned(1024))) int8_t lx1[BM * BK];
    __shared__ __attribute__((aligned(1024))) int8_t lw0[BN * BK];
    __shared__ __attribute__((aligned(1024))) int8_t lw1[BN * BK];

    const int M = p.M, N = p.N, K = p.K;
    const int nbm = (M + BM - 1) / BM, nbn = (N + BN - 1) / BN;
    const int ntiles = nbm * nbn;
    const int per_group = GM * nbn;
    // tile L of the launch order (workgroup b takes b, b + grid, ...; with a
    // grid that is a multiple of 8, tile L runs on the XCD that dispatch id
    // L would, so xcd_remap keeps each XCD's tiles together)
    auto tile_of = [&](int L, int& tm0, int& tn0) __attribute__((always_inline)) {
        const int id = xcd_remap(L, ntiles);
        const int first_m = (id / per_group) * GM;
        const int gsz = min(nbm - first_m, GM);
        tm0 = (first_m + (id % per_group) % gsz) * BM;
        tn0 = ((id % per_group) / gsz) * BN;
    };

    const int tid = threadIdx.x, lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wid % WM, wn = wid / WM;
    const int q4 = lane >> 4;

    const __amdgpu_buffer_rsrc_t xr = make_rsrc(p.x, operand_extent(M, p.ldx, K));
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(p.w, operand_extent(N, p.ldw, K));
    const int lrow = lane >> 3, lslot = lane & 7;
    const int xv[2] = {lrow * (int)p.ldx + ((lslot ^ lrow) << 4), lrow * (int)p.ldx + ((lslot ^ lrow ^ 1) << 4)};
    const int wv[2] = {lrow * (int)p.ldw + ((lslot ^ lrow) << 4), lrow * (int)p.ldw + ((lslot ^ lrow ^ 1) << 4)};

    // direct loads of stage kt of the tile at (xs0, ws0), instructions
    // [i0, i1) of the wave's 10
    auto issue = [&](int kt, int8_t* bx, int8_t* bw, int i0, int i1, int xs0, int ws0)
        __attribute__((always_inline)) {
        const int koff = kt * BK;
#pragma unroll
        for (int i = 0; i < XIW + WIW; ++i) {
            if (i < i0 || i >= i1) continue;
            if (i < XIW)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    xr, (Q8_LDS void*)(bx + (wid * XIW + i) * 1024), 16,
                    lane_offset(xv[(wid * XIW + i) & 1], xs0 + i * 8 * (int)p.ldx + koff), 0, 0, 0);
            else
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    wr, (Q8_LDS void*)(bw + (wid * WIW + i - XIW) * 1024), 16,
                    lane_offset(wv[(wid * WIW + i - XIW) & 1], ws0 + (i - XIW) * 8 * (int)p.ldw + koff), 0, 0, 0);
        }
    };
    auto xs_of = [&](int tm0) __attribute__((always_inline)) { return (tm0 + wid * XIW * 8) * (int)p.ldx; };
    auto ws_of = [&](int tn0) __attribute__((always_inline)) { return (tn0 + wid * WIW * 8) * (int)p.ldw; };

    // fragment offsets: sub-step kk reads chunk 4 kk + lane / 16 of the
    // lane's row (lane % 16 of a 16-row block; 16 rows further per block,
    // same swizzle)
    int wbase[2], xbase[2];
    {
        const int rw0 = wn * WTN + (lane & 15), rx0 = wm * WTM + (lane & 15);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int ch = 4 * kk + q4;
            wbase[kk] = rw0 * BK + ((ch ^ lds_swizzle(rw0)) << 4);
            xbase[kk] = rx0 * BK + ((ch ^ lds_swizzle(rx0)) << 4);
        }
    }

    v4i acc[TT][TC];
    v4i fw[TC], fx[2];

    auto rdx = [&](int kk, const int8_t* bx, int t) __attribute__((always_inline)) {
        return *reinterpret_cast<const v4i*>(bx + xbase[kk] + t * 16 * BK);
    };
    auto rdw = [&](int kk, const int8_t* bw, int c) __attribute__((always_inline)) {
        return *reinterpret_cast<const v4i*>(bw + wbase[kk] + c * 16 * BK);
    };
    auto block = [&](int t) __attribute__((always_inline)) {
#pragma unroll
        for (int c = 0; c < TC; ++c)
            acc[t][c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fw[c], fx[t & 1], acc[t][c], 0, 0, 0);
    };

    const int KT = K / BK;
    int m0, n0;
    tile_of(blockIdx.x, m0, n0);
    int xs0 = xs_of(m0), ws0 = ws_of(n0);

    // one 64-deep sub-step on fw / fx[0] (already read); the next sub-step's
    // fragments come from (nkk, nbx, nbw); LAST: they belong to the next
    // stage, so the hand-over (loads landed, one barrier) comes first.
    // FIRST: this stage's sub-step 0, which also issues the next stage's
    // loads (if any), two per token block.
    auto substep = [&](int kk, const int8_t* bx, int nkk, const int8_t* nbx, const int8_t* nbw, bool first,
                       bool last, int kt, int8_t* lx_n, int8_t* lw_n) __attribute__((always_inline)) {

#pragma unroll
        for (int t = 0; t < TT; ++t) {
            if (first && t < 5) issue(kt + 1, lx_n, lw_n, 2 * t, 2 * t + 2, xs0, ws0);
            if (t + 1 < TT) fx[(t + 1) & 1] = rdx(kk, bx, t + 1);
            if (t < TT - 1) {
                block(t);
                if (t == TT - 2) {
                    if (last) {
                        __builtin_amdgcn_sched_barrier(0);
                        wait_vm_lgkm0<0>();
                        block_barrier();
                    }
                    fx[0] = rdx(nkk, nbx, 0);  // fx[0] last used by block 6
                }
            } else {
#pragma unroll
                for (int c = 0; c < TC; ++c) {
                    acc[t][c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fw[c], fx[t & 1], acc[t][c], 0, 0, 0);
                    fw[c] = rdw(nkk, nbw, c);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // Tiles in turn.  Each tile's stage 0 is issued into lx0 / lw0 before
    // the previous tile's epilogue (which stages through lw1 only), so its
    // loads land and its first MFMAs run while that epilogue's stores drain:
    // vmcnt counts loads and stores in issue order, so waiting for all but
    // the EPI_STORES stores of a whole tile waits for exactly those loads.
    constexpr int RB = BN * 2, CPR = RB / 16;
    constexpr int EPI_STORES = 4 * (64 * CPR / (NW * 64));  // per wave, whole tile
    static_assert(EPI_STORES < 64, "vmcnt range");
    issue(0, lx0, lw0, 0, XIW + WIW, xs0, ws0);
    wait_vm_lgkm0<0>();
    for (int L = blockIdx.x;;) {
        block_barrier();
        // the epilogue's scales, fp32 in lx1 there: thread tid holds token
        // scale tid (tid < 256) or channel scale tid - 256, then channel
        // scale 256 + tid (tid < 128)
        constexpr int CH0 = NW * 64 - BM, CH1 = BN - CH0;
        const float sv0 = tid < BM ? p.s_tok[min(m0 + tid, M - 1)] : p.s_w[min(n0 + tid - BM, N - 1)];
        const float sv1 = p.s_w[min(n0 + CH0 + tid % CH1, N - 1)];  // used below tid = 128
#pragma unroll
        for (int t = 0; t < TT; ++t)
#pragma unroll
            for (int c = 0; c < TC; ++c) acc[t][c] = v4i{};
#pragma unroll
        for (int c = 0; c < TC; ++c) fw[c] = rdw(0, lw0, c);
        fx[0] = rdx(0, lx0, 0);
        int kt = 0;
        for (; kt + 2 <= KT; kt += 2) {
            substep(0, lx0, 1, lx0, lw0, true, false, kt, lx1, lw1);
            substep(1, lx0, 0, lx1, lw1, false, true, kt, lx1, lw1);
            substep(0, lx1, 1, lx1, lw1, true, false, kt + 1, lx0, lw0);
            substep(1, lx1, 0, lx0, lw0, false, true, kt + 1, lx0, lw0);
        }
        if (kt < KT) {
            substep(0, lx0, 1, lx0, lw0, true, false, kt, lx1, lw1);
            substep(1, lx0, 0, lx1, lw1, false, true, kt, lx1, lw1);
        }

        // -------------------------------------------------------- epilogue --
        // four passes of one 32-token group of both wave rows (64 rows x 384
        // channels in lw1), whole lines out.  8-byte unit u of row r at
        // u ^ ((r & 15) << 1): a write instruction's 16 rows x 2 adjacent
        // units, and a read's 16 chunks of one row, fall in distinct banks,
        // and a 16-byte chunk stays in order.
        wait_vm_lgkm0<0>();
        block_barrier();  // both stage buffers are free
        // per-lane values from here on are made inside the tile loop (an
        // empty asm hides their loop invariance), so that none of them stays
        // live across the main loop
        int le = lane, te = tid;
        asm volatile("" : "+v"(le), "+v"(te));
        // the tile's scales (loaded at its start) go to lx1: the passes read
        // them from LDS, and no global load of the epilogue waits behind the
        // next tile's loads or this tile's stores
        float* sc_s = reinterpret_cast<float*>(lx1);
        const int Ln = L + (int)gridDim.x;
        const bool next = Ln < ntiles;
        int m0n = 0, n0n = 0;
        if (next) {
            tile_of(Ln, m0n, n0n);
            issue(0, lx0, lw0, 0, XIW + WIW, xs_of(m0n), ws_of(n0n));
        }
        sc_s[te] = sv0;
        if (te < CH1) sc_s[BM + CH0 + te] = sv1;
        wait_vm_lgkm0<63>();
        block_barrier();
        // C through a buffer resource from the tile's first row: every
        // lane issues its store (one past the resource, offset 2^31, for an
        // element outside C, which the hardware drops), so that each wave
        // issues exactly EPI_STORES of them
        const __amdgpu_buffer_rsrc_t cr =
            make_rsrc(static_cast<uint16_t*>(p.c) + (int64_t)m0 * p.ldc,
                      (uint32_t)(((int64_t)(min(BM, M - m0) - 1) * p.ldc + N) * 2));
#pragma unroll
        for (int a32 = 0; a32 < 4; ++a32) {
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                const int t = 2 * a32 + tt;
                const int r = wm * 32 + tt * 16 + (le & 15);
                const float st = sc_s[wm * WTM + t * 16 + (le & 15)];
#pragma unroll
                for (int c = 0; c < TC; ++c) {
                    const int c8 = wn * (WTN / 4) + c * 4 + (le >> 4);
                    const v4f sw = *reinterpret_cast<const v4f*>(sc_s + BM + 4 * c8);
                    float v[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float tv = (float)acc[t][c][e] * st;
                        v[e] = tv * sw[e];
                    }
                    v2u o;
                    o[0] = pack16x2<OUT_F16>(v[0], v[1]);
                    o[1] = pack16x2<OUT_F16>(v[2], v[3]);
                    *reinterpret_cast<v2u*>(lw1 + r * RB + ((c8 ^ ((r & 15) << 1)) << 3)) = o;
                }
            }
            wait_vm_lgkm0<63>();
            block_barrier();
#pragma unroll
            for (int i = 0; i < 64 * CPR / (NW * 64); ++i) {
                const int idx = i * NW * 64 + te;
                const int rr = idx / CPR, q = idx % CPR;
                const v4u d = *reinterpret_cast<const v4u*>(lw1 + rr * RB + ((q ^ (rr & 15)) << 4));
                const int jr = (rr >> 5) * WTM + a32 * 32 + (rr & 31);  // row in the tile
                const int ch = n0 + q * 8;
                const int off = m0 + jr < M && ch < N ? (jr * (int)p.ldc + ch) * 2 : INT32_MIN;
                __builtin_amdgcn_raw_buffer_store_b128(d, cr, off, 0, 2);  // 2: non-temporal
            }
            if (a32 < 3) {
                wait_vm_lgkm0<63>();
                block_barrier();
            }
        }
        if (!next) break;
        L = Ln;
        m0 = m0n;
        n0 = n0n;
        xs0 = xs_of(m0);
        ws0 = ws_of(n0);
        wait_vm_lgkm0<EPI_STORES>();  // the next tile's stage 0 landed
    }
}

// 32-bit buffer offsets: channel rows reach n0 + 383 < N + 383, token rows
// m0 + 255, and the loads run one stage past K.
inline bool gemm_big_offsets_fit(const GemmArgs& p) {
    const int64_t lim = (int64_t)1 << 31;
    return ((int64_t)p.M + 256) * p.ldx + 256 < lim && ((int64_t)p.N + 384) * p.ldw + 256 < lim &&
           (int64_t)257 * p.ldc * 4 < lim;  // C offsets within a tile (gemm_big16_kernel's stores)
}

// Workgroups of the 16 x 16 x 64 launch: one per CU of the current device
// (each holds a CU's whole LDS), which then take the tiles in turn.
inline int big16_grid() {
    static int cus[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cus[dev] <= 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cus[dev] = n;
    }
    return cus[dev];
}

template <int EPI>
inline hipError_t launch_gemm_big(const GemmArgs& p, hipStream_t stream) {
    const int nbm = (p.M + BIG_BM - 1) / BIG_BM, nbn = (p.N + BIG_BN - 1) / BIG_BN;
    if constexpr (epi_base(EPI) == EPI_CHANNEL)  // 16-bit outputs: the 16 x 16 x 64 form
        hipLaunchKernelGGL((gemm_big16_kernel<EPI>), dim3(nbm * nbn < big16_grid() ? nbm * nbn : big16_grid()), dim3(512), 0, stream, p);
    else
        hipLaunchKernelGGL((gemm_big_kernel<EPI>), dim3(nbm * nbn), dim3(512), 0, stream, p);
    return hipGetLastError();
}

}  // namespace q8
