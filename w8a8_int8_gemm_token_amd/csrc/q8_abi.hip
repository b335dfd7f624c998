// q8_abi.hip -- the C ABI of libq8 (declared in include/q8.h): argument
// validation and kernel dispatch.  Validation runs on the host before any
// HIP call, so an invalid call returns an error code and enqueues nothing.
#include "q8.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "gemm_i8.hpp"
#include "quant.hpp"
#include "decode_fused.hpp"
#include "norm_quant.hpp"
#include "w8a16.hpp"
#include "gemm_big.hpp"
#include "gemm_w16.hpp"
#include "stream_gemm.hpp"
#include "small_fused.hpp"
#include "stream_group.hpp"
#include "fp8.hpp"
#include "splitk.hpp"

namespace {

using namespace q8;

inline bool al(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

inline q8_status hip_status(hipError_t e) { return e == hipSuccess ? Q8_OK : Q8_EHIP; }

inline hipStream_t st(q8_stream s) { return reinterpret_cast<hipStream_t>(s); }

// Shape rules shared by the GEMM entry points (see q8.h).  `lda_mult` is the
// multiple the activation leading dimension must be (16 int8 codes or 8 bf16
// values: 16 bytes), `ldc_mult` that of the output (8 bf16 or 4 int32).
q8_status check_gemm(const void* a, int64_t lda, int64_t lda_mult, const void* b, int64_t ldb,
                     const void* c, int64_t ldc, int64_t ldc_mult, int64_t M, int64_t N,
                     int64_t K) {
    if (M < 0 || N < 0 || K < 0) return Q8_EINVAL;
    if (M == 0) return Q8_OK;
    if (!a || !b || !c || N == 0 || K == 0) return Q8_EINVAL;
    if (lda < K || ldb < K || ldc < N) return Q8_EINVAL;
    if (N % 16 != 0 || K % 128 != 0 || K > Q8_MAX_K) return Q8_EUNSUPPORTED;
    if (M > INT32_MAX / 2 || N > INT32_MAX / 2) return Q8_EUNSUPPORTED;
    if (lda % lda_mult != 0 || ldb % 16 != 0 || ldc % ldc_mult != 0) return Q8_EUNSUPPORTED;
    if (!al(a, 16) || !al(b, 16) || !al(c, 16)) return Q8_EUNSUPPORTED;
    // 32-bit buffer offsets inside the kernels (see Q8_MAX_OPERAND_BYTES)
    const int64_t lim = Q8_MAX_OPERAND_BYTES;
    if ((M + 256) * lda * (lda_mult == 8 ? 2 : 1) >= lim || (N + 256) * ldb >= lim) return Q8_EUNSUPPORTED;
    return Q8_OK;
}

// Scale vectors: non-null (Q8_EINVAL) and 4-byte aligned (Q8_EUNSUPPORTED).
inline q8_status check_scale(const float* s) {
    if (s == nullptr) return Q8_EINVAL;
    return al(s, 4) ? Q8_OK : Q8_EUNSUPPORTED;
}

// Tile configurations of the INT8 GEMM, chosen by the problem size: 32-token
// tiles for small batches, 256 x 384 or 256 x 256 tiles (8 waves) once there
// are enough of them to fill the 256 CUs, smaller tiles by workgroup count in
// between, and 256 x 256 again where 128 x 128 tiles would need a second,
// partly filled round.
template <int EPI>
hipError_t run_gemm_i8(const GemmArgs& p, hipStream_t s) {
    if constexpr (EPI == EPI_CHANNEL || EPI == EPI_CHANNEL_F16) {
        // up to 16 tokens, K a multiple of 1024 and N <= 4096 (one workgroup
        // of at most 16 channels per CU): the decode kernel's weight stream on
        // the codes, whole weight tile in LDS and each K segment multiplied as
        // it lands.  Per call in a graph on rotating weight copies: 4096 x 4096
        // 5.9-7.0 against 6.4-7.6 us, 2048 x 8192 6.6-8.6 against 8.5-9.3 us
        // (1-16 tokens).  From 5120 channels the streaming kernel's 3-slot
        // ring is as fast or faster (5120: 7.1-8.5 against 7.1-8.1 us; 15360
        // and 17408, several workgroups per CU in turn: 13-20% faster).
        if (p.N <= 4096 && p.ldx % 16 == 0 && decode_pre_fits(p.M, p.N, p.K, p.ldw)) {
            const DecodePreArgs d{p.x, p.ldx, p.s_tok, p.w, p.ldw, p.s_w, static_cast<uint16_t*>(p.c), p.ldc,
                                  p.M, p.N, p.K, decode_rows(p.N, p.K, false)};
            return launch_decode_pre<EPI == EPI_CHANNEL_F16>(d, s);
        }
        // few tokens: stream the weights once, unless the tiled kernel already
        // has half a wave of tiles or more (M > 32 with many channels)
        const bool few = p.M <= 32 || ((p.N + 127) / 128) * ((p.M + 31) / 32) < 128;
        if (few && sg_fits(p.M, p.N, p.K, p.ldw, SG_MAX_M)) {
            const StreamArgs q{p.x, p.ldx, p.w, p.ldw, p.s_tok, p.s_w, static_cast<uint16_t*>(p.c), p.ldc,
                               p.M, p.N, p.K, 0, 0, EPI == EPI_CHANNEL_F16 ? 1 : 0};
            return launch_stream<true>(q, s);
        }
        // 65-128 tokens and under 64 channel tiles of 128: the tiled grid
        // leaves most CUs idle, and two streaming passes (64 tokens, then
        // the rest) take less time (5120 x 5120: 23-33 against 42-43 us)
        if (p.M > SG_MAX_M && p.M <= 2 * SG_MAX_M && (p.N + 127) / 128 < 64 &&
            sg_fits(SG_MAX_M, p.N, p.K, p.ldw, SG_MAX_M)) {
            for (int h = 0; h < 2; ++h) {
                const int m0 = h * SG_MAX_M;
                const StreamArgs q{p.x + (int64_t)m0 * p.ldx, p.ldx, p.w, p.ldw, p.s_tok + m0, p.s_w,
                                   static_cast<uint16_t*>(p.c) + (int64_t)m0 * p.ldc, p.ldc,
                                   h ? p.M - SG_MAX_M : SG_MAX_M, p.N, p.K, 0, 0, EPI == EPI_CHANNEL_F16 ? 1 : 0};
                const hipError_t e = launch_stream<true>(q, s);
                if (e != hipSuccess) return e;
            }
            return hipSuccess;
        }
    }
    if (p.M <= 64) return launch_gemm_i8<32, 128, 1, 4, EPI, 8>(p, s);
    const int64_t nbm = (p.M + 255) / 256;
    const int64_t t256 = nbm * ((p.N + 255) / 256), t384 = nbm * ((p.N + 383) / 384);
    if (t256 < 256) {
        // Too few 256 x 256 tiles to fill the chip: the tile with the fewest
        // bytes per product among those that still give at most 420
        // workgroups (measured over 65-384 tokens at N = 5120, 15360 and
        // 17408: 32 x 128 tiles won below that count, 64 x 128 next, and
        // 128 x 128 beyond; 10-20% apart).
        const int64_t nt = (p.N + 127) / 128;
        if ((p.M + 31) / 32 * nt <= 420) return launch_gemm_i8<32, 128, 1, 4, EPI, 8>(p, s);
        if ((p.M + 63) / 64 * nt <= 420) return launch_gemm_i8<64, 128, 2, 2, EPI, 8>(p, s);
        // 128 x 128 tiles run two to a CU: past 512 of them the second, partly
        // filled round costs more than the one round of 256 x 256 tiles (K =
        // 5120, rotating weight copies: N = 17408 at 448-768 tokens 93-99
        // against 71-79 us, N = 15360 and 13824 at 576-1024 tokens 80-106
        // against 67-81 us; at 512 tiles or fewer 128 x 128 stays 20-35%
        // faster)
        if ((p.M + 127) / 128 * nt <= 512) return launch_gemm_i8<128, 128, 2, 2, EPI, 8>(p, s);
        return launch_gemm_i8<256, 256, 2, 4, EPI, 8>(p, s);
    }
    // Whole waves of 256 tiles (a partly filled last wave costs a whole
    // one); a wave of 256 x 384 tiles takes about 1.3 times as long as one
    // of 256 x 256 (1.26-1.34 measured at 8192 tokens for 5120, 13824 and
    // 15360 channels, the 256 x 384 tile on the 16 x 16 x 64 kernel; with
    // the 32 x 32 x 32 one, which the raw int32 output keeps, it was 1.4)
    const int64_t w256 = (t256 + 255) / 256, w384 = (t384 + 255) / 256;
    const int64_t ratio = epi_base(EPI) == EPI_CHANNEL ? 130 : 140;
    if (ratio * w384 < 100 * w256 && gemm_big_offsets_fit(p)) return launch_gemm_big<EPI>(p, s);
    return launch_gemm_i8<256, 256, 2, 4, EPI, 8>(p, s);
}

// Group-scaled epilogues: 32 x 128 or 64 x 128 tiles while they give at most
// one workgroup per CU, else 128 x 128 tiles of 4 waves (64 x 64 each, with
// the fold's second set of fp32 accumulators), two to a CU.
template <int EPI>
hipError_t run_gemm_grouped(const GemmArgs& p, hipStream_t s) {
    // up to 64 tokens: stream the weights once (stream_group.hpp)
    if (sgg_fits(p.M, p.N, p.K, p.ldx, p.ldw)) {
        const StreamGroupArgs q{p.x, p.ldx, p.w, p.ldw, p.s_tok, p.s_w, static_cast<uint16_t*>(p.c), p.ldc,
                                p.M, p.N, p.K, 0, 0};
        constexpr bool ACT = EPI != EPI_GROUP;
        return launch_stream_group<ACT, EPI == EPI_GROUP_ACT_F16>(q, s);
    }
    if (p.M <= 64) return launch_gemm_i8<32, 128, 1, 4, EPI, 8>(p, s);
    // 32 or 64 tokens per tile while that gives at most 256 workgroups (one
    // per CU), else 128.  Two 128 x 128 workgroups share a CU, and the last,
    // partly filled round of such tiles costs less than one of 256 x 128
    // tiles (one per CU): K = 5120, rotating weight copies, 128 x 128 against
    // 256 x 128 tiles at N = 5120, 15360 and 17408 over 128-4096 tokens were
    // 0-47% faster (4096 x 5120: 167 against 191 us; 384 x 17408: 63 against
    // 118 us) and never more than 2% slower.
    const int64_t nt = (p.N + 127) / 128;
    if ((p.M + 31) / 32 * nt <= 256) return launch_gemm_i8<32, 128, 1, 4, EPI, 8>(p, s);
    if ((p.M + 63) / 64 * nt <= 256) return launch_gemm_i8<64, 128, 2, 2, EPI, 8>(p, s);
    return launch_gemm_i8<128, 128, 2, 2, EPI, 8>(p, s);
}

template <int EPI>  // EPI_GROUP_ACT or EPI_GROUP_ACT_F16
hipError_t run_gemm_group_act(const GemmArgs& p, hipStream_t s) {
    return run_gemm_grouped<EPI>(p, s);
}

hipError_t run_gemm_fp8_block(const GemmArgs& p, hipStream_t s) {
    if (p.M <= 64) return launch_gemm_i8<32, 128, 1, 4, EPI_FP8_BLOCK, 8>(p, s);
    // 32 or 64 tokens per tile while that gives at most 256 workgroups, else
    // 128 (measured over 65-2048 tokens at N = 5120 and 15360: 20-27%
    // faster at 65-256 tokens, never slower than 128 x 128 throughout)
    const int64_t nt = (p.N + 127) / 128;
    if ((p.M + 31) / 32 * nt <= 256) return launch_gemm_i8<32, 128, 1, 4, EPI_FP8_BLOCK, 8>(p, s);
    if ((p.M + 63) / 64 * nt <= 256) return launch_gemm_i8<64, 128, 2, 2, EPI_FP8_BLOCK, 8>(p, s);
    return launch_gemm_i8<128, 128, 2, 2, EPI_FP8_BLOCK, 8>(p, s);
}

hipError_t run_gemm_group(const GemmArgs& p, hipStream_t s) { return run_gemm_grouped<EPI_GROUP>(p, s); }

// ---- split K (caller workspace) ----------------------------------------
// Between the few-token kernels and the large tiles the tiled grid has too
// few tiles to fill 256 CUs.  With a workspace the GEMM then runs on
// BM x 128 tiles (BM = 32 up to 32 tokens, 64 up to 64, else 128) with K
// split ks ways, ks = 480 / tiles (at most 10, and K at least 768 per
// split), so that about 240-480 workgroups run.  Measured over 24-512
// tokens at N = 5120, 15360 and 17408 (K = 5120) and the W8A16 shapes
// 5120 x 17408 and 5120 x 13824 against 21 (tile, ks) pairs, this rule
// picks the fastest pair or one within 10% of it: 1.0-3.5x faster than the
// unsplit route from 65 tokens, and from 24 tokens wherever that route
// would run the tiled kernel or (W8A16) the weight-streaming kernel at 24
// tokens and more (the W8A8 weight-streaming kernel stays where it runs:
// within 5% of the split or faster).  Since ks * tiles <= 480 and a tile
// covers at most 128 x 128 outputs, the planes never need more than
// 480 * 128 * 128 * 4 bytes (30 MiB).
struct SplitPlan {
    int ks = 1;         // planes (1: no split)
    int kz = 0;         // K elements per split, a multiple of 128
    int bm = 128;       // tokens per tile
    int64_t bytes = 0;  // workspace: ks planes of [M][N] 4-byte partial sums
};

inline SplitPlan split_plan(int64_t M, int64_t N, int64_t K) {
    SplitPlan sp;
    if (M < 24 || N <= 0 || K < 256) return sp;  // few tokens: the streaming kernels
    sp.bm = M <= 32 ? 32 : M <= 64 ? 64 : 128;
    const int64_t tiles = ((M + sp.bm - 1) / sp.bm) * ((N + 127) / 128);
    int64_t ks = 480 / tiles;
    if (ks > 10) ks = 10;
    if (ks > K / 768) ks = K / 768;
    if (ks < 2) return sp;
    int64_t kz = (K + ks - 1) / ks;
    kz = (kz + 127) / 128 * 128;
    const int64_t ksr = (K + kz - 1) / kz;
    if (ksr < 2) return sp;
    sp.ks = (int)ksr;
    sp.kz = (int)kz;
    sp.bytes = ksr * M * N * 4;
    return sp;
}

// The W8A8 route runs the weight-streaming kernel (one pass) at this size:
// run_gemm_i8's own test for it.
inline bool w8a8_streams(const GemmArgs& p) {
    const bool few = p.M <= 32 || ((p.N + 127) / 128) * ((p.M + 31) / 32) < 128;
    return few && sg_fits(p.M, p.N, p.K, p.ldw, SG_MAX_M);
}

// Workspace argument check: none needed -> anything (NULL included) is
// accepted; else non-null, at least `need` bytes (Q8_EINVAL) and 16-byte
// aligned (Q8_EUNSUPPORTED).
inline q8_status check_ws(const void* ws, int64_t ws_bytes, int64_t need) {
    if (need == 0) return Q8_OK;
    if (ws == nullptr || ws_bytes < need) return Q8_EINVAL;
    return al(ws, 16) ? Q8_OK : Q8_EUNSUPPORTED;
}

// The tiled kernel over ks K ranges into the workspace planes, then the
// reduction with the epilogue into p.c.  W16: the W8A16 mode (p.x bf16 or
// fp16 addressed in bytes); F16: fp16 activations (W16) and outputs.
template <bool W16, bool F16>
hipError_t run_split(const GemmArgs& p, const SplitPlan& sp, void* ws, hipStream_t s) {
    GemmArgs q = p;
    q.c = ws;
    q.ldc = p.N;
    q.kz = sp.kz;
    q.plane = (int64_t)p.M * p.N;
    constexpr int E = W16 ? (F16 ? EPI_W16_PART_F16 : EPI_W16_PART) : EPI_I32;
    const hipError_t e = sp.bm == 32   ? launch_gemm_i8<32, 128, 1, 4, E, 8>(q, s)
                         : sp.bm == 64 ? launch_gemm_i8<64, 128, 2, 2, E, 8>(q, s)
                                       : launch_gemm_i8<128, 128, 2, 2, E, 8>(q, s);
    if (e != hipSuccess) return e;
    return launch_splitk_reduce<W16 ? 1 : 0, F16>(static_cast<const int32_t*>(ws), sp.ks, q.plane, p.s_tok,
                                                    p.s_w, static_cast<uint16_t*>(p.c), p.ldc, p.M, p.N, s);
}

template <bool F16>
hipError_t run_quant(const uint16_t* x, int64_t ldx, int8_t* xq, int64_t ldxq, float* s, int M,
                     int K, hipStream_t stream) {
    const dim3 grid((M + 3) / 4), block(256);
    const bool vec = K % 8 == 0 && ldx % 8 == 0 && ldxq % 8 == 0 && al(x, 16) && al(xq, 8);
#define Q8_REG(n) hipLaunchKernelGGL((quant_per_token_reg<n, F16>), grid, block, 0, stream, x, ldx, xq, ldxq, s, M, K)
    if (vec && M <= 256 && K <= 8 * 512 * 2)  // few rows: a workgroup per row
        hipLaunchKernelGGL((quant_per_token_wg<512, 2, F16>), dim3(M), dim3(512), 0, stream, x, ldx, xq, ldxq, s, K);
    else if (vec && K <= 512) Q8_REG(1);
    else if (vec && K <= 2048) Q8_REG(4);
    else if (vec && K <= 3072) Q8_REG(6);
    else if (vec && K <= 4096) Q8_REG(8);
    else if (vec && K <= 5120) Q8_REG(10);
    else if (vec && K <= 8192) Q8_REG(16);
    else hipLaunchKernelGGL((quant_per_token_any<F16>), grid, block, 0, stream, x, ldx, xq, ldxq, s, M, K);
#undef Q8_REG
    return hipGetLastError();
}

// Entry-point bodies shared by the bf16 and fp16 variants.
template <bool F16>
q8_status quant_per_token_impl(const uint16_t* x, int64_t ldx, int8_t* xq, int64_t ldxq,
                               float* scale_tok, int64_t M, int64_t K, q8_stream stream) {
    if (M < 0 || K < 0) return Q8_EINVAL;
    if (M == 0) return Q8_OK;
    if (!x || !xq || !scale_tok || K == 0 || ldx < K || ldxq < K) return Q8_EINVAL;
    if (!al(x, 2) || !al(scale_tok, 4)) return Q8_EUNSUPPORTED;
    if (M > INT32_MAX / 2 || K > INT32_MAX / 2) return Q8_EUNSUPPORTED;
    return hip_status(run_quant<F16>(x, ldx, xq, ldxq, scale_tok, (int)M, (int)K, st(stream)));
}

template <bool F16>
q8_status scaled_mm_impl(const int8_t* a, int64_t lda, const int8_t* b, int64_t ldb,
                         const float* scale_tok, const float* scale_ch, uint16_t* c, int64_t ldc,
                         int64_t M, int64_t N, int64_t K, q8_stream stream) {
    q8_status r = check_gemm(a, lda, 16, b, ldb, c, ldc, 8, M, N, K);
    if (r == Q8_OK && M > 0) r = check_scale(scale_tok);
    if (r == Q8_OK && M > 0) r = check_scale(scale_ch);
    if (r != Q8_OK || M == 0) return r;
    GemmArgs p{a, lda, b, ldb, scale_tok, scale_ch, c, ldc, (int)M, (int)N, (int)K};
    return hip_status(run_gemm_i8<F16 ? EPI_CHANNEL_F16 : EPI_CHANNEL>(p, st(stream)));
}

template <bool F16>
q8_status quant_scaled_mm_impl(const uint16_t* x, int64_t ldx, const int8_t* b, int64_t ldb,
                               const float* scale_ch, uint16_t* c, int64_t ldc, int8_t* xq,
                               float* scale_tok, int64_t M, int64_t N, int64_t K,
                               q8_stream stream) {
    q8_status r = check_gemm(x, ldx, 8, b, ldb, c, ldc, 8, M, N, K);
    if (r == Q8_OK && M > 0) r = check_scale(scale_ch);
    if (r == Q8_OK && M > 0) r = check_scale(scale_tok);
    if (r == Q8_OK && M > 0 && !xq) r = Q8_EINVAL;
    if (r == Q8_OK && M > 0 && !al(xq, 16)) r = Q8_EUNSUPPORTED;
    if (r != Q8_OK || M == 0) return r;
    hipStream_t s = st(stream);
    // one kernel for the whole layer where one applies: below K = 1024 the
    // small-layer kernel, then the decode kernel (up to 8 tokens), then the
    // small-layer kernel at K = 1024
    const bool small = small_fits((int)M, (int)N, (int)K, ldb);
    const SmallArgs sa{x, ldx, b, ldb, scale_ch, c, ldc, xq, scale_tok, (int)M, (int)N, (int)K};
    if (small && K < SMALL_MAX_K) return hip_status(launch_small<F16>(sa, s));
    if (decode_fits((int)M, (int)N, (int)K, ldb) && decode_beats_stream((int)N, (int)K)) {
        const DecodeArgs d{x, ldx, b, ldb, scale_ch, c, ldc, xq, scale_tok,
                           (int)M, (int)N, (int)K, decode_rows((int)N, (int)K)};
        return hip_status(launch_decode<F16>(d, s));
    }
    if (small) return hip_status(launch_small<F16>(sa, s));
    hipError_t e = run_quant<F16>(x, ldx, xq, K, scale_tok, (int)M, (int)K, s);
    if (e != hipSuccess) return Q8_EHIP;
    GemmArgs p{xq, K, b, ldb, scale_tok, scale_ch, c, ldc, (int)M, (int)N, (int)K};
    return hip_status(run_gemm_i8<F16 ? EPI_CHANNEL_F16 : EPI_CHANNEL>(p, s));
}

template <bool F16>
q8_status scaled_mm_ws_impl(const int8_t* a, int64_t lda, const int8_t* b, int64_t ldb,
                            const float* scale_tok, const float* scale_ch, uint16_t* c, int64_t ldc,
                            int64_t M, int64_t N, int64_t K, void* ws, int64_t ws_bytes, q8_stream stream) {
    q8_status r = check_gemm(a, lda, 16, b, ldb, c, ldc, 8, M, N, K);
    if (r == Q8_OK && M > 0) r = check_scale(scale_tok);
    if (r == Q8_OK && M > 0) r = check_scale(scale_ch);
    const SplitPlan sp = r == Q8_OK && M > 0 ? split_plan(M, N, K) : SplitPlan{};
    if (r == Q8_OK && M > 0) r = check_ws(ws, ws_bytes, sp.bytes);
    if (r != Q8_OK || M == 0) return r;
    GemmArgs p{a, lda, b, ldb, scale_tok, scale_ch, c, ldc, (int)M, (int)N, (int)K};
    if (sp.ks > 1 && !w8a8_streams(p) && gemm_offsets_fit(p))
        return hip_status(run_split<false, F16>(p, sp, ws, st(stream)));
    return hip_status(run_gemm_i8<F16 ? EPI_CHANNEL_F16 : EPI_CHANNEL>(p, st(stream)));
}

template <bool F16>
q8_status quant_scaled_mm_ws_impl(const uint16_t* x, int64_t ldx, const int8_t* b, int64_t ldb,
                                  const float* scale_ch, uint16_t* c, int64_t ldc, int8_t* xq,
                                  float* scale_tok, int64_t M, int64_t N, int64_t K, void* ws,
                                  int64_t ws_bytes, q8_stream stream) {
    q8_status r = check_gemm(x, ldx, 8, b, ldb, c, ldc, 8, M, N, K);
    if (r == Q8_OK && M > 0) r = check_scale(scale_ch);
    if (r == Q8_OK && M > 0) r = check_scale(scale_tok);
    if (r == Q8_OK && M > 0 && !xq) r = Q8_EINVAL;
    if (r == Q8_OK && M > 0 && !al(xq, 16)) r = Q8_EUNSUPPORTED;
    const SplitPlan sp = r == Q8_OK && M > 0 ? split_plan(M, N, K) : SplitPlan{};
    if (r == Q8_OK && M > 0) r = check_ws(ws, ws_bytes, sp.bytes);
    if (r != Q8_OK || M == 0) return r;
    GemmArgs p{xq, K, b, ldb, scale_tok, scale_ch, c, ldc, (int)M, (int)N, (int)K};
    if (sp.ks < 2 || w8a8_streams(p) || !gemm_offsets_fit(p))
        return quant_scaled_mm_impl<F16>(x, ldx, b, ldb, scale_ch, c, ldc, xq, scale_tok, M, N, K, stream);
    hipStream_t s = st(stream);
    if (run_quant<F16>(x, ldx, xq, K, scale_tok, (int)M, (int)K, s) != hipSuccess) return Q8_EHIP;
    return hip_status(run_split<false, F16>(p, sp, ws, s));
}

template <bool F16>
q8_status quant_per_group128_impl(const uint16_t* x, int64_t ldx, int8_t* xq, int64_t ldxq,
                                  float* scale_grp, int64_t M, int64_t K, q8_stream stream) {
    if (M < 0 || K < 0) return Q8_EINVAL;
    if (M == 0) return Q8_OK;
    if (!x || !xq || !scale_grp || K == 0 || ldx < K || ldxq < K) return Q8_EINVAL;
    if (K % 128 != 0 || M > INT32_MAX / 2 || K > INT32_MAX / 2) return Q8_EUNSUPPORTED;
    if (ldx % 8 != 0 || ldxq % 8 != 0 || !al(x, 16) || !al(xq, 8) || !al(scale_grp, 4))
        return Q8_EUNSUPPORTED;
    const int64_t waves = M * ((K + 511) / 512);
    if ((waves + 3) / 4 > INT32_MAX) return Q8_EUNSUPPORTED;
    hipLaunchKernelGGL((quant_per_group128_kernel<F16>), dim3((unsigned)((waves + 3) / 4)), dim3(256), 0,
                       st(stream), x, ldx, xq, ldxq, scale_grp, (int)M, (int)K);
    return hip_status(hipGetLastError());
}

template <bool F16>
q8_status scaled_mm_group128_act_impl(const int8_t* a, int64_t lda, const int8_t* b, int64_t ldb,
                                      const float* scale_x, const float* scale_w, uint16_t* c,
                                      int64_t ldc, int64_t M, int64_t N, int64_t K,
                                      q8_stream stream) {
    q8_status r = check_gemm(a, lda, 16, b, ldb, c, ldc, 8, M, N, K);
    if (r == Q8_OK && M > 0) r = check_scale(scale_x);
    if (r == Q8_OK && M > 0) r = check_scale(scale_w);
    if (r != Q8_OK || M == 0) return r;
    GemmArgs p{a, lda, b, ldb, scale_x, scale_w, c, ldc, (int)M, (int)N, (int)K};
    if (!gemm_offsets_fit(p)) return Q8_EUNSUPPORTED;
    return hip_status(run_gemm_group_act<F16 ? EPI_GROUP_ACT_F16 : EPI_GROUP_ACT>(p, st(stream)));
}

// ---- the allocation-free variant's workspace ---------------------------
// A file-scope device array stands in for the caller's workspace in
// q8_quant_scaled_mm_noalloc.  Every GPU the library runs on holds its own
// copy from the time the library is loaded there until the process ends.
// In host code `scratch` names a host-side stand-in, not device memory:
// its device address comes from hipGetSymbolAddress, looked up once per
// device with that device current and kept in scratch_ptr.
constexpr int64_t SCRATCH_BYTES = Q8_NOALLOC_MAX_WORKSPACE;
static __device__ __align__(256) int32_t scratch[SCRATCH_BYTES / 4];

constexpr int MAX_DEVICES = 64;
std::atomic<void*> scratch_ptr[MAX_DEVICES];
std::mutex scratch_mutex;

// Device address of this device's scratch array (the device `stream`
// belongs to), or nullptr if HIP refuses the lookup.
void* device_scratch(hipStream_t stream) {
    int dev = -1;
    if (stream != nullptr) {
        if (hipStreamGetDevice(stream, &dev) != hipSuccess) return nullptr;
    } else if (hipGetDevice(&dev) != hipSuccess) {
        return nullptr;
    }
    if (dev < 0 || dev >= MAX_DEVICES) return nullptr;
    void* p = scratch_ptr[dev].load(std::memory_order_acquire);
    if (p != nullptr) return p;
    std::lock_guard<std::mutex> lock(scratch_mutex);
    p = scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p != nullptr) return p;
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return nullptr;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess) return nullptr;
    scratch_ptr[dev].store(p, std::memory_order_release);
    return p;
}

}  // namespace

extern "C" {

const char* q8_status_str(q8_status s) {
    switch (s) {
        case Q8_OK: return "ok";
        case Q8_EINVAL: return "invalid argument (null pointer, negative/zero size, ld < row)";
        case Q8_EUNSUPPORTED: return "unsupported shape or alignment";
        case Q8_EHIP: return "HIP launch failed";
    }
    return "unknown status";
}

q8_status q8_quant_per_token(const q8_bf16* x, int64_t ldx, int8_t* xq, int64_t ldxq,
                             float* scale_tok, int64_t M, int64_t K, q8_stream stream) {
    return quant_per_token_impl<false>(x, ldx, xq, ldxq, scale_tok, M, K, stream);
}

q8_status q8_quant_per_token_f16(const q8_f16* x, int64_t ldx, int8_t* xq, int64_t ldxq,
                                 float* scale_tok, int64_t M, int64_t K, q8_stream stream) {
    return quant_per_token_impl<true>(x, ldx, xq, ldxq, scale_tok, M, K, stream);
}

q8_status q8_scaled_mm(const int8_t* a, int64_t lda, const int8_t* b, int64_t ldb,
                       const float* scale_tok, const float* scale_ch, q8_bf16* c, int64_t ldc,
                       int64_t M, int64_t N, int64_t K, q8_stream stream) {
    return scaled_mm_impl<false>(a, lda, b, ldb, scale_tok, scale_ch, c, ldc, M, N, K, stream);
}

q8_status q8_scaled_mm_f16(const int8_t* a, int64_t lda, const int8_t* b, int64_t ldb,
                           const float* scale_tok, const float* scale_ch, q8_f16* c, int64_t ldc,
                           int64_t M, int64_t N, int64_t K, q8_stream stream) {
    return scaled_mm_impl<true>(a, lda, b, ldb, scale_tok, scale_ch, c, ldc, M, N, K, stream);
}

q8_status q8_scaled_mm_group128(const int8_t* a, int64_t lda, const int8_t* b, int64_t ldb,
                                const float* scale_tok, const float* scale_grp, q8_bf16* c,
                                int64_t ldc, int64_t M, int64_t N, int64_t K, q8_stream stream) {
    q8_status r = check_gemm(a, lda, 16, b, ldb, c, ldc, 8, M, N, K);
    if (r == Q8_OK && M > 0) r = check_scale(scale_tok);
    if (r == Q8_OK && M > 0) r = check_scale(scale_grp);
    if (r != Q8_OK || M == 0) return r;
    GemmArgs p{a, lda, b, ldb, scale_tok, scale_grp, c, ldc, (int)M, (int)N, (int)K};
    return hip_status(run_gemm_group(p, st(stream)));
}

q8_status q8_mm_i32(const int8_t* a, int64_t lda, const int8_t* b, int64_t ldb, int32_t* c,
                    int64_t ldc, int64_t M, int64_t N, int64_t K, q8_stream stream) {
    q8_status r = check_gemm(a, lda, 16, b, ldb, c, ldc, 4, M, N, K);
    if (r != Q8_OK || M == 0) return r;
    GemmArgs p{a, lda, b, ldb, nullptr, nullptr, c, ldc, (int)M, (int)N, (int)K};
    return hip_status(run_gemm_i8<EPI_I32>(p, st(stream)));
}

}  // extern "C"

namespace {
// Weight-only INT8 GEMM: bf16 or (F16) fp16 activations and outputs.
template <bool F16>
q8_status w8a16_impl(const uint16_t* x, int64_t ldx, const int8_t* w, int64_t ldw, const float* scale_ch,
                     uint16_t* c, int64_t ldc, int64_t M, int64_t N, int64_t K, q8_stream stream) {
    q8_status r = check_gemm(x, ldx, 8, w, ldw, c, ldc, 8, M, N, K);
    if (r == Q8_OK && M > 0) r = check_scale(scale_ch);
    if (r != Q8_OK || M == 0) return r;
    if (sg_fits((int)M, (int)N, (int)K, ldw, SG_MAX_M)) {  // few tokens: stream the weights once
        const StreamArgs q{x, ldx, w, ldw, nullptr, scale_ch, c, ldc, (int)M, (int)N, (int)K, 0, 0, 0};
        return hip_status(launch_stream<false, F16>(q, st(stream)));
    }
    // 65-112 tokens and under 64 channel tiles of 128: two streaming passes
    // (64 tokens, then the rest) instead of a tiled grid that leaves most
    // CUs idle (5120 x 17408: 113-129 against 165-200 us; from about 120
    // tokens the 32 x 128 tiles below are faster)
    if (M > SG_MAX_M && M <= 112 && (N + 127) / 128 < 64 &&
        sg_fits(SG_MAX_M, (int)N, (int)K, ldw, SG_MAX_M)) {
        for (int h = 0; h < 2; ++h) {
            const int64_t m0 = h * SG_MAX_M;
            const StreamArgs q{x + m0 * ldx, ldx, w, ldw, nullptr, scale_ch, c + m0 * ldc, ldc,
                               (int)(h ? M - SG_MAX_M : SG_MAX_M), (int)N, (int)K, 0, 0, 0};
            const hipError_t e = launch_stream<false, F16>(q, st(stream));
            if (e != hipSuccess) return Q8_EHIP;
        }
        return Q8_OK;
    }
    if (M <= 64) {
        W8A16Args p{x, ldx, w, ldw, scale_ch, c, ldc, (int)M, (int)N, (int)K};
        return hip_status(launch_w8a16<32, 128, 64, 1, 4, 8, F16>(p, st(stream)));
    }
    // the tiled kernel's 16-bit mode: activations addressed in bytes
    constexpr int E = F16 ? EPI_W8A16_F16 : EPI_W8A16;
    GemmArgs p{reinterpret_cast<const int8_t*>(x), 2 * ldx, w, ldw, nullptr, scale_ch, c, ldc,
               (int)M, (int)N, (int)K};
    if (!gemm_offsets_fit(p)) return Q8_EUNSUPPORTED;
    const int64_t nbm = (M + 255) / 256;
    const int64_t t128 = nbm * ((N + 127) / 128), t320 = nbm * ((N + 319) / 320);
    if (t128 < 256) {
        // Too few 256 x 128 tiles to fill the chip: 32 x 128 tiles while they
        // give at most 256 workgroups, else 64 x 128, else 128 x 128
        // (measured over 65-1024 tokens at 5120 x 17408, 5120 x 13824 and
        // 15360 x 5120: 10-16% faster than 128 x 128 where they apply).
        const int64_t nt = (N + 127) / 128;
        if ((M + 31) / 32 * nt <= 256) return hip_status(launch_gemm_i8<32, 128, 1, 4, E, 8>(p, st(stream)));
        if ((M + 63) / 64 * nt <= 256) return hip_status(launch_gemm_i8<64, 128, 2, 2, E, 8>(p, st(stream)));
        // one round of 256 x 128 tiles over at least 160 CUs beats two
        // 128 x 128 tiles per CU (5120 channels, K = 13824: 190 against
        // 214 us at 1024 tokens; 15360 x 5120 at 512 tokens: 93 against
        // 106 us); with fewer tiles it leaves too many CUs idle (K = 17408,
        // 512 tokens, 80 tiles: 249 against 200 us)
        if (t128 >= 160) return hip_status(launch_gemm_i8<256, 128, 4, 2, E, 8>(p, st(stream)));
        return hip_status(launch_gemm_i8<128, 128, 2, 2, E, 8>(p, st(stream)));
    }
    // Whole waves of 256 tiles; a wave of 256 x 320 tiles takes about 1.9
    // times as long as one of 256 x 128 (1.8-2.0 measured at 5120 channels
    // with K = 13824 and 17408 and at 15360 x 5120, 1024-8192 tokens).
    const int64_t w128 = (t128 + 255) / 256, w320 = (t320 + 255) / 256;
    if (190 * w320 < 100 * w128 && gemm_w16_offsets_fit(p)) return hip_status(launch_gemm_w16<F16>(p, st(stream)));
    return hip_status(launch_gemm_i8<256, 128, 4, 2, E, 8>(p, st(stream)));
}

template <bool F16>
q8_status w8a16_ws_impl(const uint16_t* x, int64_t ldx, const int8_t* w, int64_t ldw, const float* scale_ch,
                        uint16_t* c, int64_t ldc, int64_t M, int64_t N, int64_t K, void* ws, int64_t ws_bytes,
                        q8_stream stream) {
    q8_status r = check_gemm(x, ldx, 8, w, ldw, c, ldc, 8, M, N, K);
    if (r == Q8_OK && M > 0) r = check_scale(scale_ch);
    const SplitPlan sp = r == Q8_OK && M > 0 ? split_plan(M, N, K) : SplitPlan{};
    if (r == Q8_OK && M > 0) r = check_ws(ws, ws_bytes, sp.bytes);
    if (r != Q8_OK || M == 0) return r;
    GemmArgs p{reinterpret_cast<const int8_t*>(x), 2 * ldx, w, ldw, nullptr, scale_ch, c, ldc,
               (int)M, (int)N, (int)K};
    if (sp.ks < 2 || !gemm_offsets_fit(p))
        return w8a16_impl<F16>(x, ldx, w, ldw, scale_ch, c, ldc, M, N, K, stream);
    return hip_status(run_split<true, F16>(p, sp, ws, st(stream)));
}
}  // namespace

extern "C" {

q8_status w8a16_mm(const q8_bf16* x, int64_t ldx, const int8_t* w, int64_t ldw,
                   const float* scale_ch, q8_bf16* c, int64_t ldc, int64_t M, int64_t N, int64_t K,
                   q8_stream stream) {
    return w8a16_impl<false>(x, ldx, w, ldw, scale_ch, c, ldc, M, N, K, stream);
}

q8_status w8a16_mm_f16(const q8_f16* x, int64_t ldx, const int8_t* w, int64_t ldw,
                       const float* scale_ch, q8_f16* c, int64_t ldc, int64_t M, int64_t N, int64_t K,
                       q8_stream stream) {
    return w8a16_impl<true>(x, ldx, w, ldw, scale_ch, c, ldc, M, N, K, stream);
}

q8_status q8_quant_scaled_mm(const q8_bf16* x, int64_t ldx, const int8_t* b, int64_t ldb,
                             const float* scale_ch, q8_bf16* c, int64_t ldc, int8_t* xq,
                             float* scale_tok, int64_t M, int64_t N, int64_t K,
                             q8_stream stream) {
    return quant_scaled_mm_impl<false>(x, ldx, b, ldb, scale_ch, c, ldc, xq, scale_tok, M, N, K, stream);
}

q8_status q8_quant_scaled_mm_f16(const q8_f16* x, int64_t ldx, const int8_t* b, int64_t ldb,
                                 const float* scale_ch, q8_f16* c, int64_t ldc, int8_t* xq,
                                 float* scale_tok, int64_t M, int64_t N, int64_t K,
                                 q8_stream stream) {
    return quant_scaled_mm_impl<true>(x, ldx, b, ldb, scale_ch, c, ldc, xq, scale_tok, M, N, K, stream);
}

q8_status q8_quant_weight(const float* w, int64_t ldw, int8_t* wq, int64_t ldwq, float* scale,
                          int64_t N, int64_t K, int64_t group, q8_stream stream) {
    if (N < 0 || K < 0 || group < 0) return Q8_EINVAL;
    if (N == 0) return Q8_OK;
    if (!w || !wq || !scale || K == 0 || group == 0 || ldw < K || ldwq < K) return Q8_EINVAL;
    if (K % group != 0) return Q8_EUNSUPPORTED;
    if (!al(w, 4) || !al(scale, 4)) return Q8_EUNSUPPORTED;
    const int64_t spans = K / group;
    if (N * spans > INT32_MAX || group > INT32_MAX) return Q8_EUNSUPPORTED;
    hipLaunchKernelGGL(quant_weight_span, dim3((unsigned)(N * spans)), dim3(256), 0, st(stream),
                       w, ldw, wq, ldwq, scale, (int)group, (int)spans);
    return hip_status(hipGetLastError());
}

q8_status q8_smooth_fold(const q8_bf16* x, int64_t ldx, const float* w, int64_t ldw, float* s,
                         q8_bf16* xo, int64_t ldxo, float* wo, int64_t ldwo, int64_t M,
                         int64_t N, int64_t K, float cap, q8_stream stream) {
    if (M <= 0 || N <= 0 || K <= 0) return Q8_EINVAL;
    if (!x || !w || !s || !xo || !wo) return Q8_EINVAL;
    if (ldx < K || ldw < K || ldxo < K || ldwo < K || !(cap > 0.0f)) return Q8_EINVAL;
    if (!al(x, 2) || !al(xo, 2) || !al(w, 4) || !al(wo, 4) || !al(s, 4)) return Q8_EUNSUPPORTED;
    if (M > INT32_MAX / 2 || N > INT32_MAX / 2 || K > INT32_MAX / 2) return Q8_EUNSUPPORTED;
    hipStream_t h = st(stream);
    const int iK = (int)K, iM = (int)M, iN = (int)N;
    const unsigned kb = (unsigned)((K + 255) / 256);
    hipLaunchKernelGGL(fill_u32, dim3(kb), dim3(256), 0, h, reinterpret_cast<u32*>(s), 0u, iK);
    const int rows = 64;
    hipLaunchKernelGGL(colmax_bf16, dim3(kb, (unsigned)((M + rows - 1) / rows)), dim3(256), 0, h, x,
                       ldx, reinterpret_cast<u32*>(s), iM, iK, rows);
    hipLaunchKernelGGL(smooth_finalize, dim3(kb), dim3(256), 0, h, s, cap, iK);
    hipLaunchKernelGGL(fold_x_bf16, dim3(kb, (unsigned)(M < 65535 ? M : 65535)), dim3(256), 0, h, x,
                       ldx, s, xo, ldxo, iM, iK);
    hipLaunchKernelGGL(fold_w_f32, dim3(kb, (unsigned)(N < 65535 ? N : 65535)), dim3(256), 0, h, w,
                       ldw, s, wo, ldwo, iN, iK);
    return hip_status(hipGetLastError());
}

q8_status q8_rmsnorm_quant(const q8_bf16* x, int64_t ldx, q8_bf16* residual, int64_t ldr,
                           const q8_bf16* gamma, float eps, int8_t* xq, int64_t ldxq,
                           float* scale_tok, int64_t M, int64_t K, q8_stream stream) {
    if (M < 0 || K < 0) return Q8_EINVAL;
    if (M == 0) return Q8_OK;
    if (!x || !gamma || !xq || !scale_tok || K == 0) return Q8_EINVAL;
    if (ldx < K || ldxq < K || (residual && ldr < K) || !(eps >= 0.0f)) return Q8_EINVAL;
    if (K % 8 != 0 || K > NORM_MAX_K || M > INT32_MAX / 2) return Q8_EUNSUPPORTED;
    if (ldx % 8 != 0 || ldxq % 8 != 0 || (residual && ldr % 8 != 0)) return Q8_EUNSUPPORTED;
    if (!al(x, 16) || !al(gamma, 16) || !al(xq, 8) || !al(scale_tok, 4) ||
        (residual && !al(residual, 16)))
        return Q8_EUNSUPPORTED;
    return hip_status(launch_rmsnorm_quant(x, ldx, residual, residual ? ldr : 0, gamma, eps, xq,
                                           ldxq, scale_tok, (int)M, (int)K, st(stream)));
}

q8_status q8_quant_per_group128(const q8_bf16* x, int64_t ldx, int8_t* xq, int64_t ldxq,
                                float* scale_grp, int64_t M, int64_t K, q8_stream stream) {
    return quant_per_group128_impl<false>(x, ldx, xq, ldxq, scale_grp, M, K, stream);
}

q8_status q8_quant_per_group128_f16(const q8_f16* x, int64_t ldx, int8_t* xq, int64_t ldxq,
                                    float* scale_grp, int64_t M, int64_t K, q8_stream stream) {
    return quant_per_group128_impl<true>(x, ldx, xq, ldxq, scale_grp, M, K, stream);
}

q8_status q8_scaled_mm_group128_act(const int8_t* a, int64_t lda, const int8_t* b, int64_t ldb,
                                    const float* scale_x, const float* scale_w, q8_bf16* c,
                                    int64_t ldc, int64_t M, int64_t N, int64_t K,
                                    q8_stream stream) {
    return scaled_mm_group128_act_impl<false>(a, lda, b, ldb, scale_x, scale_w, c, ldc, M, N, K, stream);
}

q8_status q8_scaled_mm_group128_act_f16(const int8_t* a, int64_t lda, const int8_t* b, int64_t ldb,
                                        const float* scale_x, const float* scale_w, q8_f16* c,
                                        int64_t ldc, int64_t M, int64_t N, int64_t K,
                                        q8_stream stream) {
    return scaled_mm_group128_act_impl<true>(a, lda, b, ldb, scale_x, scale_w, c, ldc, M, N, K, stream);
}

q8_status q8_quant_fp8_per_group128(const q8_bf16* x, int64_t ldx, uint8_t* xq, int64_t ldxq,
                                    float* scale_grp, int64_t M, int64_t K, q8_stream stream) {
    if (M < 0 || K < 0) return Q8_EINVAL;
    if (M == 0) return Q8_OK;
    if (!x || !xq || !scale_grp || K == 0 || ldx < K || ldxq < K) return Q8_EINVAL;
    if (K % 128 != 0 || M > INT32_MAX / 2 || K > INT32_MAX / 2) return Q8_EUNSUPPORTED;
    if (ldx % 8 != 0 || ldxq % 8 != 0 || !al(x, 16) || !al(xq, 8) || !al(scale_grp, 4))
        return Q8_EUNSUPPORTED;
    const int64_t waves = M * ((K + 511) / 512);
    if ((waves + 3) / 4 > INT32_MAX) return Q8_EUNSUPPORTED;
    hipLaunchKernelGGL(quant_fp8_per_group128_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0,
                       st(stream), x, ldx, xq, ldxq, scale_grp, (int)M, (int)K);
    return hip_status(hipGetLastError());
}

q8_status q8_quant_weight_fp8_block128(const float* w, int64_t ldw, uint8_t* wq, int64_t ldwq,
                                       float* scale_blk, int64_t N, int64_t K, q8_stream stream) {
    if (N < 0 || K < 0) return Q8_EINVAL;
    if (N == 0) return Q8_OK;
    if (!w || !wq || !scale_blk || K == 0 || ldw < K || ldwq < K) return Q8_EINVAL;
    if (N % 128 != 0 || K % 128 != 0) return Q8_EUNSUPPORTED;
    if (!al(w, 4) || !al(scale_blk, 4)) return Q8_EUNSUPPORTED;
    const int64_t blocks = (N / 128) * (K / 128);
    if (blocks > INT32_MAX || K / 128 > INT32_MAX) return Q8_EUNSUPPORTED;
    hipLaunchKernelGGL(quant_weight_fp8_block_kernel, dim3((unsigned)blocks), dim3(256), 0, st(stream),
                       w, ldw, wq, ldwq, scale_blk, (int)(K / 128));
    return hip_status(hipGetLastError());
}

q8_status q8_quant_scaled_mm_noalloc(const q8_bf16* x, int64_t ldx, const int8_t* b, int64_t ldb,
                                     const float* scale_ch, q8_bf16* c, int64_t ldc, int8_t* xq,
                                     float* scale_tok, int64_t M, int64_t N, int64_t K, q8_stream stream) {
    // the checks of q8_quant_scaled_mm_ws, before any HIP call
    q8_status r = check_gemm(x, ldx, 8, b, ldb, c, ldc, 8, M, N, K);
    if (r == Q8_OK && M > 0) r = check_scale(scale_ch);
    if (r == Q8_OK && M > 0) r = check_scale(scale_tok);
    if (r == Q8_OK && M > 0 && !xq) r = Q8_EINVAL;
    if (r == Q8_OK && M > 0 && !al(xq, 16)) r = Q8_EUNSUPPORTED;
    if (r != Q8_OK || M == 0) return r;
    const int64_t need = split_plan(M, N, K).bytes;
    if (need > SCRATCH_BYTES) return Q8_EUNSUPPORTED;
    void* ws = nullptr;
    if (need > 0 && (ws = device_scratch(st(stream))) == nullptr) return Q8_EHIP;
    return quant_scaled_mm_ws_impl<false>(x, ldx, b, ldb, scale_ch, c, ldc, xq, scale_tok, M, N, K, ws,
                                          need > 0 ? SCRATCH_BYTES : 0, stream);
}

q8_status q8_wait_timeouts(uint32_t* count, int reset) {
    if (count == nullptr) return Q8_EINVAL;
    if (hipDeviceSynchronize() != hipSuccess) return Q8_EHIP;
    unsigned int v = 0;
    if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(sg_wait_timeouts), sizeof v) != hipSuccess) return Q8_EHIP;
    *count = v;
    if (reset && v != 0) {
        const unsigned int zero = 0;
        if (hipMemcpyToSymbol(HIP_SYMBOL(sg_wait_timeouts), &zero, sizeof zero) != hipSuccess) return Q8_EHIP;
    }
    return Q8_OK;
}

int64_t q8_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (M <= 0 || N <= 0 || K <= 0) return 0;
    return split_plan(M, N, K).bytes;
}

q8_status q8_scaled_mm_ws(const int8_t* a, int64_t lda, const int8_t* b, int64_t ldb,
                          const float* scale_tok, const float* scale_ch, q8_bf16* c, int64_t ldc,
                          int64_t M, int64_t N, int64_t K, void* workspace, int64_t workspace_bytes,
                          q8_stream stream) {
    return scaled_mm_ws_impl<false>(a, lda, b, ldb, scale_tok, scale_ch, c, ldc, M, N, K, workspace,
                                    workspace_bytes, stream);
}

q8_status q8_quant_scaled_mm_ws(const q8_bf16* x, int64_t ldx, const int8_t* b, int64_t ldb,
                                const float* scale_ch, q8_bf16* c, int64_t ldc, int8_t* xq,
                                float* scale_tok, int64_t M, int64_t N, int64_t K, void* workspace,
                                int64_t workspace_bytes, q8_stream stream) {
    return quant_scaled_mm_ws_impl<false>(x, ldx, b, ldb, scale_ch, c, ldc, xq, scale_tok, M, N, K, workspace,
                                          workspace_bytes, stream);
}

q8_status w8a16_mm_ws(const q8_bf16* x, int64_t ldx, const int8_t* w, int64_t ldw, const float* scale_ch,
                      q8_bf16* c, int64_t ldc, int64_t M, int64_t N, int64_t K, void* workspace,
                      int64_t workspace_bytes, q8_stream stream) {
    return w8a16_ws_impl<false>(x, ldx, w, ldw, scale_ch, c, ldc, M, N, K, workspace, workspace_bytes, stream);
}

q8_status q8_fp8_block_scaled_mm(const uint8_t* a, int64_t lda, const uint8_t* b, int64_t ldb,
                                 const float* scale_x, const float* scale_w, q8_bf16* c,
                                 int64_t ldc, int64_t M, int64_t N, int64_t K, q8_stream stream) {
    q8_status r = check_gemm(a, lda, 16, b, ldb, c, ldc, 8, M, N, K);
    if (r == Q8_OK && M > 0 && N % 128 != 0) r = Q8_EUNSUPPORTED;
    if (r == Q8_OK && M > 0) r = check_scale(scale_x);
    if (r == Q8_OK && M > 0) r = check_scale(scale_w);
    if (r != Q8_OK || M == 0) return r;
    GemmArgs p{reinterpret_cast<const int8_t*>(a), lda, reinterpret_cast<const int8_t*>(b), ldb,
               scale_x, scale_w, c, ldc, (int)M, (int)N, (int)K};
    if (!gemm_offsets_fit(p)) return Q8_EUNSUPPORTED;
    return hip_status(run_gemm_fp8_block(p, st(stream)));
}

}  // extern "C"
