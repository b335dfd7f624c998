/*
 * q8.h -- C ABI of libq8: the W8A8 INT8 linear layer (per-token dynamic
 * activations, per-channel or group-128 symmetric INT8 weights) and its
 * W8A16 companion, as hand-written HIP kernels for AMD MI355X (gfx950).
 *
 * The operation, as the pages state it (page title, section):
 *  - "Qwen3.8-27B -- SmoothQuant + activation-aware GPTQ, W8A8 INT8 (v3)",
 *    "Recipe": the W8A8 group uses INT8 per-channel symmetric weights and
 *    INT8 per-token dynamic activations; the W8A16 group keeps BF16
 *    activations with INT8 per-channel weights.  "Serving": W8A8 modules run
 *    a scaled INT8 GEMM, W8A16 modules a weight-only GEMM; the activation
 *    dtype is bfloat16.
 *  - "Qwen3.8-27B-INT8-W8A8", "Quantization": symmetric INT8 weights per
 *    output channel; INT8 dynamic per-token activations.
 *  - "Qwen3.8-27B-GPTQ-INT8-W8A8-GS128", "Quantization details": group size
 *    128, symmetric, desc_act false; true int8 x int8 compute needs one
 *    weight scale per 128-wide K block.  "Serving (vLLM, gfx908 fork)": the
 *    GEMM inputs are quantized to INT8 at run time.
 *  - "Qwen3.8-27B -- FP8 block + AWQ", "Recipe": every quantized dimension is
 *    divisible by 128; the smoothing fold (1/s into the input, s into the
 *    weight's input dimension) preserves the function.
 *
 * Conventions (all entry points):
 *  - Matrices are row-major with an explicit leading dimension in ELEMENTS.
 *    X is [M,K] (tokens x input features), W is [N,K] (output channels x
 *    input features, the PyTorch Linear layout, K contiguous), Y is [M,N].
 *  - Every pointer is a DEVICE pointer owned by the caller.  The library
 *    never allocates, frees or synchronizes; a call validates its arguments,
 *    enqueues its kernels on `stream` (0 = the null stream) and returns.
 *    Faults inside a kernel surface at the caller's next synchronization.
 *  - Errors are return codes; nothing is printed and nothing throws.
 *    Validation happens before any HIP call, so an invalid call enqueues
 *    nothing and leaves the outputs untouched.
 *  - M == 0 is a valid empty call (returns Q8_OK, enqueues nothing).
 *  - bf16 values are passed as raw 16-bit patterns (q8_bf16).
 *  - NaN or infinite inputs are outside the contract (results undefined,
 *    no fault).
 *  - Calls on one stream are ordered; calls that write the same output on
 *    different streams race.
 */
#ifndef Q8_H
#define Q8_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    Q8_OK = 0,
    Q8_EINVAL = 1,       /* null pointer, negative or zero size, ld < row */
    Q8_EUNSUPPORTED = 2, /* a shape or alignment rule below is broken     */
    Q8_EHIP = 3          /* the HIP runtime refused a launch              */
} q8_status;

typedef uint16_t q8_bf16; /* raw bfloat16 bits */
typedef uint16_t q8_f16;  /* raw IEEE fp16 (binary16) bits */
typedef void *q8_stream;  /* hipStream_t; 0 selects the null stream */

/* Largest K of any GEMM entry point: 128*128*K stays below 2^31, so the
 * int32 accumulator cannot overflow even for the code -128. */
#define Q8_MAX_K 130944

/* GEMM operands are addressed with 32-bit offsets: (rows + 256) * ld * elem
 * bytes of every matrix operand must stay below this bound (2 GiB minus
 * one 128-byte stage of slack); larger operands give Q8_EUNSUPPORTED. */
#define Q8_MAX_OPERAND_BYTES (((int64_t)1 << 31) - 256)

/* Text for a status code (static storage; never NULL). */
const char *q8_status_str(q8_status s);

/* ------------------------------------------------------------------------
 * q8_quant_per_token -- per-token dynamic symmetric INT8 quantization.
 * For every row m of X:
 *   a = max_k |x[m,k]|                    (exact, bf16 widened to fp32)
 *   scale_tok[m] = a / 127                (one correctly rounded fp32 division;
 *                                           0 when a == 0)
 *   xq[m,k] = clamp(rne(x[m,k] / scale_tok[m]), -127, 127)
 *             (correctly rounded fp32 quotient, round half to even; a zero
 *              row gives all-zero codes)
 * Cited: "...W8A8 INT8 (v3)", "Recipe" (INT8 per-token dynamic
 * activations); "Qwen3.8-27B-INT8-W8A8", "Quantization".
 *   x        [M, ldx]  bf16, read
 *   xq       [M, ldxq] int8, written (columns 0..K-1)
 *   scale_tok[M]       fp32, written
 * Rules: M >= 0, K >= 1, ldx >= K, ldxq >= K.  Any K and alignment is
 * accepted (a vector path is taken when rows are 16-byte aligned).
 * ---------------------------------------------------------------------- */
q8_status q8_quant_per_token(const q8_bf16 *x, int64_t ldx, int8_t *xq,
                             int64_t ldxq, float *scale_tok, int64_t M,
                             int64_t K, q8_stream stream);

/* ------------------------------------------------------------------------
 * q8_scaled_mm -- INT8 x INT8 -> INT32 GEMM with the per-token x
 * per-channel scale epilogue, bf16 out:
 *   acc[m,n] = sum_k a[m,k] * b[n,k]                     (exact int32)
 *   c[m,n]   = bf16_rne( ((float)acc * scale_tok[m]) * scale_ch[n] )
 *              (fp32 products in this order; no bias)
 * Cited: "...W8A8 INT8 (v3)", "Recipe" and "Serving" (INT8 x INT8 on
 * tensor cores, bfloat16 dtype); "Qwen3.8-27B-INT8-W8A8", "Quantization".
 *   a         [M, lda] int8 activations codes (full int8 range accepted)
 *   b         [N, ldb] int8 weight codes
 *   scale_tok [M] fp32, scale_ch [N] fp32
 *   c         [M, ldc] bf16, written (columns 0..N-1)
 * Rules: M >= 0; N >= 16 and N % 16 == 0; K >= 128, K % 128 == 0,
 * K <= Q8_MAX_K; lda, ldb >= K and multiples of 16; ldc >= N and a
 * multiple of 8; a, b 16-byte aligned; c 16-byte aligned; scales 4-byte
 * aligned; (M + 256) * lda and (N + 256) * ldb below Q8_MAX_OPERAND_BYTES.
 * Else Q8_EUNSUPPORTED (or Q8_EINVAL for null/negative).
 * ---------------------------------------------------------------------- */
q8_status q8_scaled_mm(const int8_t *a, int64_t lda, const int8_t *b,
                       int64_t ldb, const float *scale_tok,
                       const float *scale_ch, q8_bf16 *c, int64_t ldc,
                       int64_t M, int64_t N, int64_t K, q8_stream stream);

/* ------------------------------------------------------------------------
 * q8_scaled_mm_group128 -- INT8 GEMM with one weight scale per (output
 * channel, contiguous 128-wide K block), bf16 out.  For g = 0..K/128-1 in
 * ascending order:
 *   p_g = sum_{k in [128g, 128g+128)} a[m,k] * b[n,k]     (exact int32)
 *   acc = fmaf((float)p_g, scale_grp[n*(K/128) + g], acc) (acc starts at 0)
 * then c[m,n] = bf16_rne(acc * scale_tok[m]).
 * Cited: "Qwen3.8-27B-GPTQ-INT8-W8A8-GS128", "Quantization details" (group
 * size 128, symmetric, desc_act false; one weight scale per 128-wide K
 * block for true int8 x int8 compute).
 *   scale_grp [N, K/128] fp32 row-major (contiguous).
 * Rules: as q8_scaled_mm.
 * ---------------------------------------------------------------------- */
q8_status q8_scaled_mm_group128(const int8_t *a, int64_t lda,
                                const int8_t *b, int64_t ldb,
                                const float *scale_tok,
                                const float *scale_grp, q8_bf16 *c,
                                int64_t ldc, int64_t M, int64_t N, int64_t K,
                                q8_stream stream);

/* ------------------------------------------------------------------------
 * w8a16_mm -- weight-only INT8 GEMM with bf16 activations, bf16 out:
 *   c[m,n] = bf16_rne( scale_ch[n] * sum_k x[m,k] * (bf16)w[n,k] )
 * The int8 -> bf16 weight conversion is exact; products and sums run on
 * bf16 matrix cores with fp32 accumulation (summation order is the
 * hardware's); the channel scale is applied once in the fp32 epilogue.
 * Cited: "...W8A8 INT8 (v3)", "Recipe" (W8A16 group: INT8 per-channel
 * weights, BF16 activations); "lued/Qwen3.8-27B-INT8-W8A16-MTP", "Why W8A16
 * on Ampere" (weight-only kernels rebuild weights for a 16-bit GEMM).
 *   x [M, ldx] bf16, w [N, ldw] int8, scale_ch [N] fp32, c [M, ldc] bf16.
 * Rules: as q8_scaled_mm, with ldx >= K a multiple of 8 and x 16-byte
 * aligned.
 * ---------------------------------------------------------------------- */
q8_status w8a16_mm(const q8_bf16 *x, int64_t ldx, const int8_t *w,
                   int64_t ldw, const float *scale_ch, q8_bf16 *c,
                   int64_t ldc, int64_t M, int64_t N, int64_t K,
                   q8_stream stream);

/* ------------------------------------------------------------------------
 * q8_quant_scaled_mm -- the whole W8A8 layer in one call: per-token
 * quantization of x (as q8_quant_per_token) followed by q8_scaled_mm.
 * The quantized activations and their scales are written to the caller's
 * xq / scale_tok buffers (they are outputs, and the GEMM's inputs).  For
 * M <= 8 and K up to 8192 (a few hundred workgroups of channels at most)
 * one kernel does both (every
 * workgroup quantizes the rows for itself while its weights stream in), and
 * so does one for small layers (M <= 16, K below 1024, at most 16 MB of
 * weights).  Otherwise two kernels run back to back on `stream`: the row quantizer,
 * then the GEMM of q8_scaled_mm (for few tokens a weight-streaming kernel
 * that reads each weight byte once, else the tiled GEMM).
 *   x [M, ldx] bf16; b [N, ldb] int8; scale_ch [N]; c [M, ldc] bf16;
 *   xq [M, K] int8 (dense, ld = K), scale_tok [M] fp32.
 * Rules: as q8_scaled_mm, plus ldx >= K a multiple of 8, x 16-byte aligned.
 * ---------------------------------------------------------------------- */
q8_status q8_quant_scaled_mm(const q8_bf16 *x, int64_t ldx, const int8_t *b,
                             int64_t ldb, const float *scale_ch, q8_bf16 *c,
                             int64_t ldc, int8_t *xq, float *scale_tok,
                             int64_t M, int64_t N, int64_t K,
                             q8_stream stream);

/* ------------------------------------------------------------------------
 * q8_mm_i32 -- the raw INT32 product acc[m,n] = sum_k a[m,k]*b[n,k]
 * (exact), written as int32 [M, ldc].  A test hook for the INT8 mainloop.
 * Rules: as q8_scaled_mm, with ldc >= N a multiple of 4.
 * ---------------------------------------------------------------------- */
q8_status q8_mm_i32(const int8_t *a, int64_t lda, const int8_t *b,
                    int64_t ldb, int32_t *c, int64_t ldc, int64_t M,
                    int64_t N, int64_t K, q8_stream stream);

/* ------------------------------------------------------------------------
 * q8_wait_timeouts -- diagnostics of the few-token weight-streaming kernels
 * (q8_scaled_mm, q8_quant_scaled_mm and w8a16_mm at up to 64 tokens, and in
 * two passes up to 128).  Their waves hand weight segments over through
 * counters in on-chip memory; every wait on them is bounded (about 2^20
 * polls, some 30 ms), so a broken hand-over gives a wrong result instead of
 * a hung device.  A wave that has run for more than 10 ms -- which no call
 * takes unless a wait gave up -- adds one to a per-device count.
 * This call waits for the current device to finish its work
 * (hipDeviceSynchronize), stores that device's count in *count and, with
 * reset nonzero, sets it back to 0.  The count is 0 in correct operation.
 * Errors: Q8_EINVAL for a NULL count; Q8_EHIP if HIP refuses the
 * synchronization or the copy.  Not for hot paths: it synchronizes.
 * ---------------------------------------------------------------------- */
q8_status q8_wait_timeouts(uint32_t *count, int reset);

/* ------------------------------------------------------------------------
 * Split K with a caller workspace.  Between the few-token kernels and the
 * large tiles (roughly 24-512 tokens at the model's shapes) the output has
 * too few tiles to keep 256 compute units busy.  The _ws entry points then
 * split K: ks workgroups per output tile each sum a contiguous K range into
 * a plane of the caller's workspace, and a second kernel adds the planes and
 * applies the epilogue.  They compute exactly what their namesakes without
 * _ws compute (same arguments, layouts, rules and errors, plus the two
 * workspace arguments):
 *  - q8_scaled_mm_ws, q8_quant_scaled_mm_ws: the planes hold exact int32
 *    partial sums, added in int32, so acc and the bf16 output are the same
 *    bits as q8_scaled_mm's ("...W8A8 INT8 (v3)", "Recipe" and "Serving").
 *  - w8a16_mm_ws: the planes hold fp32 partial sums added in fp32 in plane
 *    order; the result is W8A16's fp32-accumulated sum in another order
 *    ("lued/Qwen3.8-27B-INT8-W8A16-MTP", "Why W8A16 on Ampere").
 * Ownership: the workspace is the caller's device memory, read and written
 * only during the call's kernels (no state is kept between calls, nothing
 * needs clearing).  Calls that share one workspace must be ordered (the
 * same stream); concurrent calls need their own.
 * ---------------------------------------------------------------------- */

/* Bytes of workspace the _ws entry points need for an (M, N, K) problem:
 * 0 when none of them splits K at that size (then the workspace may be
 * NULL), else ks * M * N * 4 for the library's split count ks (2 <= ks <=
 * 10; at 24-64 tokens the W8A8 calls keep the weight-streaming kernel, and
 * leave the workspace unused, where that kernel runs).  Never more than
 * 31,457,280 bytes (30 MiB).  Nonpositive sizes give 0. */
int64_t q8_workspace_bytes(int64_t M, int64_t N, int64_t K);

/* As q8_scaled_mm, with workspace [workspace_bytes] (device, 16-byte
 * aligned).  Errors: those of q8_scaled_mm; Q8_EINVAL when a workspace is
 * needed and workspace is NULL or workspace_bytes < q8_workspace_bytes(M,
 * N, K); Q8_EUNSUPPORTED when it is misaligned. */
q8_status q8_scaled_mm_ws(const int8_t *a, int64_t lda, const int8_t *b,
                          int64_t ldb, const float *scale_tok,
                          const float *scale_ch, q8_bf16 *c, int64_t ldc,
                          int64_t M, int64_t N, int64_t K, void *workspace,
                          int64_t workspace_bytes, q8_stream stream);

/* As q8_quant_scaled_mm (the whole layer in one call), with a workspace as
 * q8_scaled_mm_ws. */
q8_status q8_quant_scaled_mm_ws(const q8_bf16 *x, int64_t ldx,
                                const int8_t *b, int64_t ldb,
                                const float *scale_ch, q8_bf16 *c,
                                int64_t ldc, int8_t *xq, float *scale_tok,
                                int64_t M, int64_t N, int64_t K,
                                void *workspace, int64_t workspace_bytes,
                                q8_stream stream);

/* As w8a16_mm, with a workspace as q8_scaled_mm_ws. */
q8_status w8a16_mm_ws(const q8_bf16 *x, int64_t ldx, const int8_t *w,
                      int64_t ldw, const float *scale_ch, q8_bf16 *c,
                      int64_t ldc, int64_t M, int64_t N, int64_t K,
                      void *workspace, int64_t workspace_bytes,
                      q8_stream stream);

/* ------------------------------------------------------------------------
 * q8_quant_scaled_mm_noalloc -- for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): q8_quant_scaled_mm_ws with the library's own
 * workspace, a device array of Q8_NOALLOC_MAX_WORKSPACE bytes that each
 * GPU holds from the time the library is loaded there until the process
 * ends.  Same arguments, result and errors as q8_quant_scaled_mm (the
 * caller still passes the output, xq and scale_tok buffers), plus
 * Q8_EUNSUPPORTED when the problem would need more than that workspace
 * (never for the library's current split rule, whose largest need is 30
 * MiB) and Q8_EHIP when HIP refuses the lookup of the array's address.
 * It calls no allocating routine: the first call on a device looks up the
 * array's device address (hipGetSymbolAddress) and keeps it.  Every call on
 * one GPU uses that GPU's one array, which holds the last call's partial
 * sums (each call writes every value it reads, so nothing needs clearing):
 * calls that overlap on one GPU (different streams) race; order them.
 * ---------------------------------------------------------------------- */
#define Q8_NOALLOC_MAX_WORKSPACE ((int64_t)32 << 20)

q8_status q8_quant_scaled_mm_noalloc(const q8_bf16 *x, int64_t ldx,
                                     const int8_t *b, int64_t ldb,
                                     const float *scale_ch, q8_bf16 *c,
                                     int64_t ldc, int8_t *xq,
                                     float *scale_tok, int64_t M, int64_t N,
                                     int64_t K, q8_stream stream);

/* ------------------------------------------------------------------------
 * q8_quant_weight -- offline symmetric INT8 weight quantization of an fp32
 * weight W [N,K]: one scale per (row, contiguous span of `group` columns),
 *   scale[n*(K/group) + g] = absmax(span) / 127   (correctly rounded)
 *   wq[n,k] = clamp(rne(w[n,k] / scale), -127, 127)   (0 for a zero span)
 * group == K gives per-output-channel scales; group == 128 the group-128
 * layout [N, K/128].
 * Cited: "...W8A8 INT8 (v3)", "Recipe" and "Qwen3.8-27B-INT8-W8A8",
 * "Quantization" (per-channel symmetric); "Qwen3.8-27B-GPTQ-INT8-W8A8-GS128",
 * "Quantization details" (group 128, symmetric, natural K order).
 *   w [N, ldw] fp32; wq [N, ldwq] int8; scale [N * K/group] fp32.
 * Rules: N >= 0, K >= 1, group >= 1 dividing K, ldw, ldwq >= K.
 * ---------------------------------------------------------------------- */
q8_status q8_quant_weight(const float *w, int64_t ldw, int8_t *wq,
                          int64_t ldwq, float *scale, int64_t N, int64_t K,
                          int64_t group, q8_stream stream);

/* ------------------------------------------------------------------------
 * q8_smooth_fold -- offline smoothing fold of an activation sample X [M,K]
 * and a weight W [N,K]:
 *   s[j]   = min(cap, sqrtf(max_m |x[m,j]|))     (0 for an all-zero column,
 *                                                  which must not be folded)
 *   xo[m,j] = bf16_rne(x[m,j] / s[j])            (correctly rounded quotient)
 *   wo[n,j] = w[n,j] * s[j]                      (fp32 product)
 * Cited: "...W8A8 INT8 (v3)", "Recipe" (SmoothQuant folds, scales capped at
 * 16); "Qwen3.8-27B -- FP8 block + AWQ", "Recipe" (1/s into the input side,
 * s into the weight's input dimension; function-preserving).  The exponent
 * 0.5 on the plain column maximum stands in for the pages' per-hook alpha
 * and windowed statistic.
 *   x [M, ldx] bf16; w [N, ldw] fp32; s [K] fp32 out; xo [M, ldxo] bf16 out;
 *   wo [N, ldwo] fp32 out.  xo may equal x and wo may equal w (in place).
 * Rules: M, N >= 1, K >= 1, lds >= K, cap > 0.
 * ---------------------------------------------------------------------- */
q8_status q8_smooth_fold(const q8_bf16 *x, int64_t ldx, const float *w,
                         int64_t ldw, float *s, q8_bf16 *xo, int64_t ldxo,
                         float *wo, int64_t ldwo, int64_t M, int64_t N,
                         int64_t K, float cap, q8_stream stream);

/* ------------------------------------------------------------------------
 * q8_rmsnorm_quant -- residual add + RMSNorm + per-token INT8 quantization
 * in one pass: the step that feeds a W8A8 linear layer, whose smoothing
 * divisor is folded into gamma offline.  Per row m (K a multiple of 8):
 *   h = bf16_rne(x + residual), residual := h   (residual != NULL)
 *   h = x                                       (residual == NULL)
 *   ss = sum of h[k]^2 (each square exact), added in fp32: its value is
 *        the exact sum S of the squares up to the error of the summation,
 *        |ss - S| <= n_d * 2^-24 * (1 + n_d * 2^-24) * S with
 *        n_d = 8 * ceil(K / 512) + 6 (64 running partial sums of at most
 *        8 * ceil(K/512) squares each, combined pairwise in 6 levels)
 *   rstd = 1 / sqrtf(ss / K + eps)              (correctly rounded)
 *   y[k] = bf16_rne((h[k] * rstd) * gamma[k])   (fp32 products)
 *   xq, scale_tok = q8_quant_per_token of the bf16 row y
 * The plain definition takes ss as S rounded once to fp32; the codes and
 * scale of a row are those of that definition at the kernel's own ss, which
 * lies within the bound above (a different ss can move y across a bf16
 * rounding boundary, so rows may differ from the definition's at the
 * correctly rounded S while matching it at a nearby fp32 ss).
 * Cited: "...W8A8 INT8 (v3)", "Recipe" (smoothing folded into the preceding
 * norm); "Qwen3.8-27B -- FP8 block + AWQ", "Recipe" (the same fold);
 * "Qwen3.8-27B-GPTQ-INT8-W8A8-GS128", "Serving (vLLM, gfx908 fork)"
 * (residual add, RMSNorm and INT8 quantization fused into one step).
 *   x        [M, ldx]  bf16, read
 *   residual [M, ldr]  bf16, read and overwritten with h (may be NULL; may
 *                      be the same buffer as x)
 *   gamma    [K]       bf16, read
 *   xq       [M, ldxq] int8, written; scale_tok [M] fp32, written
 * Rules: M >= 0, 8 <= K <= 8192 with K % 8 == 0 (else Q8_EUNSUPPORTED);
 * eps >= 0 (else Q8_EINVAL); ldx, ldr >= K and multiples of 8 with x,
 * residual and gamma 16-byte aligned; ldxq >= K, a multiple of 8, xq
 * 8-byte aligned.  The normalized row itself is not stored.  With eps == 0
 * an all-zero row has no defined norm (0 * inf) and its outputs are
 * unspecified; with eps > 0 it gives scale 0 and all-zero codes.
 * ---------------------------------------------------------------------- */
q8_status q8_rmsnorm_quant(const q8_bf16 *x, int64_t ldx, q8_bf16 *residual,
                           int64_t ldr, const q8_bf16 *gamma, float eps,
                           int8_t *xq, int64_t ldxq, float *scale_tok,
                           int64_t M, int64_t K, q8_stream stream);

/* ------------------------------------------------------------------------
 * q8_quant_per_group128 -- per-token-per-group dynamic INT8 quantization:
 * one scale per (row m, 128-wide K block g), each block quantized like a
 * token row of 128 values:
 *   scale_grp[m*(K/128) + g] = max_{k in block} |x[m,k]| / 127 (correctly
 *                              rounded; 0 for an all-zero block)
 *   xq[m,k] = clamp(rne(x[m,k] / scale), -127, 127)
 * Cited: "Qwen3.8-27B-GPTQ-INT8-W8A8-GS128", "Serving (vLLM, gfx908 fork)"
 * (per-group INT8 quantization of the activations) and "Quantization
 * details" (group size 128); "Qwen3.8-27B -- FP8 block + AWQ", "Recipe"
 * (dynamic per-group activation scales).
 *   x [M, ldx] bf16; xq [M, ldxq] int8; scale_grp [M, K/128] fp32 (dense)
 * Rules: M >= 0; K % 128 == 0 (else Q8_EUNSUPPORTED); ldx, ldxq >= K and
 * multiples of 8; x 16-byte, xq 8-byte aligned.
 * ---------------------------------------------------------------------- */
q8_status q8_quant_per_group128(const q8_bf16 *x, int64_t ldx, int8_t *xq,
                                int64_t ldxq, float *scale_grp, int64_t M,
                                int64_t K, q8_stream stream);

/* ------------------------------------------------------------------------
 * q8_scaled_mm_group128_act -- INT8 GEMM with one scale per (token, 128-wide
 * K block) on the activations and one per (channel, 128-wide K block) on
 * the weights, bf16 out.  For g = 0..K/128-1 in ascending order:
 *   p_g = sum_{k in [128g, 128g+128)} a[m,k] * b[n,k]        (exact int32)
 *   acc = fmaf((float)p_g, fl32(scale_x[m,g] * scale_w[n,g]), acc)  (from 0)
 * then c[m,n] = bf16_rne(acc).  (The two block scales are multiplied first,
 * then applied to the block sum with one rounding.)
 * Cited: as q8_quant_per_group128 and q8_scaled_mm_group128.
 *   a [M, lda] int8 codes of q8_quant_per_group128; b [N, ldb] int8;
 *   scale_x [M, K/128], scale_w [N, K/128] fp32 row-major; c [M, ldc] bf16.
 * Rules: as q8_scaled_mm_group128.
 * ---------------------------------------------------------------------- */
q8_status q8_scaled_mm_group128_act(const int8_t *a, int64_t lda,
                                    const int8_t *b, int64_t ldb,
                                    const float *scale_x, const float *scale_w,
                                    q8_bf16 *c, int64_t ldc, int64_t M,
                                    int64_t N, int64_t K, q8_stream stream);

/* ------------------------------------------------------------------------
 * fp16 variant.  The same layer with IEEE fp16 activations and fp16
 * outputs: "Qwen3.8-27B-GPTQ-INT8-W8A8-GS128", "Serving (vLLM, gfx908
 * fork)" serves in half precision (the model's native dtype) with every
 * GEMM input quantized to INT8 at run time.  Each call computes exactly
 * what its bf16 namesake computes, with two changes: activations are fp16
 * values (decoded exactly to fp32), and the fp32 result is rounded to fp16
 * (round to nearest even; magnitudes from 65520 up become infinity) instead
 * of bf16.  Arguments, layouts, alignment rules and errors are those of the
 * bf16 call; every q8_f16 pointer takes the place of the q8_bf16 one.
 * ---------------------------------------------------------------------- */

/* As q8_quant_per_token, on fp16 activations. */
q8_status q8_quant_per_token_f16(const q8_f16 *x, int64_t ldx, int8_t *xq,
                                 int64_t ldxq, float *scale_tok, int64_t M,
                                 int64_t K, q8_stream stream);

/* As q8_scaled_mm, writing fp16 outputs:
 *   c[m,n] = fp16_rne(fl32(fl32((float)acc * scale_tok[m]) * scale_ch[n])) */
q8_status q8_scaled_mm_f16(const int8_t *a, int64_t lda, const int8_t *b,
                           int64_t ldb, const float *scale_tok,
                           const float *scale_ch, q8_f16 *c, int64_t ldc,
                           int64_t M, int64_t N, int64_t K, q8_stream stream);

/* As q8_quant_scaled_mm (the whole layer in one call), fp16 in and out. */
q8_status q8_quant_scaled_mm_f16(const q8_f16 *x, int64_t ldx,
                                 const int8_t *b, int64_t ldb,
                                 const float *scale_ch, q8_f16 *c, int64_t ldc,
                                 int8_t *xq, float *scale_tok, int64_t M,
                                 int64_t N, int64_t K, q8_stream stream);

/* As q8_quant_per_group128, on fp16 activations. */
q8_status q8_quant_per_group128_f16(const q8_f16 *x, int64_t ldx, int8_t *xq,
                                    int64_t ldxq, float *scale_grp, int64_t M,
                                    int64_t K, q8_stream stream);

/* As q8_scaled_mm_group128_act, writing fp16 outputs (c = fp16_rne(f)). */
q8_status q8_scaled_mm_group128_act_f16(const int8_t *a, int64_t lda,
                                        const int8_t *b, int64_t ldb,
                                        const float *scale_x,
                                        const float *scale_w, q8_f16 *c,
                                        int64_t ldc, int64_t M, int64_t N,
                                        int64_t K, q8_stream stream);

/* As w8a16_mm, with fp16 activations and fp16 outputs:
 *   c[m,n] = fp16_rne( scale_ch[n] * sum_k x[m,k] * (fp16)w[n,k] )
 * The int8 -> fp16 weight conversion is exact; products and sums run on
 * fp16 matrix cores with fp32 accumulation.  fp16 keeps 3 more significand
 * bits than bf16, so the result carries less rounding than w8a16_mm's on
 * the same values; it overflows to infinity from 65520 up. */
q8_status w8a16_mm_f16(const q8_f16 *x, int64_t ldx, const int8_t *w,
                       int64_t ldw, const float *scale_ch, q8_f16 *c,
                       int64_t ldc, int64_t M, int64_t N, int64_t K,
                       q8_stream stream);

/* ------------------------------------------------------------------------
 * FP8 block W8A8.  E4M3 is the OCP 8-bit float: sign, 4 exponent bits (bias
 * 7), 3 mantissa bits, largest finite value 448 (bytes 0x7F and 0xFF are
 * NaN), subnormal quantum 2^-9.  A block scale is fl32(absmax / 448) (0 for
 * an all-zero block, whose codes are +0); a code is the E4M3 value nearest
 * to the correctly rounded fp32 quotient x / scale, ties to the even
 * mantissa, magnitudes from 448 up saturating to 448, the sign kept (so -0
 * and tiny negative values give the -0 byte 0x80).
 * Cited: "Qwen3.8-27B -- FP8 block + AWQ", "Recipe" (FP8 block-scaled
 * [128,128] weights with dynamic per-group activations; every quantized
 * dimension divisible by 128) and its "KV cache" section (E4M3 scaled by
 * amax/448).
 * ---------------------------------------------------------------------- */

/* q8_quant_fp8_per_group128 -- dynamic FP8 activations, one scale per
 * (token m, 128-wide K block g):
 *   scale_grp[m*(K/128) + g] = max_{k in block} |x[m,k]| / 448
 *   xq[m,k] = E4M3 code of x[m,k] / scale_grp[m*(K/128) + g]
 *   x [M, ldx] bf16; xq [M, ldxq] E4M3 bytes; scale_grp [M, K/128] fp32
 *   (dense), all written by the call.
 * Rules: M >= 0; K % 128 == 0 (else Q8_EUNSUPPORTED); ldx, ldxq >= K and
 * multiples of 8; x 16-byte, xq 8-byte, scale_grp 4-byte aligned. */
q8_status q8_quant_fp8_per_group128(const q8_bf16 *x, int64_t ldx,
                                    uint8_t *xq, int64_t ldxq,
                                    float *scale_grp, int64_t M, int64_t K,
                                    q8_stream stream);

/* q8_quant_weight_fp8_block128 -- offline FP8 weights, one scale per
 * [128,128] block (rows 128*nb .. 128*nb+127, columns 128*g .. 128*g+127):
 *   scale_blk[nb*(K/128) + g] = max |w| over the block / 448
 *   wq[n,k] = E4M3 code of w[n,k] / scale_blk[(n/128)*(K/128) + k/128]
 *   w [N, ldw] fp32 (PyTorch Linear layout, K contiguous); wq [N, ldwq]
 *   E4M3 bytes; scale_blk [N/128, K/128] fp32 row-major.
 * Rules: N >= 0; N and K multiples of 128 (else Q8_EUNSUPPORTED); ldw,
 * ldwq >= K; w and scale_blk 4-byte aligned.  Not on the timed path. */
q8_status q8_quant_weight_fp8_block128(const float *w, int64_t ldw,
                                       uint8_t *wq, int64_t ldwq,
                                       float *scale_blk, int64_t N, int64_t K,
                                       q8_stream stream);

/* q8_fp8_block_scaled_mm -- FP8 block-scaled GEMM, bf16 out.  The value
 * computed is
 *   c[m,n] = sum_g scale_x[m,g] * scale_w[n/128, g] * P_g,
 *   P_g    = sum_{k in [128g, 128g+128)} a[m,k] * b[n,k]  (E4M3 values)
 * on the FP8 matrix cores: each P_g is an MFMA sum, folded in ascending g
 * as f = fmaf(P_g, fl32(scale_x * scale_w), f) from 0; c = bf16_rne(f).
 * The matrix cores do not sum E4M3 products in fp32: each group of 8
 * consecutive products is aligned to the group's largest product with 13
 * fractional bits and truncated (measured on MI355X).  So c differs from
 * the exact value by up to sum_g |scale product| * sum over groups of
 * sum_k min(|a*b|, 2^-12 * max_group |a*b|) (about 1e-3 of sum |a*b| at
 * most), plus fp32 rounding of the fold and the final bf16 rounding.
 *   a [M, lda] E4M3 codes of q8_quant_fp8_per_group128; b [N, ldb] E4M3
 *   codes of q8_quant_weight_fp8_block128; scale_x [M, K/128] and scale_w
 *   [N/128, K/128] fp32 row-major; c [M, ldc] bf16, written.
 * Rules: as q8_scaled_mm, and N % 128 == 0 (else Q8_EUNSUPPORTED).  A NaN
 * byte (0x7F, 0xFF) in an operand gives NaN outputs in its row or column. */
q8_status q8_fp8_block_scaled_mm(const uint8_t *a, int64_t lda,
                                 const uint8_t *b, int64_t ldb,
                                 const float *scale_x, const float *scale_w,
                                 q8_bf16 *c, int64_t ldc, int64_t M, int64_t N,
                                 int64_t K, q8_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* Q8_H */
