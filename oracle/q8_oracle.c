/*
 * q8_oracle.c -- the CPU oracle for the W8A8 INT8 linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the HIP library and includes nothing from it.
 *
 * Every routine is a plain, slow, obviously correct loop nest written from the
 * definitions on the pages (IEEE fp32 arithmetic, round-to-nearest-even, no
 * reordering beyond what the definition states).  Build with
 *     gcc -O2 -fopenmp -ffp-contract=off -fno-fast-math -shared -fPIC
 * so that no multiply-add is fused unless fmaf() is written, and so that the
 * rounding mode is the default round-to-nearest-even (checked at run time by
 * q8o_env_ok()).  OpenMP splits only independent outer loops (rows), which
 * cannot change any result.
 *
 * Sources (page title, then section):
 *  [P1] "Qwen3.8-27B -- SmoothQuant + activation-aware GPTQ, W8A8 INT8 (v3)",
 *       section "Recipe": SmoothQuant folds with scales capped at 16; INT8
 *       per-channel symmetric weights and INT8 per-token dynamic activations
 *       for the W8A8 group; INT8 per-channel weights with BF16 activations for
 *       the W8A16 group.  Section "Serving": --dtype bfloat16.
 *  [P2] "lued/Qwen3.8-27B-INT8-W8A16-MTP", section "Why W8A16 on Ampere":
 *       weight-only kernels rebuild the weights for a 16-bit GEMM.
 *  [P3] "Qwen3.8-27B -- FP8 block + AWQ", section "Recipe": the smoothing fold
 *       preserves the function; the new weight over the old one is a
 *       separable row-times-column scale.
 *  [P4] "Qwen3.8-27B-INT8-W8A8", section "Quantization": symmetric INT8
 *       weights per output channel, INT8 dynamic per-token activations.
 *  [P5] "Qwen3.8-27B-GPTQ-INT8-W8A8-GS128", section "Quantization details":
 *       8 bits, group size 128, symmetric, desc_act false (groups are the
 *       natural contiguous K blocks); true int8 x int8 compute with one weight
 *       scale per 128-wide K block.
 *
 * Readings where the pages are silent (each one is also listed in the design
 * notes):
 *  - the activation scale is absmax/127 computed as ONE correctly rounded
 *    fp32 division; a row whose absmax is 0 gets scale 0 and all-zero codes;
 *  - a code is round-half-to-even of the correctly rounded fp32 quotient
 *    x/s (a division, not a multiply by a reciprocal), clamped to [-127,127];
 *  - (float)acc is the round-to-nearest-even int32 -> fp32 conversion;
 *  - the per-channel epilogue is bf16_rne( (((float)acc) * s_tok) * s_ch ),
 *    fp32 products in that order; there is no bias;
 *  - the group-128 epilogue accumulates in fp32 with one fmaf per group in
 *    ascending group order, starting from 0, then multiplies by s_tok once;
 *  - W8A16 converts the int8 weight exactly and applies the channel scale in
 *    the epilogue; the oracle returns the fp64 value of that sum;
 *  - the smoothing scale is s_j = min(cap, sqrtf(max_m |X[m,j]|)) with cap 16
 *    (exponent 0.5 on the plain column maximum), X' = bf16_rne(X / s_j) and
 *    W' = fl32(W * s_j).
 *  - FP8 block W8A8 ([P3] "Recipe": FP8 block-scaled [128,128] weights with
 *    dynamic per-group activations; its "KV cache" section scales E4M3 by
 *    amax/448): E4M3 is the OCP 8-bit float with 4 exponent bits (bias 7)
 *    and 3 mantissa bits, largest finite value 448; a scale is
 *    fl32(absmax / 448) over the block (0 for an all-zero block, whose codes
 *    are all +0); a code is the E4M3 value nearest to the correctly rounded
 *    fp32 quotient x/s, ties to the even mantissa, magnitudes from 448 up
 *    saturating to 448, the sign always kept (so -0 and tiny negatives give
 *    the -0 code).
 */
#include <fenv.h>
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- bf16 -- */

/* bf16 -> fp32 is exact: the bf16 bits are the top half of the fp32 bits. */
static float bf16_bits_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* fp32 -> bf16 with round-to-nearest, ties to even, on the bit pattern.
 * NaN is kept a (quiet) NaN; infinities and overflow follow IEEE. */
uint16_t q8o_f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0)
        return (uint16_t)((u >> 16) | 0x0040u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

float q8o_bf16_to_f32(uint16_t b) { return bf16_bits_to_f32(b); }

/* ---------------------------------------------------------------- fp16 -- */
/* IEEE binary16: sign, 5 exponent bits (bias 15), 10 fraction bits.  The
 * fp16 variant of the layer takes fp16 activations and writes fp16
 * outputs ("Qwen3.8-27B-GPTQ-INT8-W8A8-GS128", "Serving (vLLM, gfx908
 * fork)": --dtype half is the model's native dtype, GEMM inputs quantized
 * to INT8 at run time). */

/* fp16 -> fp32 is exact, decoded by the definition. */
float q8o_f16_to_f32(uint16_t h)
{
    const int E = (h >> 10) & 31, f = h & 1023;
    double v;
    if (E == 31)
        v = f ? NAN : INFINITY;
    else if (E == 0)
        v = ldexp((double)f, -24);
    else
        v = ldexp((double)(1024 + f), E - 25);
    return (float)((h & 0x8000) ? -v : v);
}

/* fp32 -> fp16, round to nearest, ties to even, by the definition:
 * subnormal quantum 2^-24, magnitudes from 65520 (the midpoint above the
 * largest finite value 65504) up overflow to infinity, NaN stays NaN. */
uint16_t q8o_f32_to_f16(float f)
{
    if (isnan(f))
        return 0x7E00;
    const uint16_t sign = signbit(f) ? 0x8000 : 0;
    const double a = fabs((double)f);
    if (a >= 65520.0)
        return sign | 0x7C00;
    if (a < ldexp(1.0, -14))  /* subnormal range (exact scaling) */
        return sign | (uint16_t)nearbyint(a * ldexp(1.0, 24));
    int ex;
    frexp(a, &ex);            /* a = fr * 2^ex, fr in [0.5, 1) */
    int e = ex - 1;           /* 2^e <= a < 2^(e+1) */
    double mant = nearbyint(ldexp(a, 10 - e)); /* in [1024, 2048] */
    if (mant == 2048.0) {
        mant = 1024.0;
        e += 1;
    }
    if (e > 15)
        return sign | 0x7C00;
    return sign | (uint16_t)(((e + 15) << 10) | ((int)mant - 1024));
}

/* 1 if the FPU is in round-to-nearest-even mode (every routine relies on it). */
int q8o_env_ok(void) { return fegetround() == FE_TONEAREST; }

/* Threads the parallel loops below run on. */
int q8o_threads(void) { return omp_get_max_threads(); }

/* ------------------------------------------------- symmetric INT8 codes -- */

/* Absmax scale of n fp32 values: s = fl32(absmax / 127); 0 for a zero span.
 * [P1 "Recipe"; P4 "Quantization"; P5 "Quantization details": symmetric] */
static float absmax_scale(const float *v, int64_t n)
{
    float a = 0.0f;
    for (int64_t k = 0; k < n; ++k) {
        float m = fabsf(v[k]);
        if (m > a)
            a = m;
    }
    return a / 127.0f; /* one IEEE division; a == 0 gives 0 */
}

/* q = clamp(rne(fl32(x / s)), -127, 127); s == 0 gives 0. */
static int8_t code_of(float x, float s)
{
    if (s == 0.0f)
        return 0;
    float t = x / s;          /* correctly rounded fp32 quotient */
    float r = nearbyintf(t);  /* round half to even (default mode) */
    if (r > 127.0f)
        r = 127.0f;
    if (r < -127.0f)
        r = -127.0f;
    return (int8_t)r;
}

/* Per-token dynamic quantization of a 16-bit activation matrix whose
 * values `dec` decodes (bf16 or fp16).
 * x: [M][K] bits, row-major.  xq: [M][K] int8.  s_tok: [M] fp32.
 * [P1 "Recipe": INT8 per-token dynamic activations; P4 "Quantization"] */
static void quant_per_token_fmt(const uint16_t *x, float (*dec)(uint16_t),
                                int64_t M, int64_t K, int8_t *xq,
                                float *s_tok)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        float *row = (float *)malloc((size_t)K * sizeof(float));
        for (int64_t k = 0; k < K; ++k)
            row[k] = dec(x[m * K + k]);
        float s = absmax_scale(row, K);
        s_tok[m] = s;
        for (int64_t k = 0; k < K; ++k)
            xq[m * K + k] = code_of(row[k], s);
        free(row);
    }
}

void q8o_quant_per_token(const uint16_t *x, int64_t M, int64_t K,
                         int8_t *xq, float *s_tok)
{
    quant_per_token_fmt(x, bf16_bits_to_f32, M, K, xq, s_tok);
}

void q8o_quant_per_token_f16(const uint16_t *x, int64_t M, int64_t K,
                             int8_t *xq, float *s_tok)
{
    quant_per_token_fmt(x, q8o_f16_to_f32, M, K, xq, s_tok);
}

/* Offline symmetric weight quantization of an fp32 weight W [N][K].
 * group == K: one scale per output channel (s: [N]).
 * group == 128: one scale per (channel, contiguous 128-wide K block),
 * s: [N][K/128] row-major.
 * [P1 "Recipe" and P4 "Quantization": per-channel symmetric;
 *  P5 "Quantization details": group size 128, symmetric, desc_act false]
 * Returns 0, or -1 if group does not divide K. */
int q8o_quant_weight(const float *w, int64_t N, int64_t K, int64_t group,
                     int8_t *wq, float *s)
{
    if (group <= 0 || K % group != 0)
        return -1;
    const int64_t G = K / group;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t g = 0; g < G; ++g) {
            const float *span = w + n * K + g * group;
            float sg = absmax_scale(span, group);
            s[n * G + g] = sg;
            for (int64_t k = 0; k < group; ++k)
                wq[n * K + g * group + k] = code_of(span[k], sg);
        }
    }
    return 0;
}

/* ---------------------------------------------------------- INT8 GEMM -- */

/* INT8 GEMM: acc[m][n] = sum_k a[m][k] * b[n][k], exact (int64 loop).
 * a: [M][K] int8, b: [N][K] int8 (PyTorch Linear layout), acc: [M][N] int32.
 * [P1 "Serving": INT8 x INT8 on tensor cores; P5: true int8 x int8 compute]
 * Returns 0, or -1 if some sum does not fit in int32 (then acc is clamped). */
int q8o_mm_i32(const int8_t *a, const int8_t *b, int64_t M, int64_t N,
               int64_t K, int32_t *acc)
{
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            int64_t t = 0;
            for (int64_t k = 0; k < K; ++k)
                t += (int64_t)a[m * K + k] * (int64_t)b[n * K + k];
            if (t > INT32_MAX) {
                t = INT32_MAX;
                bad = 1;
            }
            if (t < INT32_MIN) {
                t = INT32_MIN;
                bad = 1;
            }
            acc[m * N + n] = (int32_t)t;
        }
    }
    return bad ? -1 : 0;
}

/* Per-channel epilogue: y[m][n] = bf16_rne( fl32( fl32((float)acc * s_tok[m]) * s_ch[n] ) ).
 * [P1 "Recipe": per-token x per-channel scales; "Serving": bf16 dtype] */
void q8o_epilogue_channel(const int32_t *acc, const float *s_tok,
                          const float *s_ch, int64_t M, int64_t N,
                          uint16_t *y)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            float v = (float)acc[m * N + n]; /* RNE int32 -> fp32 */
            v = v * s_tok[m];
            v = v * s_ch[n];
            y[m * N + n] = q8o_f32_to_bf16(v);
        }
    }
}

/* GEMM and per-channel epilogue in one call, without storing the int32
 * matrix; `enc` rounds the fp32 result to the 16-bit output format. */
static int scaled_mm_fmt(const int8_t *a, const int8_t *b, const float *s_tok,
                         const float *s_ch, int64_t M, int64_t N, int64_t K,
                         uint16_t (*enc)(float), uint16_t *y)
{
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            int64_t t = 0;
            for (int64_t k = 0; k < K; ++k)
                t += (int64_t)a[m * K + k] * (int64_t)b[n * K + k];
            if (t > INT32_MAX || t < INT32_MIN)
                bad = 1;
            float v = (float)(int32_t)t;
            v = v * s_tok[m];
            v = v * s_ch[n];
            y[m * N + n] = enc(v);
        }
    }
    return bad ? -1 : 0;
}

int q8o_scaled_mm(const int8_t *a, const int8_t *b, const float *s_tok,
                  const float *s_ch, int64_t M, int64_t N, int64_t K,
                  uint16_t *y)
{
    return scaled_mm_fmt(a, b, s_tok, s_ch, M, N, K, q8o_f32_to_bf16, y);
}

/* The same with fp16 outputs (fp16 RNE of the same fp32 value). */
int q8o_scaled_mm_f16(const int8_t *a, const int8_t *b, const float *s_tok,
                      const float *s_ch, int64_t M, int64_t N, int64_t K,
                      uint16_t *y)
{
    return scaled_mm_fmt(a, b, s_tok, s_ch, M, N, K, q8o_f32_to_f16, y);
}

/* GEMM with group-128 weights.  For g = 0 .. K/128-1 in order:
 *   p_g = sum_{k in [128g, 128g+128)} a[m][k]*b[n][k]   (int32, exact;
 *         |p_g| <= 128*128*128 < 2^24 so (float)p_g is exact)
 *   acc = fmaf((float)p_g, s_grp[n][g], acc)           (acc starts at 0)
 * then y = bf16_rne( fl32(acc * s_tok[m]) ).
 * [P5 "Quantization details": one weight scale per 128-wide K block]
 * Returns 0, or -1 if K is not a multiple of 128. */
int q8o_scaled_mm_group128(const int8_t *a, const int8_t *b,
                           const float *s_tok, const float *s_grp,
                           int64_t M, int64_t N, int64_t K, uint16_t *y)
{
    if (K % 128 != 0)
        return -1;
    const int64_t G = K / 128;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            float acc = 0.0f;
            for (int64_t g = 0; g < G; ++g) {
                int32_t p = 0;
                for (int64_t k = g * 128; k < g * 128 + 128; ++k)
                    p += (int32_t)a[m * K + k] * (int32_t)b[n * K + k];
                acc = fmaf((float)p, s_grp[n * G + g], acc);
            }
            float v = acc * s_tok[m];
            y[m * N + n] = q8o_f32_to_bf16(v);
        }
    }
    return 0;
}

/* W8A16 reference.  y_ref[m][n] = s_ch[n] * sum_k x[m][k] * q[n][k] in
 * fp64 (each product is exact in fp64), plus the magnitude sum
 * mag[m][n] = s_ch[n] * sum_k |x[m][k]| * |q[n][k]| that sizes the
 * floating-point error bound of any summation order.
 * [P1 "Recipe": W8A16 group, INT8 per-channel weights with BF16 activations;
 *  P2 "Why W8A16 on Ampere": weights are rebuilt for a 16-bit GEMM] */
static void w8a16_ref_fmt(const uint16_t *x, float (*dec)(uint16_t),
                          const int8_t *q, const float *s_ch, int64_t M,
                          int64_t N, int64_t K, double *y_ref, double *mag)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double t = 0.0, u = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double xv = (double)dec(x[m * K + k]);
                double qv = (double)q[n * K + k];
                t += xv * qv;
                u += fabs(xv) * fabs(qv);
            }
            y_ref[m * N + n] = (double)s_ch[n] * t;
            if (mag)
                mag[m * N + n] = (double)s_ch[n] * u;
        }
    }
}

void q8o_w8a16_ref(const uint16_t *x, const int8_t *q, const float *s_ch,
                   int64_t M, int64_t N, int64_t K, double *y_ref,
                   double *mag)
{
    w8a16_ref_fmt(x, bf16_bits_to_f32, q, s_ch, M, N, K, y_ref, mag);
}

/* The same with fp16 activations ("lued/Qwen3.8-27B-INT8-W8A16-MTP": FP16
 * or BF16 activations). */
void q8o_w8a16_ref_f16(const uint16_t *x, const int8_t *q, const float *s_ch,
                       int64_t M, int64_t N, int64_t K, double *y_ref,
                       double *mag)
{
    w8a16_ref_fmt(x, q8o_f16_to_f32, q, s_ch, M, N, K, y_ref, mag);
}

/* ------------------------------------------------------ smoothing fold -- */

/* s_j = min(cap, sqrtf(max_m |x[m][j]|)), j < K.  [P1 "Recipe": SmoothQuant
 * folds, scales capped at 16; the plain column maximum with exponent 0.5
 * stands in for the per-hook alpha and windowed statistic.]
 * Returns 0, or -1 if some s_j is 0 (an all-zero column cannot be folded). */
int q8o_smooth_scales(const uint16_t *x, int64_t M, int64_t K, float cap,
                      float *s)
{
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t j = 0; j < K; ++j) {
        float a = 0.0f;
        for (int64_t m = 0; m < M; ++m) {
            float v = fabsf(bf16_bits_to_f32(x[m * K + j]));
            if (v > a)
                a = v;
        }
        float r = sqrtf(a);
        if (r > cap)
            r = cap;
        s[j] = r;
        if (!(r > 0.0f))
            bad = 1;
    }
    return bad ? -1 : 0;
}

/* X' = bf16_rne(fl32(x / s_j)).  [P3 "Recipe": 1/s folded into the input] */
void q8o_smooth_fold_x(const uint16_t *x, const float *s, int64_t M,
                       int64_t K, uint16_t *xo)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t j = 0; j < K; ++j)
            xo[m * K + j] = q8o_f32_to_bf16(bf16_bits_to_f32(x[m * K + j]) / s[j]);
}

/* W' = fl32(w * s_j).  [P3 "Recipe": s folded into the next linear's input
 * dimension] */
void q8o_smooth_fold_w(const float *w, const float *s, int64_t N, int64_t K,
                       float *wo)
{
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t j = 0; j < K; ++j)
            wo[n * K + j] = w[n * K + j] * s[j];
}

/* ------------------------------- residual add + RMSNorm + per-token quant --
 * The step before a W8A8 linear layer in the model: the normalization whose
 * weight absorbs the smoothing divisor, fused with the per-token INT8 quant
 * of its output [P1 "Recipe": smoothing folded into the preceding norm; P3
 * "Recipe": the same fold; P5 "Serving (vLLM, gfx908 fork)": residual add,
 * RMSNorm and INT8 quantization fused into one output step].
 * Readings (the pages give no RMSNorm numerics; this is the plain RMSNorm):
 *  - with a residual stream: h = bf16_rne(fl32(x) + fl32(res)), and res := h;
 *    without one: h = x;
 *  - ss = the exact sum of h[k]^2 over the row, rounded once to fp32 (round
 *    to nearest even).  Each square of a bf16 value is exact, so ss is the
 *    sum of squares as a real number, with one rounding;
 *  - rstd = 1 / sqrtf(ss / K + eps) (correctly rounded division and root);
 *  - y[k] = bf16_rne(fl32(fl32(h[k] * rstd) * gamma[k]));
 *  - then the per-token quantization above, applied to the bf16 row y.
 * A summation in fp32 in any other order gives a value near ss; what a
 * kernel's order may change is stated where the kernel is declared, and the
 * tests accept the codes of every fp32 ss within that bound
 * (q8o_rmsnorm_quant_at_ss computes them). */

/* Exact sum of the squares of n bf16 values, rounded once to fp32.
 * A nonzero bf16 magnitude is m * 2^e with an integer m < 2^8 (m = 128 + the
 * 7 stored bits for a normal value with biased exponent E, e = E - 134; the
 * stored bits alone with e = -133 for a subnormal), so its square is the
 * integer m^2 < 2^16 times 2^(2e), 2e >= -266.  The squares are added as
 * integers into a fixed-point register whose bit i stands for 2^(i - 266):
 * 2e + 266 >= 0, and the largest square, below 2^256, plus 2^13 more of them
 * stays below 2^270, so 9 limbs of 64 bits (576 bits) hold every sum exactly.
 * The register is then rounded to the fp32 grid: 24 significant bits, or the
 * subnormal quantum 2^-149, ties to even. */
#define SSQ_LIMBS 9
#define SSQ_BIAS 266

static int ssq_bit(const uint64_t *acc, int i)
{
    return (int)((acc[i >> 6] >> (i & 63)) & 1u);
}

static float sum_squares_bf16_rn(const uint16_t *h, int64_t n)
{
    uint64_t acc[SSQ_LIMBS];
    memset(acc, 0, sizeof acc);
    for (int64_t k = 0; k < n; ++k) {
        const uint32_t b = h[k] & 0x7FFFu;
        if (b == 0) continue;
        const uint32_t E = b >> 7, f = b & 0x7Fu;
        const uint64_t m = E ? 128u + f : f;
        const int e = E ? (int)E - 134 : -133;
        const uint64_t sq = m * m;
        const int pos = 2 * e + SSQ_BIAS;
        int limb = pos >> 6;
        const int sh = pos & 63;
        uint64_t lo = sq << sh, hi = sh ? sq >> (64 - sh) : 0;
        /* add (hi:lo) at limb, then carry upwards */
        uint64_t old = acc[limb];
        acc[limb] = old + lo;
        uint64_t carry = acc[limb] < old;
        for (++limb; limb < SSQ_LIMBS && (hi | carry); ++limb) {
            old = acc[limb];
            const uint64_t add = hi + carry;  /* hi < 2^16: no overflow */
            acc[limb] = old + add;
            carry = acc[limb] < old;
            hi = 0;
        }
    }
    int top = -1;
    for (int i = SSQ_LIMBS * 64 - 1; i >= 0; --i)
        if (ssq_bit(acc, i)) { top = i; break; }
    if (top < 0) return 0.0f;
    /* value = acc * 2^-266; its leading bit has exponent top - 266 */
    int qe = top - SSQ_BIAS - 23;          /* exponent of the last kept bit */
    if (qe < -149) qe = -149;
    const int qp = qe + SSQ_BIAS;          /* its position in the register */
    uint64_t keep = 0;
    for (int i = top; i >= qp; --i) keep = (keep << 1) | (uint64_t)ssq_bit(acc, i);
    int half = 0, sticky = 0;
    if (qp >= 1) {
        half = ssq_bit(acc, qp - 1);
        for (int i = qp - 2; i >= 0 && !sticky; --i) sticky = ssq_bit(acc, i);
    }
    if (half && (sticky || (keep & 1u))) keep += 1;
    const double v = ldexp((double)keep, qe);  /* exact: keep <= 2^24 */
    return v >= 0x1p128 ? INFINITY : (float)v;
}

/* ss of each of M rows of K bf16 values (the exact sum, rounded once). */
void q8o_sum_squares_bf16(const uint16_t *h, int64_t M, int64_t K, float *ss)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) ss[m] = sum_squares_bf16_rn(h + m * K, K);
}

/* The normalization and the quantization of M rows h [M][K] (bf16, the row
 * after the residual add) for given sums of squares ss [M]:
 *   rstd = 1 / sqrtf(ss / K + eps); y = bf16_rne((h * rstd) * gamma);
 *   xq, s = the per-token quantization of y.  y_out (optional) receives y. */
int q8o_rmsnorm_quant_at_ss(const uint16_t *h, const uint16_t *gamma,
                            float eps, int64_t M, int64_t K, const float *ss,
                            int8_t *xq, float *s, uint16_t *y_out)
{
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t m = 0; m < M; ++m) {
        float *yf = (float *)malloc((size_t)K * sizeof(float));
        if (!yf) { bad = 1; continue; }
        const float var = ss[m] / (float)K;
        const float rstd = 1.0f / sqrtf(var + eps);
        for (int64_t k = 0; k < K; ++k) {
            const float t = bf16_bits_to_f32(h[m * K + k]) * rstd;
            const uint16_t yb = q8o_f32_to_bf16(t * bf16_bits_to_f32(gamma[k]));
            yf[k] = bf16_bits_to_f32(yb);
            if (y_out) y_out[m * K + k] = yb;
        }
        const float sc = absmax_scale(yf, K);
        s[m] = sc;
        for (int64_t k = 0; k < K; ++k) xq[m * K + k] = code_of(yf[k], sc);
        free(yf);
    }
    return bad ? -2 : 0;
}

/* The whole step: residual add (res may be NULL; it is overwritten with h),
 * exact sum of squares, normalization and quantization.  ss_out and y_out
 * are optional.  Returns -1 if K is not a multiple of 8 (the vector layout
 * of the step's entry point). */
int q8o_rmsnorm_quant(const uint16_t *x, uint16_t *res, const uint16_t *gamma,
                      float eps, int64_t M, int64_t K, int8_t *xq, float *s,
                      uint16_t *y_out, float *ss_out)
{
    if (K % 8 != 0) return -1;
    uint16_t *h = (uint16_t *)malloc((size_t)(M * K > 0 ? M * K : 1) * sizeof(uint16_t));
    float *ss = (float *)malloc((size_t)(M > 0 ? M : 1) * sizeof(float));
    if (!h || !ss) { free(h); free(ss); return -2; }
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < K; ++k) {
            if (res) {
                const float sum = bf16_bits_to_f32(x[m * K + k]) + bf16_bits_to_f32(res[m * K + k]);
                h[m * K + k] = q8o_f32_to_bf16(sum);
                res[m * K + k] = h[m * K + k];
            } else {
                h[m * K + k] = x[m * K + k];
            }
        }
    q8o_sum_squares_bf16(h, M, K, ss);
    const int rc = q8o_rmsnorm_quant_at_ss(h, gamma, eps, M, K, ss, xq, s, y_out);
    if (ss_out) memcpy(ss_out, ss, (size_t)M * sizeof(float));
    free(h);
    free(ss);
    return rc;
}

/* --------------------- per-token-per-group activations, group-128 weights --
 * Activations quantized with one scale per (token, 128-wide K block) and
 * weights with one scale per (channel, 128-wide K block) [P5 "Serving
 * (vLLM, gfx908 fork)": per-group INT8 quant-out before the GEMM; P3
 * "Recipe": dynamic per-group activation scales; P5 "Quantization details":
 * group size 128, natural K order].
 * Quantization: every 128-wide block of a row is quantized like a token row
 * on its own: s_x[m][g] = fl32(absmax / 127), codes RNE of fl32(x / s),
 * clamped to [-127, 127]; s_x is [M][K/128] row-major. */
static int quant_per_group128_fmt(const uint16_t *x, float (*dec)(uint16_t),
                                  int64_t M, int64_t K, int8_t *xq, float *s_x)
{
    if (K % 128 != 0) return -1;
    const int64_t G = K / 128;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        float v[128];
        for (int64_t g = 0; g < G; ++g) {
            for (int k = 0; k < 128; ++k) v[k] = dec(x[m * K + g * 128 + k]);
            const float sc = absmax_scale(v, 128);
            s_x[m * G + g] = sc;
            for (int k = 0; k < 128; ++k) xq[m * K + g * 128 + k] = code_of(v[k], sc);
        }
    }
    return 0;
}

int q8o_quant_per_group128(const uint16_t *x, int64_t M, int64_t K,
                           int8_t *xq, float *s_x)
{
    return quant_per_group128_fmt(x, bf16_bits_to_f32, M, K, xq, s_x);
}

int q8o_quant_per_group128_f16(const uint16_t *x, int64_t M, int64_t K,
                               int8_t *xq, float *s_x)
{
    return quant_per_group128_fmt(x, q8o_f16_to_f32, M, K, xq, s_x);
}

/* GEMM with both scales per 128-wide K block.  For g = 0 .. K/128-1 in
 * order (reading: the two scales are multiplied first, as block-scaled
 * GEMMs do, then one fused multiply-add per block):
 *   p_g = sum_{k in [128g, 128g+128)} a[m][k]*b[n][k]    (exact int32)
 *   acc = fmaf((float)p_g, fl32(s_x[m][g] * s_w[n][g]), acc)   (from 0)
 * y = bf16_rne(acc).  Returns -1 if K is not a multiple of 128. */
static int scaled_mm_group128_act_fmt(const int8_t *a, const int8_t *b,
                                      const float *s_x, const float *s_w,
                                      int64_t M, int64_t N, int64_t K,
                                      uint16_t (*enc)(float), uint16_t *y)
{
    if (K % 128 != 0) return -1;
    const int64_t G = K / 128;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            float acc = 0.0f;
            for (int64_t g = 0; g < G; ++g) {
                int32_t p = 0;
                for (int64_t k = g * 128; k < g * 128 + 128; ++k)
                    p += (int32_t)a[m * K + k] * (int32_t)b[n * K + k];
                const float sc = s_x[m * G + g] * s_w[n * G + g];
                acc = fmaf((float)p, sc, acc);
            }
            y[m * N + n] = enc(acc);
        }
    }
    return 0;
}

int q8o_scaled_mm_group128_act(const int8_t *a, const int8_t *b,
                               const float *s_x, const float *s_w,
                               int64_t M, int64_t N, int64_t K, uint16_t *y)
{
    return scaled_mm_group128_act_fmt(a, b, s_x, s_w, M, N, K, q8o_f32_to_bf16, y);
}

int q8o_scaled_mm_group128_act_f16(const int8_t *a, const int8_t *b,
                                   const float *s_x, const float *s_w,
                                   int64_t M, int64_t N, int64_t K, uint16_t *y)
{
    return scaled_mm_group128_act_fmt(a, b, s_x, s_w, M, N, K, q8o_f32_to_f16, y);
}

/* ------------------------------------------------------- FP8 block W8A8 -- */

/* Value of an E4M3 code, by its definition: sign bit 7, exponent field
 * E = bits 6..3 (bias 7), mantissa m = bits 2..0.  E == 0: m * 2^-9
 * (subnormal); E == 15 with m == 7: NaN; otherwise (1 + m/8) * 2^(E-7).
 * [P3 "Recipe": FP8 block weights; its "KV cache" section: E4M3, 448] */
double q8o_e4m3_value(uint8_t c)
{
    const int E = (c >> 3) & 15, m = c & 7;
    double v;
    if (E == 15 && m == 7)
        return NAN;
    if (E == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp((double)(8 + m), E - 10);
    return (c & 0x80) ? -v : v;
}

/* E4M3 code of v: the nearest value of the non-negative codes 0x00..0x7E
 * (found by bisection: their values increase with the code), ties to the
 * code with an even mantissa, |v| >= 448 saturating to 0x7E, sign bit from
 * v.  NaN gives 0x7F. */
uint8_t q8o_e4m3_rne(float v)
{
    if (isnan(v))
        return 0x7F;
    const uint8_t sign = signbit(v) ? 0x80 : 0x00;
    const double a = fabs((double)v);
    if (a >= 448.0)
        return sign | 0x7E;
    int lo = 0, hi = 0x7E; /* largest c with value(c) <= a */
    while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if (q8o_e4m3_value((uint8_t)mid) <= a)
            lo = mid;
        else
            hi = mid - 1;
    }
    int c = lo;
    const double below = a - q8o_e4m3_value((uint8_t)c);       /* exact */
    const double above = q8o_e4m3_value((uint8_t)(c + 1)) - a; /* exact */
    if (below > above || (below == above && (c & 1)))
        c += 1;
    return sign | (uint8_t)c;
}

/* Absmax scale for E4M3: fl32(absmax / 448); 0 for a zero span. */
static float absmax_scale_e4m3(const float *v, int64_t n)
{
    float a = 0.0f;
    for (int64_t k = 0; k < n; ++k) {
        float m = fabsf(v[k]);
        if (m > a)
            a = m;
    }
    return a / 448.0f;
}

/* E4M3 code of x under scale s: the code of the correctly rounded quotient;
 * s == 0 (an all-zero span) gives +0. */
static uint8_t e4m3_code_of(float x, float s)
{
    if (s == 0.0f)
        return 0x00;
    return q8o_e4m3_rne(x / s);
}

/* Dynamic per-token-per-group FP8 activations: every 128-wide K block of a
 * bf16 row gets s_x[m][g] = fl32(absmax / 448) and E4M3 codes of x / s.
 * x: [M][K] bf16 bits; xq: [M][K] E4M3 bytes; s_x: [M][K/128].
 * [P3 "Recipe": dynamic per-group activations, dimensions divisible by 128]
 * Returns -1 if K is not a multiple of 128. */
int q8o_quant_fp8_per_group128(const uint16_t *x, int64_t M, int64_t K,
                               uint8_t *xq, float *s_x)
{
    if (K % 128 != 0)
        return -1;
    const int64_t G = K / 128;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        float v[128];
        for (int64_t g = 0; g < G; ++g) {
            for (int k = 0; k < 128; ++k)
                v[k] = bf16_bits_to_f32(x[m * K + g * 128 + k]);
            const float sc = absmax_scale_e4m3(v, 128);
            s_x[m * G + g] = sc;
            for (int k = 0; k < 128; ++k)
                xq[m * K + g * 128 + k] = e4m3_code_of(v[k], sc);
        }
    }
    return 0;
}

/* Offline FP8 block weights: one scale per [128,128] block of the fp32
 * weight W [N][K], s_w[nb][g] = fl32(absmax over rows 128nb.. and columns
 * 128g.. / 448), row-major [N/128][K/128]; wq [N][K] E4M3 codes.
 * [P3 "Recipe": FP8 block-scaled [128,128] weights, scales from the weight
 * tensor alone]  Returns -1 unless N and K are multiples of 128. */
int q8o_quant_weight_fp8_block128(const float *w, int64_t N, int64_t K,
                                  uint8_t *wq, float *s_w)
{
    if (N % 128 != 0 || K % 128 != 0)
        return -1;
    const int64_t NB = N / 128, G = K / 128;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t nb = 0; nb < NB; ++nb) {
        for (int64_t g = 0; g < G; ++g) {
            float a = 0.0f;
            for (int64_t n = nb * 128; n < nb * 128 + 128; ++n)
                for (int64_t k = g * 128; k < g * 128 + 128; ++k) {
                    float m = fabsf(w[n * K + k]);
                    if (m > a)
                        a = m;
                }
            const float sc = a / 448.0f;
            s_w[nb * G + g] = sc;
            for (int64_t n = nb * 128; n < nb * 128 + 128; ++n)
                for (int64_t k = g * 128; k < g * 128 + 128; ++k)
                    wq[n * K + k] = e4m3_code_of(w[n * K + k], sc);
        }
    }
    return 0;
}

/* FP8 block-scaled GEMM, the value the method defines:
 *   y[m][n] = sum_g s_x[m][g] * s_w[n/128][g] * P_g,
 *   P_g     = sum_{k in [128g, 128g+128)} e4m3(a[m][k]) * e4m3(b[n][k]).
 * P_g is exact in fp64 (each product of two E4M3 values is a multiple of
 * 2^-18 below 2^18, so a block sum needs at most 44 bits); the scale
 * products and the sum over g are fp64.  mag (if not NULL) receives
 * sum_g |s_x * s_w| * sum_k |e4m3(a) * e4m3(b)|, the size that error bounds
 * of fp32 accumulation are stated in.  Returns -1 unless N and K are
 * multiples of 128, -2 if a NaN code is met. */
int q8o_fp8_block_mm(const uint8_t *a, const uint8_t *b, const float *s_x,
                     const float *s_w, int64_t M, int64_t N, int64_t K,
                     double *y, double *mag)
{
    if (N % 128 != 0 || K % 128 != 0)
        return -1;
    const int64_t G = K / 128;
    for (int64_t i = 0; i < M * K; ++i)
        if (isnan(q8o_e4m3_value(a[i])))
            return -2;
    for (int64_t i = 0; i < N * K; ++i)
        if (isnan(q8o_e4m3_value(b[i])))
            return -2;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0, am = 0.0;
            for (int64_t g = 0; g < G; ++g) {
                double p = 0.0, pa = 0.0;
                for (int64_t k = g * 128; k < g * 128 + 128; ++k) {
                    const double t = q8o_e4m3_value(a[m * K + k]) * q8o_e4m3_value(b[n * K + k]);
                    p += t;
                    pa += fabs(t);
                }
                const double sc = (double)s_x[m * G + g] * (double)s_w[(n / 128) * G + g];
                acc += sc * p;
                am += fabs(sc) * pa;
            }
            y[m * N + n] = acc;
            if (mag)
                mag[m * N + n] = am;
        }
    }
    return 0;
}
