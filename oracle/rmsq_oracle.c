/*
 * rmsq_oracle.c - plain, slow, double-precision CPU oracle.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load or call this library. The HIP
 * product library never includes, links or calls it, and the two share no
 * code. Build: gcc -O2 -ffp-contract=off -fopenmp -shared -fPIC (no
 * fast-math); the arithmetic below relies on IEEE double and on the default
 * round-to-nearest-even mode.
 *
 * What it computes follows four pull-request pages, cited by title:
 *   [FRQ]  "fused rmsnorm quant fp8 work"
 *   [ARQ]  "[AMD] Add fused all-reduce RMSNorm per-group quant for Qwen3.5 FP8"
 *   [ATF]  "[Feat] Support input_rmsnorm_quant & qknorm_quant fused for Atom
 *           dpsk v2 model"
 *   [ATT]  "[Triton] DS FP4/FP8 Triton fusion and GEMM optimization"
 * The pages name the steps but print no formulas; every place where this file
 * picks a reading is marked READING and is listed with its reason in the
 * design notes of the repository.
 *
 * Parity pins: every function here is checked by tests that do not call it
 * for their expected values (brute-force nearest-code search, torch's own
 * casts, a 60-digit decimal re-derivation, hand-worked rows, closed forms and
 * invariants). No function is "parity unpinned".
 */
#include "rmsq_oracle.h"

#include <fenv.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* Minifloat rounding                                                        */
/* ------------------------------------------------------------------------ */

/*
 * Round a finite a >= 0 to the nearest point of a binary floating-point grid
 * with `mbits` stored mantissa bits and smallest normal exponent `emin`
 * (gradual underflow below it), ties to even. Returns the format's magnitude
 * code, exponent field above mbits mantissa bits; a value that rounds past the
 * largest finite code returns a code past it (callers saturate or overflow).
 *
 * With 2^E <= a < 2^(E+1) (E raised to emin in the subnormal range) the grid
 * spacing is 2^(E-mbits), so k = a / 2^(E-mbits) rounded to an integer is the
 * number of spacings. The scaling by a power of two is exact; nearbyint rounds
 * half to even in the default mode. For a normal result k lies in
 * [2^mbits, 2^(mbits+1)] and the code is (E - emin + 1) << mbits | (k - 2^mbits),
 * which equals (E - emin) * 2^mbits + k; k = 2^(mbits+1) carries into the next
 * exponent. In the subnormal range E = emin and the code is k.
 */
static uint32_t minifloat_code(double a, int emin, int mbits)
{
    if (a == 0.0)
        return 0;
    int e2;
    (void)frexp(a, &e2);            /* a = f * 2^e2 with f in [0.5, 1) */
    int E = e2 - 1;
    if (E < emin)
        E = emin;
    double k = nearbyint(ldexp(a, mbits - E));
    return (uint32_t)(E - emin) * (1u << mbits) + (uint32_t)k;
}

/* Value of a magnitude code on the same grid. */
static double minifloat_value(uint32_t code, int emin, int mbits)
{
    uint32_t ef = code >> mbits;
    uint32_t m = code & ((1u << mbits) - 1u);
    if (ef == 0)
        return ldexp((double)m, emin - mbits);
    return ldexp((double)((1u << mbits) | m), (int)ef - 1 + emin - mbits);
}

/* bf16: 8 exponent bits (bias 127), 7 stored mantissa bits. */
uint16_t oracle_bf16_from_double(double v)
{
    if (isnan(v))
        return 0x7FC0;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isinf(a))
        return sign | 0x7F80;
    uint32_t c = minifloat_code(a, -126, 7);
    if (c >= 0x7F80)                /* rounded past the largest finite value */
        c = 0x7F80;
    return (uint16_t)(sign | c);
}

double oracle_bf16_to_double(uint16_t b)
{
    uint32_t mag = b & 0x7FFFu;
    double s = (b & 0x8000u) ? -1.0 : 1.0;
    if ((mag >> 7) == 0xFF)
        return (mag & 0x7F) ? NAN : s * INFINITY;
    return s * minifloat_value(mag, -126, 7);
}

/*
 * FP8 e4m3fn (OCP 8-bit floating point, "fn" variant): 4 exponent bits with
 * bias 7, 3 mantissa bits, no infinities, 0x7F / 0xFF are NaN, largest finite
 * magnitude 448 (code 0x7E). [FRQ, Motivation] names FP8 group quantization;
 * READING: the e4m3fn variant with maximum 448 and saturating conversion.
 */
uint8_t oracle_e4m3fn_encode(double v)
{
    if (isnan(v))
        return 0x7F;
    uint8_t sign = signbit(v) ? 0x80 : 0;
    double a = fabs(v);
    uint32_t c = isinf(a) ? 0x7Eu : minifloat_code(a, -6, 3);
    if (c > 0x7E)
        c = 0x7E;
    return (uint8_t)(sign | c);
}

double oracle_e4m3fn_decode(uint8_t c)
{
    uint32_t mag = c & 0x7Fu;
    if (mag == 0x7F)
        return NAN;
    double v = minifloat_value(mag, -6, 3);
    return (c & 0x80) ? -v : v;
}

/*
 * FP4 e2m1 (OCP MX element type): 2 exponent bits with bias 1, 1 mantissa
 * bit; magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}; no NaN or infinity, so the
 * conversion saturates at 6. [ATF, Technical Details] routes the norm through
 * an MXFP4 quantization; READING: round to nearest even, saturate, keep sign.
 */
uint8_t oracle_e2m1_encode(double v)
{
    uint8_t sign = signbit(v) ? 0x8 : 0;
    double a = fabs(v);
    uint32_t c = (isinf(a) || isnan(a)) ? 0x7u : minifloat_code(a, 0, 1);
    if (c > 0x7)
        c = 0x7;
    return (uint8_t)(sign | c);
}

double oracle_e2m1_decode(uint8_t c)
{
    double v = minifloat_value(c & 0x7u, 0, 1);
    return (c & 0x8) ? -v : v;
}

/*
 * Shared MX scale exponent for a block whose largest magnitude is amax > 0:
 * floor(log2(amax)) minus the largest exponent of the element type (2 for
 * e2m1), clamped to the e8m0 range [-127, 127]. READING: the OCP Microscaling
 * rule; the pages name MXFP4 [ATF, Technical Details] and e8m0 scale bytes
 * [ATT, review thread] without the rule itself.
 */
int oracle_mx_scale_exponent(double amax)
{
    int e2;
    (void)frexp(amax, &e2);         /* floor(log2(amax)) = e2 - 1 */
    int e = (e2 - 1) - 2;
    if (e < -127)
        e = -127;
    if (e > 127)
        e = 127;
    return e;
}

void oracle_bf16_from_double_n(const double* v, uint16_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_bf16_from_double(v[i]);
}

void oracle_e4m3fn_encode_n(const double* v, uint8_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_e4m3fn_encode(v[i]);
}

void oracle_e2m1_encode_n(const double* v, uint8_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_e2m1_encode(v[i]);
}

/* ------------------------------------------------------------------------ */
/* Stage 1: residual add and RMSNorm                                         */
/* ------------------------------------------------------------------------ */

/*
 * One row.
 *  1. h = bf16(x + r) when a residual is given, else h = x. The sum of two
 *     bf16 values is formed in double and rounded to bf16; that equals the
 *     correctly rounded bf16 of the exact sum (the double sum is exact unless
 *     the exponents differ by more than 45, and then both round to the larger
 *     operand). [ARQ, kernel
 *     count table] lists the add + RMSNorm kernel that this step replaces and
 *     [ARQ, Modifications] returns the residual. READING: the residual handed
 *     back is the bf16 sum, and the norm reads that same bf16 sum.
 *  2. RMSNorm [FRQ, Motivation]. READING: the textbook form,
 *     inv = 1 / sqrt(mean(h^2) + eps) with the mean over the N columns, eps
 *     inside the root (eps is the float the caller passes, widened exactly),
 *     gamma multiplicative. A zero denominator (zero row with eps = 0) gives
 *     inv = 0, so the row normalizes to zeros.
 *  3. y = h * gamma * inv in double, rounded once to bf16: the normalized
 *     activation that [ARQ, Modifications] hands to consumers that need bf16.
 */
static void add_rmsnorm_row(const uint16_t* x, const uint16_t* r,
                            const uint16_t* gamma, float eps, int64_t N,
                            uint16_t* h_out, uint16_t* yb_out, double* hbuf)
{
    for (int64_t j = 0; j < N; ++j) {
        double xv = oracle_bf16_to_double(x[j]);
        if (r) {
            double sum = xv + oracle_bf16_to_double(r[j]);
            uint16_t hb = oracle_bf16_from_double(sum);
            if (h_out)
                h_out[j] = hb;
            hbuf[j] = oracle_bf16_to_double(hb);
        } else {
            hbuf[j] = xv;
        }
    }

    double ss = 0.0;
    for (int64_t j = 0; j < N; ++j)
        ss += hbuf[j] * hbuf[j];
    double denom = ss / (double)N + (double)eps;
    double inv = denom > 0.0 ? 1.0 / sqrt(denom) : 0.0;

    for (int64_t j = 0; j < N; ++j) {
        double y = hbuf[j] * oracle_bf16_to_double(gamma[j]) * inv;
        yb_out[j] = oracle_bf16_from_double(y);
    }
}

void oracle_add_rmsnorm(const uint16_t* x, int64_t ldx,
                        const uint16_t* residual, int64_t ldr,
                        const uint16_t* gamma, float eps, int64_t M, int64_t N,
                        uint16_t* h_out, int64_t ldh,
                        uint16_t* yb_out, int64_t ldy)
{
#pragma omp parallel
    {
        double* hbuf = (double*)malloc((size_t)N * sizeof(double));
#pragma omp for schedule(static)
        for (int64_t m = 0; m < M; ++m)
            add_rmsnorm_row(x + m * ldx, residual ? residual + m * ldr : NULL,
                            gamma, eps, N, h_out ? h_out + m * ldh : NULL,
                            yb_out + m * ldy, hbuf);
        free(hbuf);
    }
}

/* ------------------------------------------------------------------------ */
/* Stage 2: per-group dynamic quantization                                   */
/* ------------------------------------------------------------------------ */

/* Byte offset of e8m0 scale (m, g) in the 32-row tiled layout: tiles of 32
 * rows, group-major inside a tile, so the 32 rows' scales for one group are
 * contiguous. READING: [ATT, review thread] views the byte scales as tiles of
 * the MXFP4 block size in rows when there are at least that many rows; the
 * order inside a tile is not on the pages. */
static int64_t tiled32_offset(int64_t m, int64_t g, int64_t groups_per_row)
{
    return (m / 32) * (32 * groups_per_row) + g * 32 + (m % 32);
}

/* Scale offset (in scale elements) of (row m, group g) for M rows and G groups
 * per row: layout 0 row-major [M][G], 1 the 32-row tiles above, 2 column-major
 * [G][M] (group-major: one group's scales for all rows adjacent, the order a
 * GEMM walking K in 128-column blocks reads them). READING: [ARQ, Motivation]
 * hands (fp8, scale) to a block-scaled FP8 GEMM without fixing how it reads
 * the scales; the column-major option is this library's, not the pages'. */
static int64_t scale_offset(int64_t m, int64_t g, int64_t M, int64_t G, int32_t layout)
{
    if (layout == 1)
        return tiled32_offset(m, g, G);
    if (layout == 2)
        return g * M + m;
    return m * G + g;
}

/*
 * One row of bf16 values, groups of `group` consecutive columns.
 * FP8 [FRQ, Motivation] (group 128) / [ARQ, Fallback order] (1x128 groups):
 *   amax = max |yb| over the group; s = amax / 448 rounded once to fp32
 *   (READING: the scale is computed at run time from the group, as the
 *   dynamic per-group quant kernel of [ARQ, kernel count table] implies);
 *   an all-zero group takes s = 1 (READING: a finite, invertible scale).
 *   q = e4m3fn(yb / s) with the quotient in double.
 * MXFP4 [ATF, Technical Details] (group 32): e = mx_scale_exponent(amax), the
 *   scale byte is e + 127; q = e2m1(yb * 2^-e), exact scaling. An all-zero
 *   group takes e = 0 (byte 127). Two codes per byte, element 2k in the low
 *   nibble (READING).
 */
static void group_quant_row(const uint16_t* yb, int64_t m, int64_t M, int64_t N,
                            int32_t group, int32_t fmt, int32_t layout,
                            uint8_t* q_row, void* scale)
{
    int64_t groups = N / group;
    for (int64_t g = 0; g < groups; ++g) {
        const uint16_t* v = yb + g * group;
        double amax = 0.0;
        for (int32_t i = 0; i < group; ++i) {
            double a = fabs(oracle_bf16_to_double(v[i]));
            if (a > amax)
                amax = a;
        }
        if (fmt == 0) {
            float s = amax == 0.0 ? 1.0f : (float)(amax / 448.0);
            ((float*)scale)[scale_offset(m, g, M, groups, layout)] = s;
            for (int32_t i = 0; i < group; ++i)
                q_row[g * group + i] =
                    oracle_e4m3fn_encode(oracle_bf16_to_double(v[i]) / (double)s);
        } else {
            int e = amax == 0.0 ? 0 : oracle_mx_scale_exponent(amax);
            uint8_t byte = (uint8_t)(e + 127);
            ((uint8_t*)scale)[scale_offset(m, g, M, groups, layout)] = byte;
            for (int32_t i = 0; i < group; i += 2) {
                uint8_t lo = oracle_e2m1_encode(ldexp(oracle_bf16_to_double(v[i]), -e));
                uint8_t hi = oracle_e2m1_encode(ldexp(oracle_bf16_to_double(v[i + 1]), -e));
                q_row[(g * group + i) / 2] = (uint8_t)(lo | (hi << 4));
            }
        }
    }
}

static int shape_ok(int64_t N, int32_t group, int32_t fmt, int32_t layout)
{
    if (fmt == 0)
        return group == 128 && N % 128 == 0 && (layout == 0 || layout == 2);
    if (fmt == 1)
        return group == 32 && N % 32 == 0 && (layout == 0 || layout == 1 || layout == 2);
    return 0;
}

void oracle_group_quant(const uint16_t* yb, int64_t ldy, int64_t M, int64_t N,
                        int32_t group, int32_t fmt, int32_t scale_layout,
                        uint8_t* q, void* scale)
{
    if (!shape_ok(N, group, fmt, scale_layout))
        return;
    int64_t qpitch = fmt == 0 ? N : N / 2;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        group_quant_row(yb + m * ldy, m, M, N, group, fmt, scale_layout,
                        q + m * qpitch, scale);
}

int oracle_rmsnorm_quant_group(const uint16_t* x, int64_t ldx,
                               const uint16_t* residual_in, int64_t ldr,
                               const uint16_t* gamma, float eps,
                               int64_t M, int64_t N, int32_t group, int32_t fmt,
                               int32_t scale_layout,
                               uint8_t* out_q, void* out_scale,
                               uint16_t* residual_out,
                               uint16_t* out_bf16, int64_t ldb)
{
    if (!shape_ok(N, group, fmt, scale_layout) || M < 0 || N <= 0)
        return -1;
    if ((residual_in == NULL) != (residual_out == NULL))
        return -1;
    if (fegetround() != FE_TONEAREST)
        return -1;
    int64_t qpitch = fmt == 0 ? N : N / 2;
#pragma omp parallel
    {
        double* hbuf = (double*)malloc((size_t)N * sizeof(double));
        uint16_t* ybuf = (uint16_t*)malloc((size_t)N * sizeof(uint16_t));
#pragma omp for schedule(static)
        for (int64_t m = 0; m < M; ++m) {
            add_rmsnorm_row(x + m * ldx, residual_in ? residual_in + m * ldr : NULL,
                            gamma, eps, N,
                            residual_out ? residual_out + m * ldr : NULL, ybuf, hbuf);
            if (out_bf16)
                memcpy(out_bf16 + m * ldb, ybuf, (size_t)N * sizeof(uint16_t));
            group_quant_row(ybuf, m, M, N, group, fmt, scale_layout,
                            out_q + m * qpitch, out_scale);
        }
        free(ybuf);
        free(hbuf);
    }
    return 0;
}

/*
 * A16WFP4 "prequant" GEMM ([ATT], the AITER pull requests it lists: a GEMM of
 * bf16 activations with FP4 weights that quantizes the activations inside
 * the GEMM; [ATT, run notes]: the path used at concurrency 4). The pages name
 * the kernel only; READING: the activation rows are quantized exactly as the
 * MXFP4 group quantization above (1x32 groups along K, e8m0 scale from the
 * group amax, e2m1 codes), the weights come as e2m1 codes [N, K/2] (element
 * 2k of a row in the low nibble) with e8m0 scales [N, K/32], and
 *   C[m][n] = sum_k (qa[m][k] * 2^(ea[m][k/32] - 127)) * (qw[n][k] * 2^(ew[n][k/32] - 127)),
 * accumulated here in double in k order.
 */
static double e8m0_value(uint8_t byte)
{
    return ldexp(1.0, (int)byte - 127);
}

int oracle_gemm_a16wfp4_prequant(const uint16_t* a, int64_t lda,
                                 const uint8_t* w, const uint8_t* w_scale,
                                 int64_t M, int64_t N, int64_t K,
                                 double* out, int64_t ldc)
{
    if (M < 0 || N < 0 || K <= 0 || K % 32 != 0 || lda < K || ldc < N)
        return -1;
    if (fegetround() != FE_TONEAREST)
        return -1;
#pragma omp parallel
    {
        uint8_t* qa = (uint8_t*)malloc((size_t)K / 2);
        uint8_t* ea = (uint8_t*)malloc((size_t)K / 32);
        double* da = (double*)malloc((size_t)K * sizeof(double));
#pragma omp for schedule(static)
        for (int64_t m = 0; m < M; ++m) {
            /* the activation row's MXFP4 quantization, then its values */
            group_quant_row(a + m * lda, 0, 1, K, 32, 1, 0, qa, ea);
            for (int64_t k = 0; k < K; ++k) {
                uint8_t code = (uint8_t)((qa[k / 2] >> (4 * (k % 2))) & 0xF);
                da[k] = oracle_e2m1_decode(code) * e8m0_value(ea[k / 32]);
            }
            for (int64_t n = 0; n < N; ++n) {
                const uint8_t* wr = w + n * (K / 2);
                const uint8_t* sr = w_scale + n * (K / 32);
                double acc = 0.0;
                for (int64_t k = 0; k < K; ++k) {
                    uint8_t code = (uint8_t)((wr[k / 2] >> (4 * (k % 2))) & 0xF);
                    acc += da[k] * (oracle_e2m1_decode(code) * e8m0_value(sr[k / 32]));
                }
                out[m * ldc + n] = acc;
            }
        }
        free(da);
        free(ea);
        free(qa);
    }
    return 0;
}

/*
 * A16W8 prequant GEMM, the FP8 counterpart that [ATT] lists for its DS FP8
 * runs (an a16w8 GEMM). READING: the activation rows are quantized exactly
 * as the FP8 group quantization above (1x128 groups along K, fp32 scale
 * amax/448, e4m3fn codes of the quotient); the weights come as e4m3fn codes
 * [N, K] with fp32 scales per 128x128 block [ceil(N/128), K/128] (the block
 * layout of the DeepSeek FP8 checkpoints those runs serve), and
 *   C[m][n] = sum_k (qa[m][k] * sa[m][k/128]) * (qw[n][k] * sw[n/128][k/128]),
 * accumulated here in double in k order.
 */
int oracle_gemm_a16w8_prequant(const uint16_t* a, int64_t lda,
                               const uint8_t* w, const float* w_scale,
                               int64_t M, int64_t N, int64_t K,
                               double* out, int64_t ldc)
{
    if (M < 0 || N < 0 || K <= 0 || K % 128 != 0 || lda < K || ldc < N)
        return -1;
    if (fegetround() != FE_TONEAREST)
        return -1;
    const int64_t kb = K / 128;
#pragma omp parallel
    {
        uint8_t* qa = (uint8_t*)malloc((size_t)K);
        float* sa = (float*)malloc((size_t)kb * sizeof(float));
        double* da = (double*)malloc((size_t)K * sizeof(double));
#pragma omp for schedule(static)
        for (int64_t m = 0; m < M; ++m) {
            /* the activation row's FP8 quantization, then its values */
            group_quant_row(a + m * lda, 0, 1, K, 128, 0, 0, qa, sa);
            for (int64_t k = 0; k < K; ++k)
                da[k] = oracle_e4m3fn_decode(qa[k]) * (double)sa[k / 128];
            for (int64_t n = 0; n < N; ++n) {
                const uint8_t* wr = w + n * K;
                const float* sr = w_scale + (n / 128) * kb;
                double acc = 0.0;
                for (int64_t k = 0; k < K; ++k)
                    acc += da[k] * (oracle_e4m3fn_decode(wr[k]) * (double)sr[k / 128]);
                out[m * ldc + n] = acc;
            }
        }
        free(da);
        free(sa);
        free(qa);
    }
    return 0;
}

/*
 * The GEMMs that consume activations already quantized by the fused kernel:
 * [ATT, run notes] pairs the fused RMSNorm + quant with a separate GEMM above
 * concurrency 4, fed by gemm_afp4wfp4_preshuffle (MXFP4) and, for the FP8
 * runs, the block-scaled a8w8 GEMMs it lists; [ATF, Technical Details]
 * requires the quantized activations' scales to come in the layout the GEMM
 * reads. READING: the activations are exactly what the group quantization
 * above writes - codes [M, K/2] (MXFP4, element 2k in the low nibble) or
 * [M, K] (FP8), rows dense - with their scales in any of its layouts
 * (scale_offset), and the weights are as in the prequant GEMMs:
 *   MXFP4: C[m][n] = sum_k (qa[m][k] 2^(ea[m][k/32] - 127)) (qw[n][k] 2^(ew[n][k/32] - 127))
 *   FP8:   C[m][n] = sum_k (qa[m][k] sa[m][k/128]) (qw[n][k] sw[n/128][k/128])
 * accumulated here in double in k order.
 */
int oracle_gemm_afp4wfp4(const uint8_t* a_q, const uint8_t* a_scale, int32_t a_layout,
                         const uint8_t* w, const uint8_t* w_scale,
                         int64_t M, int64_t N, int64_t K, double* out, int64_t ldc)
{
    if (M < 0 || N < 0 || K <= 0 || K % 32 != 0 || ldc < N || a_layout < 0 || a_layout > 2)
        return -1;
    const int64_t G = K / 32;
#pragma omp parallel
    {
        double* av = (double*)malloc((size_t)K * sizeof(double));
#pragma omp for schedule(static)
        for (int64_t m = 0; m < M; ++m) {
            /* the given activation row's values: code times its group's scale */
            const uint8_t* arow = a_q + m * (K / 2);
            for (int64_t k = 0; k < K; ++k) {
                uint8_t c = (uint8_t)((arow[k / 2] >> (4 * (k % 2))) & 0xF);
                av[k] = oracle_e2m1_decode(c) * e8m0_value(a_scale[scale_offset(m, k / 32, M, G, a_layout)]);
            }
            for (int64_t n = 0; n < N; ++n) {
                const uint8_t* wrow = w + n * (K / 2);
                const uint8_t* erow = w_scale + n * G;
                double sum = 0.0;
                for (int64_t k = 0; k < K; ++k) {
                    uint8_t c = (uint8_t)((wrow[k / 2] >> (4 * (k % 2))) & 0xF);
                    sum += av[k] * (oracle_e2m1_decode(c) * e8m0_value(erow[k / 32]));
                }
                out[m * ldc + n] = sum;
            }
        }
        free(av);
    }
    return 0;
}

int oracle_gemm_a8w8_blockscale(const uint8_t* a_q, const float* a_scale, int32_t a_layout,
                                const uint8_t* w, const float* w_scale,
                                int64_t M, int64_t N, int64_t K, double* out, int64_t ldc)
{
    if (M < 0 || N < 0 || K <= 0 || K % 128 != 0 || ldc < N || (a_layout != 0 && a_layout != 2))
        return -1;
    const int64_t blocks = K / 128;
#pragma omp parallel
    {
        double* av = (double*)malloc((size_t)K * sizeof(double));
#pragma omp for schedule(static)
        for (int64_t m = 0; m < M; ++m) {
            const uint8_t* arow = a_q + m * K;
            for (int64_t k = 0; k < K; ++k)
                av[k] = oracle_e4m3fn_decode(arow[k]) *
                        (double)a_scale[scale_offset(m, k / 128, M, blocks, a_layout)];
            for (int64_t n = 0; n < N; ++n) {
                const uint8_t* wrow = w + n * K;
                const float* brow = w_scale + (n / 128) * blocks;   /* the weight row's 128-row block */
                double sum = 0.0;
                for (int64_t k = 0; k < K; ++k)
                    sum += av[k] * (oracle_e4m3fn_decode(wrow[k]) * (double)brow[k / 128]);
                out[m * ldc + n] = sum;
            }
        }
        free(av);
    }
    return 0;
}

/* Threads the oracle's parallel loops use from now on (n >= 1): the
 * process environment may fix OMP_NUM_THREADS for every child process, so
 * the thread count is set through the runtime instead. */
void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
