/*
 * rmsq_oracle.h - plain double-precision CPU oracle for residual-add +
 * RMSNorm + per-group dynamic quantization (FP8 e4m3fn / MXFP4).
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load or call this library. The HIP
 * product library never includes, links or calls it, and the two share no
 * code.
 *
 * All tensors are host arrays. bf16 values travel as their uint16 bit
 * patterns. Row strides are in elements.
 */
#ifndef RMSQ_ORACLE_H
#define RMSQ_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Format codecs (exact, round-to-nearest-even with ties to even mantissa). */
uint16_t oracle_bf16_from_double(double v);
double   oracle_bf16_to_double(uint16_t b);
uint8_t  oracle_e4m3fn_encode(double v);   /* saturates to +-448, keeps the sign */
double   oracle_e4m3fn_decode(uint8_t c);   /* 0x7F / 0xFF decode to NaN       */
uint8_t  oracle_e2m1_encode(double v);     /* 4-bit code, saturates to +-6     */
double   oracle_e2m1_decode(uint8_t c);
int      oracle_mx_scale_exponent(double amax); /* amax > 0; clamped to [-127, 127] */

/* Vector forms of the codecs, for the tests. */
void oracle_bf16_from_double_n(const double* v, uint16_t* out, int64_t n);
void oracle_e4m3fn_encode_n(const double* v, uint8_t* out, int64_t n);
void oracle_e2m1_encode_n(const double* v, uint8_t* out, int64_t n);

/* Stage 1: h = x (+ residual), RMSNorm, bf16 normalized row. residual and
 * h_out may be NULL (no residual: h = x). yb_out receives bf16(h*gamma*inv). */
void oracle_add_rmsnorm(const uint16_t* x, int64_t ldx,
                        const uint16_t* residual, int64_t ldr,
                        const uint16_t* gamma, float eps, int64_t M, int64_t N,
                        uint16_t* h_out, int64_t ldh,
                        uint16_t* yb_out, int64_t ldy);

/* Stage 2: per-group dynamic quantization of bf16 rows.
 * fmt 0 (FP8 e4m3fn, group 128): q [M, N] bytes, scale fp32 [M, N/group].
 * fmt 1 (MXFP4 e2m1, group 32): q [M, N/2] bytes (element 2k in the low
 * nibble), scale e8m0 bytes. Scale layouts: 0 = row-major [M, N/group];
 * 1 (MXFP4 only) = 32-row tiles: byte (m/32)*(32*N/32) + g*32 + m%32;
 * 2 = column-major [N/group, M]. */
void oracle_group_quant(const uint16_t* yb, int64_t ldy, int64_t M, int64_t N,
                        int32_t group, int32_t fmt, int32_t scale_layout,
                        uint8_t* q, void* scale);

/* The fused result: stage 1 then stage 2 on the bf16 normalized rows.
 * out_bf16 may be NULL. Returns 0, or -1 for arguments the oracle does not
 * define (the oracle does not validate beyond that). */
int oracle_rmsnorm_quant_group(const uint16_t* x, int64_t ldx,
                               const uint16_t* residual_in, int64_t ldr,
                               const uint16_t* gamma, float eps,
                               int64_t M, int64_t N, int32_t group, int32_t fmt,
                               int32_t scale_layout,
                               uint8_t* out_q, void* out_scale,
                               uint16_t* residual_out,
                               uint16_t* out_bf16, int64_t ldb);

/* A16WFP4 prequant GEMM: a [M, K] bf16 (row stride lda) quantized to MXFP4
 * per 1x32 group along K as oracle_group_quant does, times the MXFP4 weights
 * w [N, K/2] codes (element 2k in the low nibble) with e8m0 scales
 * w_scale [N, K/32]: out[m*ldc + n] = sum over k of the dequantized products,
 * in double. Returns 0, or -1 for arguments it does not define (K a positive
 * multiple of 32). */
int oracle_gemm_a16wfp4_prequant(const uint16_t* a, int64_t lda,
                                 const uint8_t* w, const uint8_t* w_scale,
                                 int64_t M, int64_t N, int64_t K,
                                 double* out, int64_t ldc);

/* A16W8 prequant GEMM: a [M, K] bf16 (row stride lda) quantized to FP8
 * e4m3fn per 1x128 group along K as oracle_group_quant does, times the FP8
 * weights w [N, K] e4m3fn codes with fp32 scales per 128x128 block
 * w_scale [ceil(N/128), K/128]: out[m*ldc + n] = sum over k of the
 * dequantized products, in double. Returns 0, or -1 for arguments it does not
 * define (K a positive multiple of 128). */
int oracle_gemm_a16w8_prequant(const uint16_t* a, int64_t lda,
                               const uint8_t* w, const float* w_scale,
                               int64_t M, int64_t N, int64_t K,
                               double* out, int64_t ldc);

/* GEMMs of activations already quantized by the group quantization above
 * (codes with dense rows, scales in its layout a_layout) and the prequant
 * GEMMs' weights, the dequantized products summed in double:
 * MXFP4: a_q [M, K/2], a_scale e8m0 (layout 0, 1 or 2), w [N, K/2],
 *        w_scale e8m0 [N, K/32];
 * FP8:   a_q [M, K] e4m3fn, a_scale fp32 (layout 0 or 2), w [N, K] e4m3fn,
 *        w_scale fp32 [ceil(N/128), K/128].
 * Return 0, or -1 for arguments they do not define. */
int oracle_gemm_afp4wfp4(const uint8_t* a_q, const uint8_t* a_scale, int32_t a_layout,
                         const uint8_t* w, const uint8_t* w_scale,
                         int64_t M, int64_t N, int64_t K, double* out, int64_t ldc);
int oracle_gemm_a8w8_blockscale(const uint8_t* a_q, const float* a_scale, int32_t a_layout,
                                const uint8_t* w, const float* w_scale,
                                int64_t M, int64_t N, int64_t K, double* out, int64_t ldc);

int oracle_num_threads(void);
void oracle_set_num_threads(int n);

#ifdef __cplusplus
}
#endif
#endif
