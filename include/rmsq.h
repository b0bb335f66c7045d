/*
 * rmsq.h - C ABI of the fused residual-add + RMSNorm + per-group dynamic
 * quantization library for AMD Instinct MI355X (gfx950).
 *
 * The operation follows four pull-request pages, cited by title:
 *   [FRQ]  "fused rmsnorm quant fp8 work"
 *   [ARQ]  "[AMD] Add fused all-reduce RMSNorm per-group quant for Qwen3.5 FP8"
 *   [ATF]  "[Feat] Support input_rmsnorm_quant & qknorm_quant fused for Atom
 *           dpsk v2 model"
 *   [ATT]  "[Triton] DS FP4/FP8 Triton fusion and GEMM optimization"
 *
 * Per token row (all arithmetic on the device, one kernel launch per call):
 *   h  = bf16(x + residual_in)            (h = x without a residual)
 *   y  = h * gamma / sqrt(mean(h^2) + eps)
 *   yb = bf16(y)                          (optional side-output)
 *   per group of G columns: scale from max |yb|, codes = quantize(yb / scale)
 *     FP8:   G = 128, scale = amax / 448 in fp32, codes are OCP e4m3fn bytes
 *     MXFP4: G = 32, scale = 2^(floor(log2 amax) - 2) stored as an e8m0 byte,
 *            codes are e2m1 nibbles, two per byte, element 2k in the low nibble
 * Every rounding is to nearest, ties to even; all-zero groups get scale 1.0
 * (FP8) or byte 127 (MXFP4). Results are bit-for-bit those of the double
 * precision definition above.
 *
 * Conventions shared by every entry point:
 *  - Data pointers are DEVICE pointers owned by the caller. The library
 *    allocates no device memory and never synchronizes the host: work is
 *    enqueued on `stream` (a hipStream_t; NULL is the default stream) and
 *    the call returns. The only state it keeps between calls is a cached
 *    per-device answer to "is this a gfx950"; a call's launch plan depends on
 *    its own arguments only (see rmsq_launch_hint).
 *  - bf16 tensors are row-major with a row stride (ld, in elements) that is a
 *    multiple of 8 and >= N; bf16 pointers are 16-byte aligned. Codes and
 *    scales are dense: codes [M, N] bytes (FP8) or [M, N/2] (MXFP4); scales
 *    fp32 (FP8, 4-byte aligned) or e8m0 bytes (MXFP4), in one of the layouts
 *    below (row-major [M, N/group] by default). FP8 code pointers are 8-byte aligned, MXFP4 ones 4-byte.
 *  - Outputs must not overlap each other or the inputs, except that
 *    residual_out may be the very same buffer as residual_in (in place).
 *  - Validation happens before any HIP call; a status other than RMSQ_OK
 *    means nothing was enqueued. M == 0 is a no-op returning RMSQ_OK.
 *  - Size limit: the hardware dispatch counts a launch's work-items in 32
 *    bits, and a row takes 64 to 1024 of them (64 per wave of its launch
 *    shape; the quantization alone, 128 per row), so a call whose rows would
 *    need more than 2^32 work-items in one launch (e.g. more than 67M rows of
 *    512 elements, 4.1M rows of any width always fit) returns
 *    RMSQ_ERR_UNSUPPORTED; split such a batch into several calls.
 *  - Non-finite inputs are outside the contract (no fault, undefined values).
 *  - Thread safety: calls are re-entrant and may come from any number of
 *    host threads at once; calls on different streams may run concurrently.
 *    The message of rmsq_last_error is kept per thread.
 */
#ifndef RMSQ_H
#define RMSQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The library is built with hidden visibility; these declarations are its
 * exported interface. */
#pragma GCC visibility push(default)

typedef int32_t rmsq_status;
#define RMSQ_OK 0
#define RMSQ_ERR_INVALID_ARG 1 /* bad pointer, alignment, stride, shape or overlap */
#define RMSQ_ERR_UNSUPPORTED 2 /* not a gfx950 device, or format/group/N outside what is built */
#define RMSQ_ERR_HIP 3         /* the HIP runtime reported an error at launch */

#define RMSQ_FMT_FP8_E4M3FN 0  /* group 128, fp32 scales            */
#define RMSQ_FMT_MXFP4_E2M1 1  /* group 32, e8m0 scales, packed e2m1 */

/* Scale layouts, G = N/group scales per row:
 *  RMSQ_SCALE_ROW_MAJOR  [M, G] (both formats).
 *  RMSQ_SCALE_TILED32    MXFP4 only: tiles of 32 rows, byte offset of (m, g)
 *                        (m/32)*(32*G) + g*32 + m%32, so the 32 rows' scales of
 *                        one group are adjacent; the buffer holds
 *                        ceil(M/32)*32*G bytes and the bytes of the padding rows
 *                        of the last tile are left untouched. [ATT, review
 *                        thread] views the byte scales in tiles of the MXFP4
 *                        block size in rows when the row count reaches it.
 *  RMSQ_SCALE_COL_MAJOR  [G, M] (both formats): one group column's scales for
 *                        all rows adjacent, the order a GEMM walking K in
 *                        group-sized blocks reads them.
 * [ATF, Technical Details] selects the activation scale layout that the
 * consuming GEMM expects; the consumers' own permutations are not defined on
 * the pages, so these three are this library's. */
#define RMSQ_SCALE_ROW_MAJOR 0
#define RMSQ_SCALE_TILED32 1
#define RMSQ_SCALE_COL_MAJOR 2

#define RMSQ_MAX_PROBLEMS 4
#define RMSQ_N_MAX 32768
#define RMSQ_GEMM_N_MAX (1 << 20)
#define RMSQ_GEMM_K_MAX (1 << 20)
#define RMSQ_GEMM_LDA_MAX (1 << 25)   /* row stride of the prequant GEMMs' bf16 activations, elements */

/* Weight layouts of gemm_a16wfp4_prequant (this library's; the page names a
 * preshuffled-weight GEMM without giving its layout).
 * ROW_MAJOR: codes [N, K/2] (element 2j of a row in the low nibble of byte
 *   j), scales [N, K/32].
 * PRESHUFFLED: the operand order of the kernel's matrix-core steps. For
 *   column tile t (rows 16t .. 16t+15), 128-wide K step s and lane l in
 *   0..63, the 16 code bytes of row 16t + l%16, 32-group 4s + l/16 sit at
 *   byte ((t * K/128 + s) * 64 + l) * 16, and that group's scale byte at
 *   (t * K/128 + s) * 64 + l. Same sizes as ROW_MAJOR; made by
 *   mxfp4_weight_preshuffle. */
#define RMSQ_W_ROW_MAJOR 0
#define RMSQ_W_PRESHUFFLED 1

/*
 * Fused residual add + RMSNorm + per-group dynamic quantization of M rows of
 * N bf16 values, contiguous rows (ld = N), row-major scales.
 * [FRQ, Motivation]: RMSNorm and FP8 group quantization with group size 128
 * in one kernel. [ARQ, Modifications]: results ((codes, scale), residual) or,
 * with the bf16 side-output, ((bf16, codes, scale), residual).
 * [ARQ, kernel count table]: replaces the add + RMSNorm kernel and the
 * dynamic per-group quant kernel (and the extra quant of the bf16 path).
 * [ATF, Technical Details]: the MXFP4 variant.
 *
 *  x            [M, N] bf16, read only.
 *  residual_in  [M, N] bf16 or NULL (no residual add; then residual_out must
 *               be NULL too, else RMSQ_ERR_INVALID_ARG).
 *  gamma        [N] bf16 RMSNorm weight.
 *  eps          finite, >= 0; added to mean(h^2) inside the square root.
 *  group, fmt   128 with RMSQ_FMT_FP8_E4M3FN, 32 with RMSQ_FMT_MXFP4_E2M1;
 *               other pairs give RMSQ_ERR_UNSUPPORTED.
 *  out_q        codes; out_scale: scales (row-major).
 *  residual_out [M, N] bf16: the bf16 sum h, or NULL.
 *  out_bf16_or_null [M, N] bf16 normalized rows, or NULL to skip them.
 *  stream       hipStream_t to enqueue on.
 * N must be a multiple of the group and at most RMSQ_N_MAX.
 */
rmsq_status rmsnorm_quant_group(const void* x, const void* residual_in, const void* gamma,
                                float eps, int64_t M, int64_t N, int32_t group, int32_t fmt,
                                void* out_q, void* out_scale, void* residual_out,
                                void* out_bf16_or_null, void* stream);

/* One independent row problem for rmsnorm_quant_group_multi. ld values are in
 * elements; 0 means N. ldr is the stride of both residual_in and residual_out. */
typedef struct rmsq_problem {
    const void* x;
    int64_t ldx;
    const void* residual_in;
    void* residual_out;
    int64_t ldr;
    const void* gamma;
    float eps;
    int64_t M;
    int64_t N;
    int32_t group;
    int32_t fmt;
    int32_t scale_layout;
    void* out_q;
    void* out_scale;
    void* out_bf16;
    int64_t ldb;
} rmsq_problem;

/*
 * 1 to RMSQ_MAX_PROBLEMS independent problems in ONE kernel launch, e.g. the
 * two latent norms of multi-head latent attention (q and kv), which
 * [FRQ, Modifications] fuses at the attention module and [ATF, Technical
 * Details] fuses as "qknorm quant". Each problem is the operation of
 * rmsnorm_quant_group with its own shapes, strides, residual, side-output
 * and scale layout; all problems use the same fmt. A set in which some
 * problems have a residual and others do not takes two launches (those
 * with a residual first), both on `stream`. The problem array is read on the
 * host during the call and may be freed when it returns.
 */
rmsq_status rmsnorm_quant_group_multi(const rmsq_problem* problems, int32_t count, void* stream);

/*
 * Optional per-call launch hint for rmsnorm_quant_group_multi_ex and
 * rmsq_plan_launch, for measurement sweeps and callers that tune their own
 * shapes. A zero field leaves that choice to the library. Results never
 * depend on the launch plan (every plan computes the same bytes); only the
 * speed does. The hint applies to the one call it is passed to: the library
 * keeps no launch state between calls.
 *  chunks_per_lane, waves_per_row  J 16-byte chunks per lane (1, 2, 3, 4, 7,
 *        8 or 14) and W waves per row (1..16; 1..4 when J >= 7), set
 *        together; J*W*64 chunks must cover the widest row of the launch.
 *  row_group  consecutive rows kept on one XCD (1..64, rounded down to a
 *        power of two; 1 = plain dispatch order). Automatic: 16 when a
 *        problem writes tiled or column-major scales, else 1.
 *  waves_per_workgroup  packed rows: waves per workgroup when a row fits one
 *        wave (1..16; 1 = no packing: one row per workgroup). Automatic: 8
 *        once a launch has at least 1024 rows, else 1. Not used when rows
 *        span several waves.
 *  lanes_per_row  packed rows of one chunk per lane (J = 1, rows of at most
 *        512 elements): lanes per row for every problem of the launch (16, 32
 *        or 64; a wave then holds 4, 2 or 1 rows, whose statistics share one
 *        instruction sequence). Automatic, per problem: the fewest that hold
 *        the row (128-wide rows 16 lanes each). Below 64 with J > 1 it is
 *        refused; ignored when rows are not packed.
 *  row_splits  workgroups sharing each row (1..8, rounded down to a power of
 *        two; each computes the row's statistics and normalizes / quantizes
 *        its own share of the groups). Automatic: the largest power of two
 *        S <= 8 with rows * S <= 256 for launches of at most 128 rows, else 1.
 *        Rows are never split when a problem's residual is updated in place,
 *        when rows are packed per workgroup, or below one group per split.
 * A field outside its range, or a J x W (packed by lanes: lanes_per_row)
 * that does not cover a row, gives RMSQ_ERR_INVALID_ARG (nothing is
 * launched).
 */
typedef struct rmsq_launch_hint {
    int32_t chunks_per_lane;
    int32_t waves_per_row;
    int32_t row_group;
    int32_t waves_per_workgroup;
    int32_t row_splits;
    int32_t lanes_per_row;
} rmsq_launch_hint;

/* rmsnorm_quant_group_multi with an optional launch hint (NULL: the
 * library's own plan, exactly as rmsnorm_quant_group_multi). Same contract,
 * errors and stream semantics. */
rmsq_status rmsnorm_quant_group_multi_ex(const rmsq_problem* problems, int32_t count, const rmsq_launch_hint* hint,
                                         void* stream);

/* One planned launch of the fused kernel. */
typedef struct rmsq_launch_info {
    int32_t problems;               /* problems in this launch                  */
    int32_t rows;                   /* rows over those problems                 */
    int32_t chunks_per_lane;        /* J                                        */
    int32_t waves_per_row;          /* W                                        */
    int32_t waves_per_workgroup;    /* R > 1: packed rows, R waves per workgroup (1: one row,
                                       or a share of one, per workgroup) */
    int32_t row_splits;             /* S workgroups per row                     */
    int32_t row_group;              /* consecutive rows kept on one XCD         */
    int32_t threads_per_workgroup;
    int64_t workgroups;
    int32_t residual;               /* 1 if this launch's problems have a residual */
    int32_t tail;                   /* how its rows end: 1 every row fills the launch shape exactly,
                                       2 rows one wave each, all whole 64-lane steps (steps past a row's
                                       end skipped by the wave), 0 otherwise (lanes past the end bounded) */
    int32_t lanes_per_row[4];       /* lanes holding one row of each of its problems: 64 x W; packed
                                       64, or 16, 32 or 64 when packed by lanes (J = 1) */
} rmsq_launch_info;

typedef struct rmsq_launch_plan {
    int32_t launches;               /* 0 (every M is 0), 1, or 2 (a set mixing problems with and
                                       without a residual: those with one first) */
    int32_t reserved;
    rmsq_launch_info launch[2];
} rmsq_launch_plan;

/* The launches rmsnorm_quant_group_multi_ex would make for these arguments,
 * written to *plan, without launching anything and without any HIP call
 * (host arithmetic only, so it runs without a GPU and from any thread).
 * Validates exactly as the launching call does and returns its status; on
 * an error *plan is zeroed. The problems' pointers are checked (alignment,
 * overlap) but never dereferenced. */
rmsq_status rmsq_plan_launch(const rmsq_problem* problems, int32_t count, const rmsq_launch_hint* hint,
                             rmsq_launch_plan* plan);

/*
 * The two kernels the fused call replaces, for callers that need them apart
 * (the separate-quant fallback of [ARQ, Fallback order]) and for measuring
 * what the fusion saves. Their composition equals rmsnorm_quant_group bit
 * for bit.
 *
 * add_rmsnorm: [ARQ, kernel count table] "add_rmsnorm_quant_kernel
 * (RMSNorm+add)": h = bf16(x + residual_in) written to residual_out (both
 * NULL: h = x), and the bf16 normalized rows to out_bf16 (required). N must
 * be a multiple of 8 and at most RMSQ_N_MAX; contiguous rows (ld = N).
 */
rmsq_status add_rmsnorm(const void* x, const void* residual_in, const void* gamma, float eps,
                        int64_t M, int64_t N, void* residual_out, void* out_bf16, void* stream);

/*
 * dynamic_per_group_scaled_quant: [ARQ, kernel count table] "dynamic per
 * group scaled quant kernel" / [ARQ, Fallback order] the separate per-1x128
 * quant: per-group dynamic quantization of M contiguous bf16 rows `x` of N
 * elements, with the group scales, codes and scale layouts of
 * rmsnorm_quant_group_multi.
 */
rmsq_status dynamic_per_group_scaled_quant(const void* x, int64_t M, int64_t N, int32_t group, int32_t fmt,
                                           int32_t scale_layout, void* out_q, void* out_scale, void* stream);

/*
 * gemm_a16wfp4_prequant: [ATT, required aiter changes] the A16WFP4 GEMM with
 * the activation quantization inside the GEMM ("prequant"), which the page
 * pairs with the norm fused into the all-reduce at concurrency 4 (small M).
 *   out[m, n] = sum_k dq(a)[m, k] * dq(w)[n, k]
 * where dq(a) is the MXFP4 group quantization (1x32 along K, e8m0 scale from
 * the group amax, e2m1 codes rounded to nearest even, as
 * rmsnorm_quant_group_multi computes it for RMSQ_FMT_MXFP4_E2M1) of each bf16
 * row of `a`, dequantized, and dq(w) the dequantized weights. Products are
 * exact in fp32 when they lie in its normal range, and accumulate in fp32 on
 * the matrix cores in an order fixed for a given shape (so results repeat
 * bit for bit).
 *
 *  a        [M, K] bf16, row stride lda elements (K <= lda <= RMSQ_GEMM_LDA_MAX,
 *           lda % 8 == 0), 16-byte aligned, read only; finite values.
 *  w        e2m1 codes, N * K/2 bytes in layout w_layout, 16-byte aligned.
 *  w_scale  e8m0 bytes (scale 2^(byte - 127)), N * K/32 bytes in layout
 *           w_layout; byte 255 is not a number and gives unspecified results.
 *  w_layout RMSQ_W_ROW_MAJOR or RMSQ_W_PRESHUFFLED (faster loads).
 *  out      [M, N] fp32, row stride ldc >= N, 4-byte aligned, written, must
 *           not overlap the inputs.
 *  M >= 0 (0: nothing is launched), N a positive multiple of 16 up to
 *  RMSQ_GEMM_N_MAX, K a positive multiple of 128 up to RMSQ_GEMM_K_MAX.
 *  Tuned for small M (decode batches); any M up to 65535 * 64 is accepted.
 * The caller owns every buffer. Bad sizes, strides, layout, alignment or
 * overlap: RMSQ_ERR_INVALID_ARG, nothing launched. Asynchronous on `stream`.
 */
rmsq_status gemm_a16wfp4_prequant(const void* a, int64_t lda, const void* w, const void* w_scale, int32_t w_layout,
                                  int64_t M, int64_t N, int64_t K, void* out, int64_t ldc, void* stream);

/*
 * mxfp4_weight_preshuffle: [ATT, required aiter changes] the weight
 * preshuffle that the page's preshuffled-weight GEMM relies on, here for
 * MXFP4 weights: rearranges row-major codes `w` [N, K/2] and scales
 * `w_scale` [N, K/32] into RMSQ_W_PRESHUFFLED order in `w_out` and
 * `w_scale_out` (same sizes, caller-owned, must not overlap the inputs; w and
 * w_out 16-byte aligned). A byte permutation, done once per weight matrix.
 * N, K as for gemm_a16wfp4_prequant. Errors as there. Asynchronous.
 */
rmsq_status mxfp4_weight_preshuffle(const void* w, const void* w_scale, int64_t N, int64_t K, void* w_out,
                                    void* w_scale_out, void* stream);

/*
 * gemm_a16w8_prequant: [ATT, required aiter changes] the a16w8 GEMM of the
 * page's DS FP8 runs, with the activation quantization inside the GEMM as in
 * gemm_a16wfp4_prequant:
 *   out[m, n] = sum_k dq(a)[m, k] * dq(w)[n, k]
 * where dq(a) is the FP8 group quantization (1x128 along K, fp32 scale
 * amax/448, e4m3fn codes rounded to nearest even, as
 * rmsnorm_quant_group_multi computes it for RMSQ_FMT_FP8_E4M3FN) of each bf16
 * row of `a`, dequantized, and dq(w)[n, k] = w[n, k] * w_scale[n/128, k/128].
 * Each 128-wide K block's sum of code products comes from the matrix cores
 * and is scaled by the two scales and accumulated in fp32, in an order fixed
 * for a given shape.
 *
 *  a        [M, K] bf16, row stride lda elements (K <= lda <= RMSQ_GEMM_LDA_MAX,
 *           lda % 8 == 0), 16-byte aligned, read only; finite values.
 *  w        e4m3fn codes, N * K bytes in layout w_layout (RMSQ_W_ROW_MAJOR:
 *           [N, K]; RMSQ_W_PRESHUFFLED: made by fp8_weight_preshuffle),
 *           16-byte aligned; no NaN codes (0x7F, 0xFF).
 *  w_scale  fp32 [ceil(N/128), K/128] row-major block scales, finite,
 *           4-byte aligned.
 *  out      [M, N] fp32, row stride ldc >= N, 4-byte aligned, written, must
 *           not overlap the inputs.
 *  M, N, K, ownership, errors and the stream as for gemm_a16wfp4_prequant,
 *  except that M may be at most 65535 * 32.
 */
rmsq_status gemm_a16w8_prequant(const void* a, int64_t lda, const void* w, const void* w_scale, int32_t w_layout,
                                int64_t M, int64_t N, int64_t K, void* out, int64_t ldc, void* stream);

/*
 * fp8_weight_preshuffle: [ATT, required aiter changes] the a16w8 GEMM's
 * weight preshuffle: rearranges row-major e4m3fn codes `w` [N, K] into the
 * operand order of gemm_a16w8_prequant in `w_out` (N * K bytes, caller-owned,
 * must not overlap `w`; both 16-byte aligned). For column tile t (rows 16t ..
 * 16t+15), 128-wide K step s, half h in {0, 1} and lane l in 0..63, the 16
 * bytes at ((t * K/128 + s) * 2 + h) * 64 + l (in 16-byte units) are bytes
 * 128s + 32(l/16) + 16h .. +15 of row 16t + l%16. The block scales keep their
 * layout. N, K and errors as for gemm_a16wfp4_prequant. Asynchronous.
 */
rmsq_status fp8_weight_preshuffle(const void* w, int64_t N, int64_t K, void* w_out, void* stream);

/*
 * gemm_afp4wfp4: [ATT, run notes] above concurrency 4 the fused RMSNorm +
 * quant feeds a separate GEMM of the quantized activations with MXFP4
 * weights (gemm_afp4wfp4_preshuffle there), and [ATF, Technical Details]
 * requires the activation scales in the layout that GEMM reads. This one
 * reads what rmsnorm_quant_group_multi and dynamic_per_group_scaled_quant
 * write for RMSQ_FMT_MXFP4_E2M1, in any of their scale layouts:
 *   out[m, n] = sum_k dq(a)[m, k] * dq(w)[n, k]
 * with dq(a)[m, k] = e2m1(a_q[m, k]) * 2^(e - 127), e the scale byte of
 * (row m, group k/32) in layout a_scale_layout, and dq(w) as for
 * gemm_a16wfp4_prequant. Accumulation as there; gemm_afp4wfp4 of the group
 * quantization of rows `a` equals gemm_a16wfp4_prequant of `a` bit for bit
 * when the two run with the same launch shape, and agrees within fp32
 * rounding otherwise.
 *
 *  a_q            [M, K/2] e2m1 codes, rows dense (K/2 bytes apart), element
 *                 2j of a row in the low nibble of byte j; 16-byte aligned.
 *  a_scale        e8m0 bytes, rmsq_scale_bytes(M, K, 32, RMSQ_FMT_MXFP4_E2M1,
 *                 a_scale_layout) of them.
 *  a_scale_layout RMSQ_SCALE_ROW_MAJOR, RMSQ_SCALE_TILED32 or
 *                 RMSQ_SCALE_COL_MAJOR.
 *  w, w_scale, w_layout, out, ldc, M, N, K, ownership, errors and the stream
 *                 as for gemm_a16wfp4_prequant.
 */
rmsq_status gemm_afp4wfp4(const void* a_q, const void* a_scale, int32_t a_scale_layout, const void* w,
                          const void* w_scale, int32_t w_layout, int64_t M, int64_t N, int64_t K, void* out,
                          int64_t ldc, void* stream);

/*
 * gemm_a8w8_blockscale: the FP8 counterpart, [ATT]'s block-scaled a8w8 GEMMs
 * and [FRQ, Motivation]'s (fp8, scale) hand-off to the block-FP8 linear: the
 * activations as rmsnorm_quant_group_multi writes them for
 * RMSQ_FMT_FP8_E4M3FN,
 *   out[m, n] = sum_k (a_q[m, k] * s[m, k/128]) * dq(w)[n, k]
 * with s[m, b] the fp32 scale of (row m, group b) in layout a_scale_layout
 * and dq(w) as for gemm_a16w8_prequant. Each 128-wide K block's sum of code
 * products comes from the matrix cores and is scaled and accumulated in
 * fp32 as there; of the group quantization of rows `a` it equals
 * gemm_a16w8_prequant of `a` within that accumulation's rounding.
 *
 *  a_q            [M, K] e4m3fn codes, rows dense, 16-byte aligned; no NaN
 *                 codes.
 *  a_scale        fp32, M * K/128 of them, finite, 4-byte aligned.
 *  a_scale_layout RMSQ_SCALE_ROW_MAJOR or RMSQ_SCALE_COL_MAJOR.
 *  w, w_scale, w_layout, out, ldc, M, N, K, ownership, errors and the stream
 *                 as for gemm_a16w8_prequant.
 */
rmsq_status gemm_a8w8_blockscale(const void* a_q, const void* a_scale, int32_t a_scale_layout, const void* w,
                                 const void* w_scale, int32_t w_layout, int64_t M, int64_t N, int64_t K, void* out,
                                 int64_t ldc, void* stream);

/* 1 if HIP device `device` is a gfx950 (MI355X-class) GPU, else 0.
 * [ARQ, Motivation]: the single-kernel path is gated to gfx95x devices and
 * callers fall back otherwise; this library's entry points return
 * RMSQ_ERR_UNSUPPORTED on other devices. */
int32_t rmsq_device_supported(int32_t device);

/* Bytes of the scale buffer for a problem (0 for an invalid combination). */
size_t rmsq_scale_bytes(int64_t M, int64_t N, int32_t group, int32_t fmt, int32_t scale_layout);

/* Static, human-readable name of a status code. */
const char* rmsq_status_string(rmsq_status s);

/* Message of the last validation or HIP error on the calling thread, or "". */
const char* rmsq_last_error(void);

/* The launch shape the library picks (without a hint) for rows of N
 * elements, the widest problem of a call, and `rows` rows in total: J chunks
 * of 8 elements per lane and W waves per workgroup (one workgroup per row).
 * RMSQ_ERR_INVALID_ARG for N outside (0, RMSQ_N_MAX] or not a multiple of 8. */
rmsq_status rmsq_query_shape(int64_t N, int64_t rows, int32_t* J, int32_t* W);

#pragma GCC visibility pop

#ifdef __cplusplus
}
#endif
#endif
