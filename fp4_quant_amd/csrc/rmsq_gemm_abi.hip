// rmsq_gemm_abi.hip - C ABI of the GEMMs: argument validation, launch
// configuration and dispatch of the kernels in rmsq_gemm.h.
// Declarations and the contract are in include/rmsq.h.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "rmsq.h"
#include "rmsq_abi_common.h"
#include "rmsq_gemm.h"

namespace {

using namespace rmsq_abi;

// Steps per batch of the quantized-activation MXFP4 kernel with MT row and
// CT column tiles: registers per step are 5 per row tile (codes, scale) and
// 5 per column tile (weights, scale), beside 4 * MT * CT accumulators, within
// 128 per lane.
constexpr int aq_fp4_steps(int MT, int CT) { return CT == 1 ? (MT <= 2 ? 4 : 2) : 2; }

// Column tiles per workgroup of the quantized-activation MXFP4 kernel
// (measured, N = 2112, K = 7168): one up to 64 rows, where the weight stream
// wants the most workgroups; two above (then MT = 4), where each workgroup's
// activation loads - the kernel is bound by vector L1 accesses there - serve
// twice the columns (128 rows: 33 -> 18.7 us, 256 rows: 49 -> 34 us; 64
// rows: 17.4 -> 18.6 us).
int aq_fp4_col_tiles(int64_t M, int64_t N) { return M > 64 && (N / 16) % 2 == 0 ? 2 : 1; }

template <bool SHUF, int MT, int CT, int AQ = 2>
void launch_aq_fp4(const rmsq::GemmArgs& G, dim3 grid, dim3 block, size_t lds, hipStream_t s) {
  hipLaunchKernelGGL((rmsq::rmsq_gemm_fp4_kernel<MT, aq_fp4_steps(MT, CT), SHUF, false, CT, AQ>), grid, block, lds, s,
                     G);
}

// The MXFP4 GEMM: grid x = groups of CT 16-column tiles of the output, y =
// blocks of 64 rows; the row tiles per block (MT) follow M.
template <bool SHUF>
void launch_gemm(const rmsq::GemmArgs& G, int MT, int CT, bool small_m, bool aq, int waves, hipStream_t s) {
  const dim3 grid((unsigned)(G.N / (16 * CT)),
                  (unsigned)((G.M + rmsq::kGemmRowsPerBlock - 1) / rmsq::kGemmRowsPerBlock)),
      block(64 * waves);
  const size_t lds = rmsq::gemm_lds_bytes(MT, CT, waves);
  constexpr int SS = rmsq::kGemmSmallSteps;
  if (aq) {
    // two column tiles come with four row tiles (aq_fp4_col_tiles); up to
    // four rows the codes are loaded directly, else by pairs of steps
    switch (CT == 2 ? 0 : G.M <= rmsq::kGemmSmallRows ? -1 : MT) {
      case -1: launch_aq_fp4<SHUF, 1, 1, 1>(G, grid, block, lds, s); break;
      case 0: launch_aq_fp4<SHUF, 4, 2>(G, grid, block, lds, s); break;
      case 1: launch_aq_fp4<SHUF, 1, 1>(G, grid, block, lds, s); break;
      case 2: launch_aq_fp4<SHUF, 2, 1>(G, grid, block, lds, s); break;
      case 3: launch_aq_fp4<SHUF, 3, 1>(G, grid, block, lds, s); break;
      default: launch_aq_fp4<SHUF, 4, 1>(G, grid, block, lds, s); break;
    }
    return;
  }
  if (small_m && CT == 2) {
    hipLaunchKernelGGL((rmsq::rmsq_gemm_fp4_kernel<1, SS, SHUF, true, 2, 0>), grid, block, lds, s, G);
    return;
  }
  if (small_m) {
    hipLaunchKernelGGL((rmsq::rmsq_gemm_fp4_kernel<1, SS, SHUF, true, 1, 0>), grid, block, lds, s, G);
    return;
  }
  switch (MT) {
    case 1: hipLaunchKernelGGL((rmsq::rmsq_gemm_fp4_kernel<1, 4, SHUF, false, 1, 0>), grid, block, lds, s, G); break;
    case 2: hipLaunchKernelGGL((rmsq::rmsq_gemm_fp4_kernel<2, 2, SHUF, false, 1, 0>), grid, block, lds, s, G); break;
    case 3: hipLaunchKernelGGL((rmsq::rmsq_gemm_fp4_kernel<3, 1, SHUF, false, 1, 0>), grid, block, lds, s, G); break;
    default: hipLaunchKernelGGL((rmsq::rmsq_gemm_fp4_kernel<4, 1, SHUF, false, 1, 0>), grid, block, lds, s, G); break;
  }
}

rmsq_status check_gemm_weights(int64_t N, int64_t K) {
  if (N <= 0 || K <= 0 || N % 16 || K % 128)
    return fail(RMSQ_ERR_INVALID_ARG, "gemm: need N a positive multiple of 16 and K a positive multiple of 128 "
                "(N=%lld K=%lld)", (long long)N, (long long)K);
  if (K > RMSQ_GEMM_K_MAX || N > RMSQ_GEMM_N_MAX)
    return fail(RMSQ_ERR_INVALID_ARG, "gemm: N=%lld K=%lld beyond the supported sizes", (long long)N, (long long)K);
  return RMSQ_OK;
}

// Checks shared by the GEMMs: weights, M (rows per block `rows`), layout
// and output stride.
rmsq_status check_gemm_shape(int64_t M, int64_t N, int64_t K, int32_t w_layout, int64_t ldc, int64_t rows) {
  if (const rmsq_status st = check_gemm_weights(N, K); st != RMSQ_OK) return st;
  if (M < 0 || (M + rows - 1) / rows > 65535)
    return fail(RMSQ_ERR_INVALID_ARG, "gemm: M=%lld outside [0, 65535 * %lld]", (long long)M, (long long)rows);
  if (w_layout != RMSQ_W_ROW_MAJOR && w_layout != RMSQ_W_PRESHUFFLED)
    return fail(RMSQ_ERR_INVALID_ARG, "gemm: unknown weight layout %d", w_layout);
  if (ldc < N) return fail(RMSQ_ERR_INVALID_ARG, "gemm: need ldc >= N (ldc=%lld)", (long long)ldc);
  return RMSQ_OK;
}

// The activations (prequant: bf16 rows a with stride lda; quantized: codes
// a_q and scales a_scale in layout a_layout) and their byte ranges.
struct GemmActs {
  const void* a;
  int64_t lda;
  const void* a_q;
  const void* a_scale;
  int32_t a_layout;
  bool quantized;
};

rmsq_status check_gemm_acts(const GemmActs& A, int32_t fmt, int64_t M, int64_t K, Range* rs, int* nr) {
  if (!A.quantized) {
    if (A.lda < K || A.lda % 8 || A.lda > RMSQ_GEMM_LDA_MAX)
      return fail(RMSQ_ERR_INVALID_ARG, "gemm: need K <= lda <= %d with lda %% 8 == 0 (lda=%lld)", RMSQ_GEMM_LDA_MAX,
                  (long long)A.lda);
    if (M == 0) return RMSQ_OK;
    if (!A.a) return fail(RMSQ_ERR_INVALID_ARG, "gemm: NULL buffer");
    if (!aligned(A.a, 16)) return fail(RMSQ_ERR_INVALID_ARG, "gemm: a must be 16-byte aligned");
    const uintptr_t pa = reinterpret_cast<uintptr_t>(A.a);
    rs[(*nr)++] = Range{pa, pa + (uintptr_t)(((M - 1) * A.lda + K) * 2), false, 0, 0};
    return RMSQ_OK;
  }
  const bool fp8 = fmt == RMSQ_FMT_FP8_E4M3FN;
  if (A.a_layout != RMSQ_SCALE_ROW_MAJOR && A.a_layout != RMSQ_SCALE_COL_MAJOR &&
      (fp8 || A.a_layout != RMSQ_SCALE_TILED32))
    return fail(RMSQ_ERR_INVALID_ARG, "gemm: activation scale layout %d not defined for this format", A.a_layout);
  if (M == 0) return RMSQ_OK;
  if (!A.a_q || !A.a_scale) return fail(RMSQ_ERR_INVALID_ARG, "gemm: NULL buffer");
  if (!aligned(A.a_q, 16) || (fp8 && !aligned(A.a_scale, 4)))
    return fail(RMSQ_ERR_INVALID_ARG, "gemm: a_q must be 16-byte aligned%s", fp8 ? ", a_scale 4-byte aligned" : "");
  const uintptr_t pq = reinterpret_cast<uintptr_t>(A.a_q), ps = reinterpret_cast<uintptr_t>(A.a_scale);
  rs[(*nr)++] = Range{pq, pq + (uintptr_t)(M * (fp8 ? K : K / 2)), false, 0, 0};
  rs[(*nr)++] = Range{ps, ps + (uintptr_t)rmsq_scale_bytes(M, K, fp8 ? 128 : 32, fmt, A.a_layout), false, 0, 5};
  return RMSQ_OK;
}

rmsq_status run_gemm(const GemmActs& A, const void* w, const void* w_scale, int32_t w_layout, int64_t M, int64_t N,
                     int64_t K, void* out, int64_t ldc, void* stream) {
  g_err[0] = 0;
  if (const rmsq_status st = check_gemm_shape(M, N, K, w_layout, ldc, rmsq::kGemmRowsPerBlock); st != RMSQ_OK)
    return st;
  Range rs[5];
  int nr = 0;
  if (const rmsq_status st = check_gemm_acts(A, RMSQ_FMT_MXFP4_E2M1, M, K, rs, &nr); st != RMSQ_OK) return st;
  if (M == 0) return RMSQ_OK;
  if (!w || !w_scale || !out) return fail(RMSQ_ERR_INVALID_ARG, "gemm: NULL buffer");
  if (!aligned(w, 16) || !aligned(out, 4))
    return fail(RMSQ_ERR_INVALID_ARG, "gemm: w must be 16-byte aligned, out 4-byte aligned");
  const uintptr_t pw = reinterpret_cast<uintptr_t>(w), ps = reinterpret_cast<uintptr_t>(w_scale),
                  po = reinterpret_cast<uintptr_t>(out);
  rs[nr++] = {pw, pw + (uintptr_t)(N * (K / 2)), false, 0, 3};
  rs[nr++] = {ps, ps + (uintptr_t)(N * (K / 32)), false, 0, 5};
  rs[nr++] = {po, po + (uintptr_t)(((M - 1) * ldc + N) * 4), true, 0, 4};
  if (const rmsq_status st = check_overlaps(rs, nr); st != RMSQ_OK) return st;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || !device_is_gfx950(dev))
    return fail(RMSQ_ERR_UNSUPPORTED, "current HIP device is not a gfx950 GPU");
  rmsq::GemmArgs G;
  G.a = static_cast<const uint16_t*>(A.a);
  G.aq = static_cast<const uint8_t*>(A.a_q);
  G.as = static_cast<const uint8_t*>(A.a_scale);
  G.a_layout = A.a_layout;
  G.w = static_cast<const uint8_t*>(w);
  G.ws = static_cast<const uint8_t*>(w_scale);
  G.out = static_cast<float*>(out);
  G.lda = A.lda;
  G.ldc = ldc;
  G.M = (int32_t)M;
  G.N = (int32_t)N;
  G.K = (int32_t)K;
  // Row tiles per block and waves per workgroup. Small M of bf16 activations
  // (at most 4 rows): enough waves that each covers at most 4 steps, one
  // batch. Otherwise SW steps per batch (registers: 16 per step and tile for
  // bf16 activations, 5 for quantized ones, 5 for the weights) and enough
  // waves that each wave's K range is one batch, at most 16.
  const int MT = M >= 64 ? 4 : (int)((M + 15) / 16);
  const int steps = (int)(K / 128);
  const int small_waves = (steps + rmsq::kGemmSmallSteps - 1) / rmsq::kGemmSmallSteps;
  const bool small_m = !A.quantized && M <= rmsq::kGemmSmallRows && small_waves <= rmsq::kGemmMaxWaves;
  // Column tiles per workgroup: on the small-M path two once there are at
  // least 256 tiles (half as many workgroups each quantize the activations
  // for twice the weights); for quantized activations as aq_fp4_col_tiles
  // chooses (N divisible).
  int CT = small_m && (N / 16) % 2 == 0 && N / 16 >= kComputeUnits ? 2 : 1;
  if (A.quantized) CT = MT == 4 ? aq_fp4_col_tiles(M, N) : 1;
  const int SW = A.quantized ? aq_fp4_steps(MT, CT) : MT == 1 ? 4 : MT == 2 ? 2 : 1;
  // the waves' partial sums (1 KiB per row and column tile of each wave)
  // stay within 64 KiB of LDS
  const int waves = std::min(rmsq::gemm_max_waves(MT * CT), small_m ? small_waves
                                                         : std::min(rmsq::kGemmMaxWaves,
                                                                    std::max(1, (steps + SW - 1) / SW)));
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (w_layout == RMSQ_W_PRESHUFFLED)
    launch_gemm<true>(G, MT, CT, small_m, A.quantized, waves, s);
  else
    launch_gemm<false>(G, MT, CT, small_m, A.quantized, waves, s);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(RMSQ_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return RMSQ_OK;
}

// The FP8 GEMM: the same grid as the MXFP4 one with blocks of 16 MT rows,
// one column tile per workgroup.
template <bool SHUF>
void launch_gemm8(const rmsq::Gemm8Args& G, int MT, bool small_m, bool aq, int waves, hipStream_t s) {
  const dim3 grid((unsigned)(G.N / 16), (unsigned)((G.M + 16 * MT - 1) / (16 * MT))), block(64 * waves);
  const size_t lds = rmsq::gemm8_lds_bytes(MT, waves);
  if (aq) {   // quantized activations: 9 registers per step and tile beside the weights' 9; up to
              // eight rows the codes are loaded directly, else 8 rows per load (as for MXFP4; measured:
              // 8 rows 5.65 direct vs 6.02 us, 16 rows 7.53 vs 6.14 us)
    if (G.M <= 2 * rmsq::kGemmSmallRows)
      hipLaunchKernelGGL((rmsq::rmsq_gemm_fp8_kernel<1, 4, SHUF, false, 1>), grid, block, lds, s, G);
    else if (MT == 1)
      hipLaunchKernelGGL((rmsq::rmsq_gemm_fp8_kernel<1, 4, SHUF, false, 2>), grid, block, lds, s, G);
    else
      hipLaunchKernelGGL((rmsq::rmsq_gemm_fp8_kernel<2, 2, SHUF, false, 2>), grid, block, lds, s, G);
  } else if (small_m) {
    hipLaunchKernelGGL((rmsq::rmsq_gemm_fp8_kernel<1, rmsq::kGemmSmallSteps, SHUF, true, 0>), grid, block, lds, s, G);
  } else if (MT == 1) {
    hipLaunchKernelGGL((rmsq::rmsq_gemm_fp8_kernel<1, 2, SHUF, false, 0>), grid, block, lds, s, G);
  } else {
    hipLaunchKernelGGL((rmsq::rmsq_gemm_fp8_kernel<2, 1, SHUF, false, 0>), grid, block, lds, s, G);
  }
}

rmsq_status run_gemm8(const GemmActs& A, const void* w, const void* w_scale, int32_t w_layout, int64_t M, int64_t N,
                      int64_t K, void* out, int64_t ldc, void* stream) {
  g_err[0] = 0;
  if (const rmsq_status st = check_gemm_shape(M, N, K, w_layout, ldc, 16 * rmsq::kGemm8MaxTiles); st != RMSQ_OK)
    return st;
  Range rs[5];
  int nr = 0;
  if (const rmsq_status st = check_gemm_acts(A, RMSQ_FMT_FP8_E4M3FN, M, K, rs, &nr); st != RMSQ_OK) return st;
  if (M == 0) return RMSQ_OK;
  if (!w || !w_scale || !out) return fail(RMSQ_ERR_INVALID_ARG, "gemm: NULL buffer");
  if (!aligned(w, 16) || !aligned(w_scale, 4) || !aligned(out, 4))
    return fail(RMSQ_ERR_INVALID_ARG, "gemm: w must be 16-byte aligned, w_scale and out 4-byte aligned");
  const uintptr_t pw = reinterpret_cast<uintptr_t>(w), ps = reinterpret_cast<uintptr_t>(w_scale),
                  po = reinterpret_cast<uintptr_t>(out);
  rs[nr++] = {pw, pw + (uintptr_t)(N * K), false, 0, 3};
  rs[nr++] = {ps, ps + (uintptr_t)(((N + 127) / 128) * (K / 128) * 4), false, 0, 5};
  rs[nr++] = {po, po + (uintptr_t)(((M - 1) * ldc + N) * 4), true, 0, 4};
  if (const rmsq_status st = check_overlaps(rs, nr); st != RMSQ_OK) return st;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || !device_is_gfx950(dev))
    return fail(RMSQ_ERR_UNSUPPORTED, "current HIP device is not a gfx950 GPU");
  rmsq::Gemm8Args G;
  G.a = static_cast<const uint16_t*>(A.a);
  G.aq = static_cast<const uint8_t*>(A.a_q);
  G.as = static_cast<const float*>(A.a_scale);
  G.a_layout = A.a_layout;
  G.w = static_cast<const uint8_t*>(w);
  G.ws = static_cast<const float*>(w_scale);
  G.out = static_cast<float*>(out);
  G.lda = A.lda;
  G.ldc = ldc;
  G.M = (int32_t)M;
  G.N = (int32_t)N;
  G.K = (int32_t)K;
  // as for the MXFP4 GEMM, with 8 registers per step for the weights and
  // 16 (bf16) or 8 (codes) per step and tile for the activations, at most
  // two row tiles
  const int MT = M > 16 ? 2 : 1;
  const int steps = (int)(K / 128);
  const int small_waves = (steps + rmsq::kGemmSmallSteps - 1) / rmsq::kGemmSmallSteps;
  const bool small_m = !A.quantized && M <= rmsq::kGemmSmallRows && small_waves <= rmsq::kGemmMaxWaves;
  const int SW = A.quantized ? (MT == 1 ? 4 : 2) : MT == 1 ? 2 : 1;
  const int waves = small_m ? small_waves : std::min(rmsq::kGemmMaxWaves, std::max(1, (steps + SW - 1) / SW));
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (w_layout == RMSQ_W_PRESHUFFLED)
    launch_gemm8<true>(G, MT, small_m, A.quantized, waves, s);
  else
    launch_gemm8<false>(G, MT, small_m, A.quantized, waves, s);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(RMSQ_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return RMSQ_OK;
}

rmsq_status run_preshuffle8(const void* w, int64_t N, int64_t K, void* w_out, void* stream) {
  g_err[0] = 0;
  if (const rmsq_status st = check_gemm_weights(N, K); st != RMSQ_OK) return st;
  if (!w || !w_out) return fail(RMSQ_ERR_INVALID_ARG, "preshuffle: NULL buffer");
  if (!aligned(w, 16) || !aligned(w_out, 16))
    return fail(RMSQ_ERR_INVALID_ARG, "preshuffle: w and w_out must be 16-byte aligned");
  Range rs[2];
  const uintptr_t pw = reinterpret_cast<uintptr_t>(w), qw = reinterpret_cast<uintptr_t>(w_out);
  rs[0] = {pw, pw + (uintptr_t)(N * K), false, 0, 3};
  rs[1] = {qw, qw + (uintptr_t)(N * K), true, 0, 4};
  if (const rmsq_status st = check_overlaps(rs, 2); st != RMSQ_OK) return st;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || !device_is_gfx950(dev))
    return fail(RMSQ_ERR_UNSUPPORTED, "current HIP device is not a gfx950 GPU");
  const int64_t units = N * (K / 16);
  const unsigned blocks = (unsigned)std::min<int64_t>((units + 255) / 256, 4096);
  hipLaunchKernelGGL(rmsq::rmsq_fp8_preshuffle_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint8_t*>(w), static_cast<uint8_t*>(w_out), (int32_t)K, units);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(RMSQ_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return RMSQ_OK;
}

rmsq_status run_preshuffle(const void* w, const void* w_scale, int64_t N, int64_t K, void* w_out, void* w_scale_out,
                           void* stream) {
  g_err[0] = 0;
  if (const rmsq_status st = check_gemm_weights(N, K); st != RMSQ_OK) return st;
  if (!w || !w_scale || !w_out || !w_scale_out) return fail(RMSQ_ERR_INVALID_ARG, "preshuffle: NULL buffer");
  if (!aligned(w, 16) || !aligned(w_out, 16))
    return fail(RMSQ_ERR_INVALID_ARG, "preshuffle: w and w_out must be 16-byte aligned");
  Range rs[4];
  const uintptr_t pw = reinterpret_cast<uintptr_t>(w), ps = reinterpret_cast<uintptr_t>(w_scale),
                  qw = reinterpret_cast<uintptr_t>(w_out), qs = reinterpret_cast<uintptr_t>(w_scale_out);
  rs[0] = {pw, pw + (uintptr_t)(N * (K / 2)), false, 0, 3};
  rs[1] = {ps, ps + (uintptr_t)(N * (K / 32)), false, 0, 5};
  rs[2] = {qw, qw + (uintptr_t)(N * (K / 2)), true, 0, 4};
  rs[3] = {qs, qs + (uintptr_t)(N * (K / 32)), true, 0, 5};
  if (const rmsq_status st = check_overlaps(rs, 4); st != RMSQ_OK) return st;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || !device_is_gfx950(dev))
    return fail(RMSQ_ERR_UNSUPPORTED, "current HIP device is not a gfx950 GPU");
  const int64_t units = N * (K / 32);
  const unsigned blocks = (unsigned)std::min<int64_t>((units + 255) / 256, 4096);
  hipLaunchKernelGGL(rmsq::rmsq_mxfp4_preshuffle_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint8_t*>(w), static_cast<const uint8_t*>(w_scale),
                     static_cast<uint8_t*>(w_out), static_cast<uint8_t*>(w_scale_out), (int32_t)K, units);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(RMSQ_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return RMSQ_OK;
}

}  // namespace

extern "C" {

rmsq_status gemm_a16wfp4_prequant(const void* a, int64_t lda, const void* w, const void* w_scale, int32_t w_layout,
                                  int64_t M, int64_t N, int64_t K, void* out, int64_t ldc, void* stream) {
  return run_gemm(GemmActs{a, lda, nullptr, nullptr, 0, false}, w, w_scale, w_layout, M, N, K, out, ldc, stream);
}

rmsq_status gemm_afp4wfp4(const void* a_q, const void* a_scale, int32_t a_scale_layout, const void* w,
                          const void* w_scale, int32_t w_layout, int64_t M, int64_t N, int64_t K, void* out,
                          int64_t ldc, void* stream) {
  return run_gemm(GemmActs{nullptr, 0, a_q, a_scale, a_scale_layout, true}, w, w_scale, w_layout, M, N, K, out, ldc,
                  stream);
}

rmsq_status mxfp4_weight_preshuffle(const void* w, const void* w_scale, int64_t N, int64_t K, void* w_out,
                                    void* w_scale_out, void* stream) {
  return run_preshuffle(w, w_scale, N, K, w_out, w_scale_out, stream);
}

rmsq_status gemm_a16w8_prequant(const void* a, int64_t lda, const void* w, const void* w_scale, int32_t w_layout,
                                int64_t M, int64_t N, int64_t K, void* out, int64_t ldc, void* stream) {
  return run_gemm8(GemmActs{a, lda, nullptr, nullptr, 0, false}, w, w_scale, w_layout, M, N, K, out, ldc, stream);
}

rmsq_status gemm_a8w8_blockscale(const void* a_q, const void* a_scale, int32_t a_scale_layout, const void* w,
                                 const void* w_scale, int32_t w_layout, int64_t M, int64_t N, int64_t K, void* out,
                                 int64_t ldc, void* stream) {
  return run_gemm8(GemmActs{nullptr, 0, a_q, a_scale, a_scale_layout, true}, w, w_scale, w_layout, M, N, K, out, ldc,
                   stream);
}

rmsq_status fp8_weight_preshuffle(const void* w, int64_t N, int64_t K, void* w_out, void* stream) {
  return run_preshuffle8(w, N, K, w_out, stream);
}

}  // extern "C"
