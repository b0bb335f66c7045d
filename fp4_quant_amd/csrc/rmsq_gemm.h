// rmsq_gemm.h - A16WFP4 "prequant" GEMM for gfx950: bf16 activations are
// quantized to MXFP4 inside the GEMM and multiplied with MXFP4 weights on the
// block-scaled matrix cores.
//
// Source, cited by title: [ATT] "[Triton] DS FP4/FP8 Triton fusion and GEMM
// optimization" lists an A16WFP4 GEMM that quantizes its activations inside
// the GEMM (with a preshuffled-weight GEMM beside it), used at concurrency 4
// (small M), where the norm is fused with the all-reduce and the group
// quantization moves into the GEMM.
//
// C[m, n] = sum_k qa[m, k] 2^(ea[m, k/32] - 127) * qw[n, k] 2^(ew[n, k/32] - 127)
// with (qa, ea) the MXFP4 group quantization (1x32 along K) of the bf16 row
// a[m, :] - the same rule and arithmetic as the fused kernel's MXFP4 path -
// and (qw, ew) the given weights. Products accumulate in fp32 on the matrix
// cores.
//
// Mapping (small M, where the weights dominate the traffic). A workgroup of
// up to 16 waves owns 16 output columns (one tile) and up to 64 rows (MT
// tiles of 16 rows); its waves split K into contiguous ranges of 128-wide
// steps. Per step and row tile a wave issues one
// v_mfma_scale_f32_16x16x128_f8f6f4: lane l holds weight row n0 + l%16 and
// activation row m0 + 16t + l%16, K elements 32*(l/16) .. +31 of the step
// (16 bytes of e2m1 codes and one e8m0 byte each), so the scale of each
// lane's operand is that of one 1x32 group. The waves' partial accumulators
// meet in LDS and are summed in wave order (a fixed order for a given shape).
//
// Weights come row-major ([N, K/2] codes, [N, K/32] scales) or preshuffled
// into exactly the operand order above: for tile t and step s, 64 lanes x 16
// bytes contiguous (codes) and 64 bytes (scales), so every weight load of a
// wave reads 1 KiB of consecutive bytes.
//
// Activations: with at most 4 rows and one batch of steps per wave, the
// workgroup first loads its rows with all lanes (consecutive 16-byte chunks,
// issued before the weight loads so the two latencies overlap), quantizes
// each 32-group once in lane quads, and keeps the codes in LDS, from where
// each wave reads its operands. Otherwise each wave loads and quantizes the
// 32-groups of its own operands (lanes of rows past M load nothing).
#pragma once

#include <algorithm>

#include "rmsq_device.h"

namespace rmsq {

typedef int v8i32 __attribute__((ext_vector_type(8)));
typedef float v4f32 __attribute__((ext_vector_type(4)));

struct GemmArgs {
  const uint16_t* a;      // bf16 [M, K], row stride lda elements
  const uint8_t* w;       // e2m1 codes, row-major [N, K/2] or preshuffled
  const uint8_t* ws;      // e8m0 scales, row-major [N, K/32] or preshuffled
  float* out;             // fp32 [M, N], row stride ldc elements
  int64_t lda, ldc;
  int32_t M, N, K;
};

constexpr int kGemmMaxWaves = 16;
constexpr int kGemmRowsPerBlock = 64;   // 4 tiles of 16 rows
constexpr int kGemmStagedRows = 4;      // at most this many activation rows are staged in LDS
constexpr int kGemmStagedChunks = 4;    // 8-element chunks per lane when staging
constexpr int kGemmStagedSteps = 4;     // steps per wave when staging (one batch)

// MXFP4 quantization of one 32-element bf16 group held by one lane (16
// packed dwords): the e8m0 byte and the 4 dwords of e2m1 codes.
__device__ __forceinline__ uint32_t mx_group32(const u32x4 v[4], u32x4* codes) {
  const uint32_t am = max(max(amax8(v[0]), amax8(v[1])), max(amax8(v[2]), amax8(v[3])));
  const uint32_t byte = mx_scale_byte(am);
  (*codes)[0] = fp4_codes8(v[0], byte);
  (*codes)[1] = fp4_codes8(v[1], byte);
  (*codes)[2] = fp4_codes8(v[2], byte);
  (*codes)[3] = fp4_codes8(v[3], byte);
  return byte;
}

// LDS bytes the kernel needs: the staged activation codes and scales, or the
// waves' partial sums, whichever is larger (the partial sums reuse the
// staging area after a barrier).
inline size_t gemm_lds_bytes(bool staged, int rows, int K, int MT, int CT, int waves) {
  const size_t stage = staged ? (size_t)(K / 32) * rows * 17 : 0;
  const size_t part = (size_t)(waves - 1) * MT * CT * 64 * sizeof(v4f32);
  return (std::max(stage, part) + 15) & ~(size_t)15;
}

// MT row tiles of 16 rows and CT column tiles per workgroup, SW steps
// loaded per batch, SHUF: preshuffled weights, STAGED: activations staged in
// LDS (MT == 1, SW == kGemmStagedSteps, M <= kGemmStagedRows, M * K/8 <= 4
// chunks per thread, every wave's steps in one batch); CT > 1 only when
// staged, where a wave reuses each activation operand for CT tiles.
template <int MT, int SW, bool SHUF, bool STAGED, int CT>
__global__ void __launch_bounds__(64 * kGemmMaxWaves) rmsq_gemm_a16wfp4_kernel(const GemmArgs G) {
  static_assert(CT == 1 || STAGED, "several column tiles only with staged activations");
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int waves = blockDim.x >> 6;
  const int tile = blockIdx.x * CT;      // first column tile of the workgroup
  const int n = tile * 16 + (lane & 15);
  const int m0 = blockIdx.y * kGemmRowsPerBlock;
  const int kb = lane >> 4;             // 32-element block of the 128-wide step
  const int steps = G.K >> 7;
  const int s_lo = (wave * steps) / waves, s_hi = ((wave + 1) * steps) / waves;

  // weight operand of this lane at step s in column tile tile + ct: 16 bytes
  // of codes at wq + ct * wq_tile + s * ws_step and the scale byte at wsc +
  // ct * ws_tile + s * ws_step
  const u32x4* wq;
  const uint8_t* wsc;
  int ws_step;
  int64_t wq_tile, ws_tile;
  if (SHUF) {
    wq = reinterpret_cast<const u32x4*>(G.w) + (int64_t)tile * steps * 64 + lane;
    wsc = G.ws + (int64_t)tile * steps * 64 + lane;
    ws_step = 64;
    wq_tile = ws_tile = (int64_t)steps * 64;
  } else {
    wq = reinterpret_cast<const u32x4*>(G.w + (int64_t)n * (G.K >> 1)) + kb;
    wsc = G.ws + (int64_t)n * (G.K >> 5) + kb;
    ws_step = 4;
    wq_tile = (int64_t)16 * (G.K >> 5);   // 16 rows of K/2 bytes, in u32x4
    ws_tile = (int64_t)16 * (G.K >> 5);
  }

  // acc[t * CT + ct]: row tile t, column tile ct
  v4f32 acc[MT * CT];
#pragma unroll
  for (int t = 0; t < MT * CT; ++t) acc[t] = v4f32{0.0f, 0.0f, 0.0f, 0.0f};

  if constexpr (STAGED) {
    // rows 0 .. R-1 (a single row block), 8-element chunk c = r * K/8 + kc
    const int R = G.M;
    const int C8 = G.K >> 3, total = R * C8, T = blockDim.x;
    u32x4 v[kGemmStagedChunks];
#pragma unroll
    for (int u = 0; u < kGemmStagedChunks; ++u) {
      const int c = min((int)threadIdx.x + u * T, total - 1);
      const int r = c / C8, kc = c - r * C8;
      v[u] = reinterpret_cast<const u32x4*>(G.a + (int64_t)r * G.lda)[kc];
    }
    __builtin_amdgcn_sched_barrier(0);
    u32x4 bw[CT][SW];
    uint32_t sb[CT][SW];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int i = 0; i < SW; ++i) {
        bw[ct][i] = u32x4{0u, 0u, 0u, 0u};
        sb[ct][i] = 127u;
        if (s_lo + i < s_hi) {
          bw[ct][i] = wq[ct * wq_tile + (s_lo + i) * ws_step];
          sb[ct][i] = wsc[ct * ws_tile + (s_lo + i) * ws_step];
        }
      }
    __builtin_amdgcn_sched_barrier(0);
    // codes of group g of row r at LDS byte (g * R + r) * 16, its scale byte
    // at NG * R * 16 + g * R + r; a lane quad holds the four chunks of a
    // group (T is a multiple of 64 and K/8 of 16, so quads never straddle
    // groups or rows, and every lane of a quad is in or out of range alike)
    const int NG = G.K >> 5;
    uint8_t* codes = lds;
    uint8_t* scl = lds + NG * R * 16;
#pragma unroll
    for (int u = 0; u < kGemmStagedChunks; ++u) {
      const int c = threadIdx.x + u * T;
      const uint32_t byte = mx_scale_byte(max4(amax8(v[u])));
      const uint32_t cw = fp4_codes8(v[u], byte);
      if (c < total) {
        const int r = c / C8, kc = c - r * C8, g = kc >> 2, d = kc & 3;
        *reinterpret_cast<uint32_t*>(codes + (g * R + r) * 16 + d * 4) = cw;
        if (d == 0) scl[g * R + r] = (uint8_t)byte;
      }
    }
    __syncthreads();
    const int r = lane & 15;
    const bool live = r < R;
#pragma unroll
    for (int i = 0; i < SW; ++i) {
      if (s_lo + i >= s_hi) break;
      const int g = (s_lo + i) * 4 + kb;
      u32x4 q = u32x4{0u, 0u, 0u, 0u};
      uint32_t sa = 127u;
      if (live) {
        q = *reinterpret_cast<const u32x4*>(codes + (g * R + r) * 16);
        sa = scl[g * R + r];
      }
      const v8i32 aop = {(int)q[0], (int)q[1], (int)q[2], (int)q[3], 0, 0, 0, 0};
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const v8i32 bop = {(int)bw[ct][i][0], (int)bw[ct][i][1], (int)bw[ct][i][2], (int)bw[ct][i][3], 0, 0, 0, 0};
        acc[ct] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aop, bop, acc[ct], 4, 4, 0, (int)sa, 0,
                                                                   (int)sb[ct][i]);
      }
    }
    __syncthreads();   // the partial sums below reuse the staging area
  } else {
    // activation row of this lane in each tile; rows past M are not loaded
    const u32x4* arow[MT];
    bool live[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const int m = m0 + 16 * t + (lane & 15);
      live[t] = m < G.M;
      arow[t] = reinterpret_cast<const u32x4*>(G.a + (int64_t)min(m, G.M - 1) * G.lda);
    }
    for (int s0 = s_lo; s0 < s_hi; s0 += SW) {
      u32x4 bw[SW];
      uint32_t sb[SW];
      u32x4 av[SW][MT][4];
#pragma unroll
      for (int i = 0; i < SW; ++i) {
        const int kg = (s0 + i) * 4 + kb;   // 32-element group index along K
        const bool in = s0 + i < s_hi;      // wave-uniform
        bw[i] = u32x4{0u, 0u, 0u, 0u};
        sb[i] = 127u;
        if (in) {
          bw[i] = wq[(s0 + i) * ws_step];
          sb[i] = wsc[(s0 + i) * ws_step];
        }
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            av[i][t][j] = u32x4{0u, 0u, 0u, 0u};
            if (in && live[t]) av[i][t][j] = arow[t][kg * 4 + j];   // 64 bytes = 32 bf16
          }
      }
#pragma unroll
      for (int i = 0; i < SW; ++i) {
        if (s0 + i >= s_hi) break;
        const v8i32 bop = {(int)bw[i][0], (int)bw[i][1], (int)bw[i][2], (int)bw[i][3], 0, 0, 0, 0};
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          u32x4 q;
          const uint32_t sa = mx_group32(av[i][t], &q);
          const v8i32 aop = {(int)q[0], (int)q[1], (int)q[2], (int)q[3], 0, 0, 0, 0};
          acc[t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aop, bop, acc[t], 4, 4, 0, (int)sa, 0, (int)sb[i]);
        }
      }
    }
  }

  // the waves' partial sums meet in LDS; wave 0 adds them in wave order
  v4f32* part = reinterpret_cast<v4f32*>(lds);
  if (wave > 0) {
#pragma unroll
    for (int t = 0; t < MT * CT; ++t) part[((wave - 1) * MT * CT + t) * 64 + lane] = acc[t];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int t = 0; t < MT * CT; ++t) {
    v4f32 c = acc[t];
    for (int w = 0; w < waves - 1; ++w) c += part[(w * MT * CT + t) * 64 + lane];
    // result lane l: column 16 (tile + ct) + l%16, rows 16 (t / CT) + 4 (l/16) + r
    const int col = n + 16 * (t % CT);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m0 + 16 * (t / CT) + 4 * (lane >> 4) + r;
      if (m < G.M) G.out[(int64_t)m * G.ldc + col] = c[r];
    }
  }
}

// Row-major MXFP4 weights to the preshuffled operand order: one thread per
// 16-byte unit u = (t * steps + s) * 64 + l of the output, which holds the
// codes of row 16t + l%16, 32-group 4s + l/16 (and the matching scale byte).
__global__ void __launch_bounds__(256) rmsq_mxfp4_preshuffle_kernel(const uint8_t* w, const uint8_t* ws,
                                                                    uint8_t* w_out, uint8_t* ws_out, int32_t K,
                                                                    int64_t units) {
  const int64_t steps = K >> 7;
  for (int64_t u = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; u < units;
       u += (int64_t)gridDim.x * blockDim.x) {
    const int l = (int)(u & 63);
    const int64_t ts = u >> 6, t = ts / steps, s = ts - t * steps;
    const int64_t row = t * 16 + (l & 15), g = s * 4 + (l >> 4);
    reinterpret_cast<u32x4*>(w_out)[u] = reinterpret_cast<const u32x4*>(w + row * (K >> 1))[g];
    ws_out[u] = ws[row * (K >> 5) + g];
  }
}

// ------------------------------------------------------------------ A16W8 --
// The FP8 counterpart ([ATT] lists an a16w8 GEMM for its DS FP8 runs): bf16
// activations quantized per 1x128 group along K to e4m3fn with fp32 scales
// (the fused kernel's FP8 rule: s = amax/448, exact codes), e4m3fn weights
// [N, K] with fp32 scales per 128x128 block [ceil(N/128), K/128]:
//   C[m, n] = sum over K blocks b of sa[m, b] sw[n/128, b] sum_{k in b} qa[m, k] qw[n, k].
// One 128-wide K step is one scale block, so each step's
// v_mfma_scale_f32_16x16x128_f8f6f4 (e4m3fn operands, unit scales) yields
// the block's integer-grid sum, which is scaled by sa * sw and added in fp32.
// Lane l holds activation row l%16 and weight row n0 + l%16, K elements
// 32*(l/16) .. +31 of the step (32 bytes each); result lane l holds column
// l%16, rows 4*(l/16) .. +3, whose activation scales it fetches from the
// lanes that own those rows. A 16-row weight tile lies in one 128-row scale
// block, so the weight scale of a step is one wave-uniform fp32 value.
//
// Weights come row-major or preshuffled: for tile t, step s and half h, the
// 16-byte halves of the 64 lanes' operands contiguous (1 KiB), so each weight
// load of a wave reads consecutive bytes.

struct Gemm8Args {
  const uint16_t* a;      // bf16 [M, K], row stride lda elements
  const uint8_t* w;       // e4m3fn codes, row-major [N, K] or preshuffled
  const float* ws;        // fp32 block scales [ceil(N/128), K/128]
  float* out;             // fp32 [M, N], row stride ldc elements
  int64_t lda, ldc;
  int32_t M, N, K;
};

// LDS bytes of the A16W8 kernel: staged codes (128 B) and scales (4 B) per
// row and K block, or the waves' partial sums.
inline size_t gemm8_lds_bytes(bool staged, int rows, int K, int MT, int waves) {
  const size_t stage = staged ? (size_t)(K / 128) * rows * (128 + 4) : 0;
  const size_t part = (size_t)(waves - 1) * MT * 64 * sizeof(v4f32);
  return (std::max(stage, part) + 15) & ~(size_t)15;
}

__device__ __forceinline__ void unpack_bf16x8(const u32x4 w, float f[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_lo(w[i]);
    f[2 * i + 1] = bf16_hi(w[i]);
  }
}

// e4m3fn codes of 32 bf16 values (16 dwords) under scale sc: 8 dwords, element
// order.
__device__ __forceinline__ v8i32 fp8_codes32(const u32x4 v[4], float sc) {
  v8i32 q;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float f[8];
    unpack_bf16x8(v[i], f);
    const u32x2 c = fp8_codes8(f, sc);
    q[2 * i] = (int)c[0];
    q[2 * i + 1] = (int)c[1];
  }
  return q;
}

// MT row tiles per workgroup, SW steps per batch, SHUF: preshuffled weights,
// STAGED: activations staged in LDS (MT == 1, SW == kGemmStagedSteps,
// M <= kGemmStagedRows, M * K/8 <= 4 chunks per thread, one batch per wave).
// Row blocks are 16 * MT rows (MT <= kGemm8MaxTiles: the activation
// registers of more tiles would not fit beside the 32-byte operands).
constexpr int kGemm8MaxTiles = 2;

template <int MT, int SW, bool SHUF, bool STAGED>
__global__ void __launch_bounds__(64 * kGemmMaxWaves) rmsq_gemm_a16w8_kernel(const Gemm8Args G) {
  static_assert(MT <= kGemm8MaxTiles, "at most two row tiles");
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int waves = blockDim.x >> 6;
  const int tile = blockIdx.x;
  const int n = tile * 16 + (lane & 15);
  const int m0 = blockIdx.y * 16 * MT;
  const int kb = lane >> 4;             // 32-element quarter of the 128-wide step
  const int steps = G.K >> 7;
  const int s_lo = (wave * steps) / waves, s_hi = ((wave + 1) * steps) / waves;

  // weight operand of this lane at step s: halves wq[s * wstep] and
  // wq[s * wstep + whalf]; the tile's block scale of step s: wsrow[s]
  const u32x4* wq;
  int wstep, whalf;
  if (SHUF) {
    wq = reinterpret_cast<const u32x4*>(G.w) + (int64_t)tile * steps * 128 + lane;
    wstep = 128;
    whalf = 64;
  } else {
    wq = reinterpret_cast<const u32x4*>(G.w + (int64_t)n * G.K) + 2 * kb;
    wstep = 8;
    whalf = 1;
  }
  const float* wsrow = G.ws + (int64_t)(tile >> 3) * steps;

  v4f32 acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = v4f32{0.0f, 0.0f, 0.0f, 0.0f};

  if constexpr (STAGED) {
    // rows 0 .. R-1 (a single row block), 8-element chunk c = r * K/8 + kc;
    // a 16-lane DPP row holds one 128-group
    const int R = G.M;
    const int C8 = G.K >> 3, total = R * C8, T = blockDim.x;
    u32x4 v[kGemmStagedChunks];
#pragma unroll
    for (int u = 0; u < kGemmStagedChunks; ++u) {
      const int c = min((int)threadIdx.x + u * T, total - 1);
      const int r = c / C8, kc = c - r * C8;
      v[u] = reinterpret_cast<const u32x4*>(G.a + (int64_t)r * G.lda)[kc];
    }
    __builtin_amdgcn_sched_barrier(0);
    u32x4 bw[SW][2];
    float sw[SW];
#pragma unroll
    for (int i = 0; i < SW; ++i) {
      bw[i][0] = bw[i][1] = u32x4{0u, 0u, 0u, 0u};
      sw[i] = 0.0f;
      if (s_lo + i < s_hi) {
        bw[i][0] = wq[(s_lo + i) * wstep];
        bw[i][1] = wq[(s_lo + i) * wstep + whalf];
        sw[i] = wsrow[s_lo + i];
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // codes of group g of row r at LDS byte (g * R + r) * 128, its fp32 scale
    // at byte NG * R * 128 + (g * R + r) * 4 (T is a multiple of 64 and K/8 of
    // 16, so a 16-lane row never straddles groups and is in or out of range
    // as a whole)
    const int NG = G.K >> 7;
    uint8_t* codes = lds;
    float* scl = reinterpret_cast<float*>(lds + NG * R * 128);
#pragma unroll
    for (int u = 0; u < kGemmStagedChunks; ++u) {
      const int c = threadIdx.x + u * T;
      const float sc = fp8_scale(max16(amax8(v[u])));
      float f[8];
      unpack_bf16x8(v[u], f);
      const u32x2 q = fp8_codes8(f, sc);
      if (c < total) {
        const int r = c / C8, kc = c - r * C8, g = kc >> 4, d = kc & 15;
        *reinterpret_cast<u32x2*>(codes + (g * R + r) * 128 + d * 8) = q;
        if (d == 0) scl[g * R + r] = sc;
      }
    }
    __syncthreads();
    const int r = lane & 15;
    const bool live = r < R;
#pragma unroll
    for (int i = 0; i < SW; ++i) {
      if (s_lo + i >= s_hi) break;
      const int g = s_lo + i;
      v8i32 aop = {0, 0, 0, 0, 0, 0, 0, 0};
      if (live) {
        const u32x4* src = reinterpret_cast<const u32x4*>(codes + (g * R + r) * 128 + kb * 32);
        const u32x4 q0 = src[0], q1 = src[1];
        aop = v8i32{(int)q0[0], (int)q0[1], (int)q0[2], (int)q0[3], (int)q1[0], (int)q1[1], (int)q1[2], (int)q1[3]};
      }
      const v8i32 bop = {(int)bw[i][0][0], (int)bw[i][0][1], (int)bw[i][0][2], (int)bw[i][0][3],
                         (int)bw[i][1][0], (int)bw[i][1][1], (int)bw[i][1][2], (int)bw[i][1][3]};
      const v4f32 d = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aop, bop, v4f32{0.0f, 0.0f, 0.0f, 0.0f}, 0,
                                                                       0, 0, 127, 0, 127);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = 4 * kb + j;
        const float ts = row < R ? scl[g * R + row] * sw[i] : 0.0f;
        acc[0][j] = __builtin_fmaf(d[j], ts, acc[0][j]);
      }
    }
    __syncthreads();   // the partial sums below reuse the staging area
  } else {
    const u32x4* arow[MT];
    bool live[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const int m = m0 + 16 * t + (lane & 15);
      live[t] = m < G.M;
      arow[t] = reinterpret_cast<const u32x4*>(G.a + (int64_t)min(m, G.M - 1) * G.lda);
    }
    for (int s0 = s_lo; s0 < s_hi; s0 += SW) {
      u32x4 bw[SW][2];
      float sw[SW];
      u32x4 av[SW][MT][4];
#pragma unroll
      for (int i = 0; i < SW; ++i) {
        const bool in = s0 + i < s_hi;      // wave-uniform
        bw[i][0] = bw[i][1] = u32x4{0u, 0u, 0u, 0u};
        sw[i] = 0.0f;
        if (in) {
          bw[i][0] = wq[(s0 + i) * wstep];
          bw[i][1] = wq[(s0 + i) * wstep + whalf];
          sw[i] = wsrow[s0 + i];
        }
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            av[i][t][j] = u32x4{0u, 0u, 0u, 0u};
            if (in && live[t]) av[i][t][j] = arow[t][(s0 + i) * 16 + kb * 4 + j];   // 32 bf16
          }
      }
#pragma unroll
      for (int i = 0; i < SW; ++i) {
        if (s0 + i >= s_hi) break;
        const v8i32 bop = {(int)bw[i][0][0], (int)bw[i][0][1], (int)bw[i][0][2], (int)bw[i][0][3],
                           (int)bw[i][1][0], (int)bw[i][1][1], (int)bw[i][1][2], (int)bw[i][1][3]};
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          // the row's 128-group spans the four lanes l%16 + 16q
          uint32_t am = max(max(amax8(av[i][t][0]), amax8(av[i][t][1])), max(amax8(av[i][t][2]), amax8(av[i][t][3])));
          am = max(am, (uint32_t)__shfl_xor((int)am, 16));
          am = max(am, (uint32_t)__shfl_xor((int)am, 32));
          const float sc = fp8_scale(am);
          const v8i32 aop = fp8_codes32(av[i][t], sc);
          const v4f32 d = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aop, bop, v4f32{0.0f, 0.0f, 0.0f, 0.0f}, 0,
                                                                           0, 0, 127, 0, 127);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float ts = __shfl(sc, 4 * kb + j) * sw[i];
            acc[t][j] = __builtin_fmaf(d[j], ts, acc[t][j]);
          }
        }
      }
    }
  }

  v4f32* part = reinterpret_cast<v4f32*>(lds);
  if (wave > 0) {
#pragma unroll
    for (int t = 0; t < MT; ++t) part[((wave - 1) * MT + t) * 64 + lane] = acc[t];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    v4f32 c = acc[t];
    for (int w = 0; w < waves - 1; ++w) c += part[(w * MT + t) * 64 + lane];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m0 + 16 * t + 4 * (lane >> 4) + r;
      if (m < G.M) G.out[(int64_t)m * G.ldc + n] = c[r];
    }
  }
}

// Row-major e4m3fn weights to the preshuffled order: 16-byte unit
// u = ((t * steps + s) * 2 + h) * 64 + l of the output holds bytes
// 128 s + 32 (l/16) + 16 h .. +15 of row 16 t + l%16.
__global__ void __launch_bounds__(256) rmsq_fp8_preshuffle_kernel(const uint8_t* w, uint8_t* w_out, int32_t K,
                                                                  int64_t units) {
  const int64_t steps = K >> 7;
  for (int64_t u = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; u < units;
       u += (int64_t)gridDim.x * blockDim.x) {
    const int l = (int)(u & 63);
    const int64_t tsh = u >> 6, h = tsh & 1, ts = tsh >> 1, t = ts / steps, s = ts - t * steps;
    const int64_t row = t * 16 + (l & 15);
    reinterpret_cast<u32x4*>(w_out)[u] =
        reinterpret_cast<const u32x4*>(w + row * K)[s * 8 + (l >> 4) * 2 + h];
  }
}

}  // namespace rmsq
