// rmsq_gemm.h - block-scaled GEMMs for gfx950 around the group
// quantization: MXFP4 and FP8 weights times activations that are either bf16
// and quantized inside the GEMM ("prequant"), or already quantized by the
// group quantization (codes plus scales in one of its layouts).
//
// Sources, cited by title: [ATT] "[Triton] DS FP4/FP8 Triton fusion and GEMM
// optimization" lists an A16WFP4 GEMM that quantizes its activations inside
// the GEMM (with a preshuffled-weight GEMM beside it), used at concurrency 4
// (small M), where the norm is fused with the all-reduce and the group
// quantization moves into the GEMM; above concurrency 4 the fused RMSNorm +
// quant feeds a separate GEMM of the quantized activations
// (gemm_afp4wfp4_preshuffle, and block-scaled a8w8 GEMMs for FP8), whose
// activation scale layout the quantization must match ([ATF, Technical
// Details]).
//
// MXFP4 (rmsq_gemm_fp4_kernel):
// C[m, n] = sum_k qa[m, k] 2^(ea[m, k/32] - 127) * qw[n, k] 2^(ew[n, k/32] - 127)
// with (qa, ea) the MXFP4 group quantization (1x32 along K) of the bf16 row
// a[m, :] - the same rule and arithmetic as the fused kernel's MXFP4 path -
// or given, and (qw, ew) the weights. Products accumulate in fp32 on the
// matrix cores.
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
// bf16 activations: with at most 4 rows and one batch of steps per wave, a
// wave's 64 activation groups are one per lane: every lane loads and
// quantizes one (loads issued before the weight loads, so the two latencies
// overlap), and the operand lanes fetch the codes with ds_bpermute; no
// workgroup barrier precedes the matrix-core steps. Otherwise each wave loads
// and quantizes the 32-groups of its own operands. Quantized activations: each
// lane loads its group's scale byte, and the codes come either straight into
// the operand lanes (up to 4 rows) or 8 rows x 128 bytes per load and then
// across lanes (more rows; the kernel is bound by vector L1 accesses there).
// Lanes of rows past M read row M-1; their results are not stored. All loads of a
// batch are unconditional: a load under a branch would make the first use of
// any later load wait for it.
#pragma once

#include <algorithm>

#include "rmsq_device.h"

namespace rmsq {

typedef int v8i32 __attribute__((ext_vector_type(8)));
typedef float v4f32 __attribute__((ext_vector_type(4)));

struct GemmArgs {
  const uint16_t* a;      // bf16 [M, K], row stride lda elements (prequant)
  const uint8_t* aq;      // or e2m1 codes [M, K/2], dense rows (quantized activations)
  const uint8_t* as;      //    and their e8m0 scales in layout a_layout
  const uint8_t* w;       // e2m1 codes, row-major [N, K/2] or preshuffled
  const uint8_t* ws;      // e8m0 scales, row-major [N, K/32] or preshuffled
  float* out;             // fp32 [M, N], row stride ldc elements
  int64_t lda, ldc;
  int32_t M, N, K;
  int32_t a_layout;       // 0 row-major [M, G], 1 32-row tiles, 2 column-major [G, M]
};

constexpr int kGemmMaxWaves = 16;
constexpr int kGemmRowsPerBlock = 64;   // 4 tiles of 16 rows
constexpr int kGemmSmallRows = 4;      // at most this many rows take the small-M path
constexpr int kGemmSmallSteps = 4;     // steps per wave on the small-M path (one batch)

// Scale (row m, group g) of quantized activations with G groups per row and
// M rows, in the layouts the group quantization writes, sits at
// row_part + g * g_stride: row-major [M, G] (m G, 1), 32-row tiles with the
// tile's 32 rows adjacent per group ((m/32) 32 G + m%32, 32), column-major
// [G, M] (m, M).
struct ScaleWalk {
  int64_t row_part, g_stride;
};
__device__ __forceinline__ ScaleWalk act_scale_walk(int layout, int64_t m, int64_t G, int64_t M) {
  if (layout == 1) return ScaleWalk{(m >> 5) * 32 * G + (m & 31), 32};
  if (layout == 2) return ScaleWalk{m, M};
  return ScaleWalk{m * G, 1};
}

// Waves per workgroup with NT accumulator tiles per wave: at most 16, and
// their partial sums (1 KiB per tile and wave) within 64 KiB of LDS. The
// launch bound follows, so kernels with more tiles get more registers.
constexpr int gemm_max_waves(int NT) { return 64 / NT < kGemmMaxWaves ? 64 / NT : kGemmMaxWaves; }

// LDS bytes the kernel needs: the waves' partial sums, NT = MT * CT tiles of
// 16 x 16 fp32 per wave.
inline size_t gemm_lds_bytes(int MT, int CT, int waves) {
  return (size_t)waves * MT * CT * 64 * sizeof(v4f32);
}

// The epilogue of both GEMM kernels. Every wave writes its NT accumulator
// tiles (lane l: column l%16, rows 4(l/16) .. +3) to LDS; after the barrier
// each thread adds up one of the workgroup's NT * 256 outputs over the waves
// in wave order (fixed for a shape, so results repeat bit for bit) and
// stores it, 16 consecutive threads storing 16 consecutive columns of a row.
// The loads of all waves' partials are issued together (waves past the
// launch's count re-read the last one and add zero) instead of one LDS round
// trip per wave. Tile t covers columns col0 + 16 (t % CT) and rows
// m0 + 16 (t / CT).
template <int NT, int CT>
__device__ __forceinline__ void gemm_reduce_store(const v4f32 (&acc)[NT], uint8_t* lds, int wave, int waves, int lane,
                                                  int col0, int m0, float* out, int64_t ldc, int M) {
  v4f32* part = reinterpret_cast<v4f32*>(lds);
#pragma unroll
  for (int t = 0; t < NT; ++t) part[(wave * NT + t) * 64 + lane] = acc[t];
  __syncthreads();
  const float* pf = reinterpret_cast<const float*>(lds);
  constexpr int kOut = NT * 256;
  for (int e = threadIdx.x; e < kOut; e += blockDim.x) {
    const int c16 = e & 15, r = (e >> 4) & 3, q = (e >> 6) & 3, t = e >> 8;
    const int idx = (t * 64 + q * 16 + c16) * 4 + r;   // float of (tile t, lane 16q + c16, row r) in one wave's part
    float c = pf[idx];
#pragma unroll
    for (int w = 1; w < kGemmMaxWaves; ++w) {
      const float p = pf[min(w, waves - 1) * kOut + idx];
      c += w < waves ? p : 0.0f;
    }
    const int m = m0 + 16 * (t / CT) + 4 * q + r;
    if (m < M) out[(int64_t)m * ldc + col0 + 16 * (t % CT) + c16] = c;
  }
}

// MT row tiles of 16 rows and CT column tiles per workgroup (a wave reuses
// each activation operand for CT tiles), SW steps loaded per batch, SHUF:
// preshuffled weights, SMALLM: the small-M path of bf16 activations (MT ==
// 1, SW == kGemmSmallSteps, M <= kGemmSmallRows, every wave's steps in one
// batch). AQ: the activations arrive quantized (1: each operand loaded
// directly, 2: a pair of steps per load, redistributed; see below).
template <int MT, int SW, bool SHUF, bool SMALLM, int CT, int AQ>
__global__ void __launch_bounds__(64 * gemm_max_waves(MT * CT)) rmsq_gemm_fp4_kernel(const GemmArgs G) {
  static_assert(!(AQ && SMALLM), "the small-M path quantizes bf16 activations");
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

  if constexpr (SMALLM) {
    // Small M: the wave's batch of SW = 4 steps needs at most 4 rows x 16
    // activation groups of 32. Step i is one load of 4 rows x 256
    // consecutive bytes (lane L: row min(L/16, M-1), elements 8 (L%16) ..
    // +7 of the step), so each load reads whole cache lines; a lane quad then
    // holds one group (its amax by DPP), each lane encodes its 8 elements, and
    // the operand lane of row r, quarter kb fetches the 4 code dwords and the
    // scale byte from lanes 16 r + 4 kb + d (ds_bpermute). With each lane
    // reading 64 bytes of one group instead, every load touched four times
    // the cache lines. No workgroup barrier precedes the matrix-core steps.
    const int R = G.M;
    const u32x4* ap = reinterpret_cast<const u32x4*>(G.a + (int64_t)min(lane >> 4, R - 1) * G.lda) + (lane & 15);
    u32x4 av[SW];
#pragma unroll
    for (int i = 0; i < SW; ++i) av[i] = ap[min(s_lo + i, s_hi - 1) * 16];   // past the range: re-read (unused)
    __builtin_amdgcn_sched_barrier(0);
    u32x4 bw[CT][SW];
    uint32_t sb[CT][SW];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int i = 0; i < SW; ++i) {
        const int st = min(s_lo + i, s_hi - 1);   // steps past the range re-read the last (unused)
        bw[ct][i] = wq[ct * wq_tile + st * ws_step];
        sb[ct][i] = wsc[ct * ws_tile + st * ws_step];
      }
    __builtin_amdgcn_sched_barrier(0);
    const int r = lane & 15;
    const bool live = r < R;
    const int src = (16 * min(r, 3) + 4 * kb) << 2;   // ds_bpermute byte address of the group's first lane
#pragma unroll
    for (int i = 0; i < SW; ++i) {
      if (s_lo + i >= s_hi) break;
      const uint32_t byte = mx_scale_byte(max4(amax8(av[i])));
      const uint32_t code = fp4_codes8(av[i], byte);
      u32x4 q;
#pragma unroll
      for (int d = 0; d < 4; ++d) q[d] = (uint32_t)__builtin_amdgcn_ds_bpermute(src + (d << 2), (int)code);
      uint32_t sa = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)byte);
      if (!live) {
        q = u32x4{0u, 0u, 0u, 0u};
        sa = 127u;
      }
      const v8i32 aop = {(int)q[0], (int)q[1], (int)q[2], (int)q[3], 0, 0, 0, 0};
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const v8i32 bop = {(int)bw[ct][i][0], (int)bw[ct][i][1], (int)bw[ct][i][2], (int)bw[ct][i][3], 0, 0, 0, 0};
        acc[ct] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aop, bop, acc[ct], 4, 4, 0, (int)sa, 0,
                                                                   (int)sb[ct][i]);
      }
    }
  } else {
    // activation rows of this lane in each tile; lanes of rows past M read
    // row M-1 (their results are not stored)
    const uint8_t* asrow[MT];   // quantized activations: the row's scale bytes, group stride a_gs
    const u32x4* arowq[MT];     // quantized activations loaded directly: the operand lane's code row
    int crow[MT][2];            // quantized activations loaded by pairs: code rows 8j + lane/8 of the tile
    const uint16_t* ablk = AQ ? nullptr : G.a + (int64_t)m0 * G.lda;   // bf16 activations: the block's first row
    int64_t a_gs = 1;
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const int64_t m = min(m0 + 16 * t + (lane & 15), G.M - 1);
      if constexpr (AQ) {
        const ScaleWalk sw = act_scale_walk(G.a_layout, m, G.K >> 5, G.M);
        asrow[t] = G.as + sw.row_part;
        a_gs = sw.g_stride;
        arowq[t] = reinterpret_cast<const u32x4*>(G.aq + m * (G.K >> 1));
#pragma unroll
        for (int j = 0; j < 2; ++j) crow[t][j] = min(m0 + 16 * t + 8 * j + (lane >> 3), G.M - 1);
      } else {
        (void)m;   // bf16 rows: 4 rows x 256 bytes per load from ablk, addressed in the batch below
      }
    }
    // AQ == 2: quantized activation codes are loaded a pair of steps at a
    // time: each load covers 8 rows x 128 consecutive bytes (lane L: row
    // 8j + L/8, bytes 16 (L%8) .. +15 of the pair's run), one full cache line
    // per row, where loading an operand directly (AQ == 1) reads 16 rows x 64
    // bytes (16 half lines); the operand lanes then fetch their 16 bytes with
    // ds_bpermute. From a few rows on the kernel is bound by vector L1
    // accesses, and this halves the accesses for the codes; with one to four
    // rows the direct loads hit the same lines anyway and skip the exchange.
    // The pair's run starts at step pb (clamped so the run stays inside the
    // row; dead steps read anything in it).
    static_assert(AQ != 2 || SW % 2 == 0, "quantized activations load pairs of steps");
    constexpr int AV = AQ ? 2 : 4;   // AQ 2: the pair's two loads (at step 2p); AQ 1: one; else 32 bf16
    const int kq = G.K >> 5;          // 16-byte units of codes per row
    for (int s0 = s_lo; s0 < s_hi; s0 += SW) {
      u32x4 bw[SW][CT];
      uint32_t sb[SW][CT];
      u32x4 av[SW][MT][AV];
      uint32_t sab[SW][MT];
      int pb[SW];
      // every load of the batch unconditionally (steps past the range re-read
      // the last one and are not used), so no use waits on a partial batch
#pragma unroll
      for (int i = 0; i < SW; ++i) {
        const int st = min(s0 + i, s_hi - 1);   // wave-uniform
        const int kg = st * 4 + kb;             // 32-element group index along K
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          bw[i][ct] = wq[ct * wq_tile + st * ws_step];
          sb[i][ct] = wsc[ct * ws_tile + st * ws_step];
        }
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          if constexpr (AQ == 1) {
            av[i][t][0] = arowq[t][kg];          // 16 bytes = 32 e2m1 codes
            sab[i][t] = asrow[t][kg * a_gs];
          } else if constexpr (AQ == 2) {
            if (i % 2 == 0) {
              pb[i] = max(0, min(s0 + i, steps - 2));   // wave-uniform
#pragma unroll
              for (int j = 0; j < 2; ++j)
                av[i][t][j] = reinterpret_cast<const u32x4*>(G.aq)[(int64_t)crow[t][j] * kq +
                                                                   min(pb[i] * 4 + (lane & 7), kq - 1)];
            }
            sab[i][t] = asrow[t][kg * a_gs];
          } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              // 32-bit offsets from the row block's first row (at most 64 rows,
              // lda <= 2^25), so each address is one register beside a scalar base
              const uint32_t row = (uint32_t)(min(m0 + 16 * t + 4 * j + (lane >> 4), G.M - 1) - m0);
              const uint32_t off = row * (uint32_t)G.lda + (uint32_t)(st * 128 + (lane & 15) * 8);
              av[i][t][j] = *reinterpret_cast<const u32x4*>(ablk + off);
            }
          }
        }
      }
      // the whole batch is in flight before any use (otherwise the scheduler
      // trades it for registers, waiting for one step's data before the next
      // step's loads)
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < SW; ++i) {
        // A step past the wave's range (its loads re-read the last one) adds
        // zero products instead of being skipped: with no branch here, the
        // compiler cannot sink a later step's loads below an earlier step's use.
        const bool live = s0 + i < s_hi;   // wave-uniform
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          u32x4 q;
          uint32_t sa;
          if constexpr (AQ == 1) {
            q = av[i][t][0];
            sa = sab[i][t];
          } else if constexpr (AQ == 2) {
            // this step's 16 bytes for row r = lane%16, quarter kb: lane
            // 8 (r%8) + 4 o + kb of the pair's load r/8, o the step's place in the run
            const int i0 = i & ~1;
            const int o = min(s0 + i - pb[i0], 1);
            const int src = (((lane & 7) << 3) + o * 4 + kb) << 2;
#pragma unroll
            for (int d = 0; d < 4; ++d) {
              const int lo = __builtin_amdgcn_ds_bpermute(src, (int)av[i0][t][0][d]);
              const int hi = __builtin_amdgcn_ds_bpermute(src, (int)av[i0][t][1][d]);
              q[d] = (uint32_t)((lane & 8) ? hi : lo);
            }
            sa = sab[i][t];
          } else {
            // Each lane quantizes its 8 elements of each load (the lane quad
            // of a 32-group shares the amax by DPP), then the operand lane of
            // row r, quarter kb fetches its 4 code dwords and scale byte
            // from lanes 16 (r%4) + 4 kb + d of load r/4.
            uint32_t code[4], byte[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              byte[j] = mx_scale_byte(max4(amax8(av[i][t][j])));
              code[j] = fp4_codes8(av[i][t][j], byte[j]);
            }
            const int src = (((lane & 3) << 4) + (kb << 2)) << 2;
            const int jr = (lane >> 2) & 3;   // load of this operand lane's row
#pragma unroll
            for (int d = 0; d < 4; ++d) {
              int v = 0;
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const int x = __builtin_amdgcn_ds_bpermute(src + (d << 2), (int)code[j]);
                v = jr == j ? x : v;
              }
              q[d] = (uint32_t)v;
            }
            sa = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int x = __builtin_amdgcn_ds_bpermute(src, (int)byte[j]);
              sa = jr == j ? (uint32_t)x : sa;
            }
            // one tile at a time: interleaving the tiles' exchanges needs more registers than 16 waves leave
            __builtin_amdgcn_sched_barrier(0);
          }
          if (!live) q = u32x4{0u, 0u, 0u, 0u};
          const v8i32 aop = {(int)q[0], (int)q[1], (int)q[2], (int)q[3], 0, 0, 0, 0};
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) {
            const v8i32 bop = {(int)bw[i][ct][0], (int)bw[i][ct][1], (int)bw[i][ct][2], (int)bw[i][ct][3], 0, 0, 0, 0};
            acc[t * CT + ct] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aop, bop, acc[t * CT + ct], 4, 4, 0,
                                                                               (int)sa, 0, (int)sb[i][ct]);
          }
        }
      }
    }
  }

  gemm_reduce_store<MT * CT, CT>(acc, lds, wave, waves, lane, tile * 16, m0, G.out, G.ldc, G.M);
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

// -------------------------------------------------------------------- FP8 --
// The FP8 counterpart (rmsq_gemm_fp8_kernel; [ATT] lists an a16w8 GEMM and
// block-scaled a8w8 GEMMs for its DS FP8 runs): activations quantized per
// 1x128 group along K to e4m3fn with fp32 scales - inside the GEMM from bf16
// by the fused kernel's FP8 rule (s = amax/448, exact codes), or given with
// their scales row- or column-major - and e4m3fn weights [N, K] with fp32
// scales per 128x128 block [ceil(N/128), K/128]:
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
  const uint16_t* a;      // bf16 [M, K], row stride lda elements (prequant)
  const uint8_t* aq;      // or e4m3fn codes [M, K], dense rows (quantized activations)
  const float* as;        //    and their fp32 scales in layout a_layout
  const uint8_t* w;       // e4m3fn codes, row-major [N, K] or preshuffled
  const float* ws;        // fp32 block scales [ceil(N/128), K/128]
  float* out;             // fp32 [M, N], row stride ldc elements
  int64_t lda, ldc;
  int32_t M, N, K;
  int32_t a_layout;       // 0 row-major [M, K/128], 2 column-major [K/128, M]
};

// LDS bytes of the FP8 kernel: the waves' partial sums.
inline size_t gemm8_lds_bytes(int MT, int waves) {
  return (size_t)waves * MT * 64 * sizeof(v4f32);
}

__device__ __forceinline__ void unpack_bf16x8(const u32x4 w, float f[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_lo(w[i]);
    f[2 * i + 1] = bf16_hi(w[i]);
  }
}

// e4m3fn codes of 32 bf16 values (16 dwords) of a group with maximum
// magnitude amax (bf16 bits) and scale sc = fp8_scale(amax): 8 dwords,
// element order.
__device__ __forceinline__ v8i32 fp8_codes32(const u32x4 v[4], float sc, uint32_t amax) {
  v8i32 q;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float f[8];
    unpack_bf16x8(v[i], f);
    const u32x2 c = fp8_codes8(f, sc, __uint_as_float(amax << 16));
    q[2 * i] = (int)c[0];
    q[2 * i + 1] = (int)c[1];
  }
  return q;
}

// MT row tiles per workgroup, SW steps per batch, SHUF: preshuffled weights,
// SMALLM: the small-M path of bf16 activations (MT == 1, SW ==
// kGemmSmallSteps, M <= kGemmSmallRows, one batch per wave), AQ: the
// activations arrive quantized (1: each operand loaded directly, 2: 8 rows x
// 128 bytes per load, redistributed, as in the FP4 kernel).
// Row blocks are 16 * MT rows (MT <= kGemm8MaxTiles: the activation
// registers of more tiles would not fit beside the 32-byte operands).
constexpr int kGemm8MaxTiles = 2;

template <int MT, int SW, bool SHUF, bool SMALLM, int AQ>
__global__ void __launch_bounds__(64 * kGemmMaxWaves) rmsq_gemm_fp8_kernel(const Gemm8Args G) {
  static_assert(MT <= kGemm8MaxTiles, "at most two row tiles");
  static_assert(!(AQ && SMALLM), "the small-M path quantizes bf16 activations");
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

  if constexpr (SMALLM) {
    // Small M: the wave's batch of SW = 4 steps needs at most 4 rows x 4
    // groups of 128. Step i is one load of 4 rows x 256 consecutive bytes
    // (lane L: row min(L/16, M-1), elements 8 (L%16) .. +7 of the step), so
    // each 16-lane DPP row holds one group (amax by DPP) and each lane
    // encodes its 8 elements; the operand lane of row r, quarter kb fetches
    // its 8 code dwords from lanes 16 r + 4 kb + d, and each result lane the
    // scales of its four rows (ds_bpermute). No workgroup barrier precedes
    // the matrix-core steps.
    const int R = G.M;
    const u32x4* ap = reinterpret_cast<const u32x4*>(G.a + (int64_t)min(lane >> 4, R - 1) * G.lda) + (lane & 15);
    u32x4 av[SW];
#pragma unroll
    for (int i = 0; i < SW; ++i) av[i] = ap[min(s_lo + i, s_hi - 1) * 16];   // past the range: re-read (unused)
    __builtin_amdgcn_sched_barrier(0);
    u32x4 bw[SW][2];
    float sw[SW];
#pragma unroll
    for (int i = 0; i < SW; ++i) {
      const int st = min(s_lo + i, s_hi - 1);   // steps past the range re-read the last (unused)
      bw[i][0] = wq[st * wstep];
      bw[i][1] = wq[st * wstep + whalf];
      sw[i] = wsrow[st];
    }
    __builtin_amdgcn_sched_barrier(0);
    const int r = lane & 15;
    const bool live = r < R;
    const int src = (16 * min(r, 3) + 4 * kb) << 2;   // ds_bpermute byte address of the quarter's first lane
#pragma unroll
    for (int i = 0; i < SW; ++i) {
      if (s_lo + i >= s_hi) break;
      const uint32_t am = max16(amax8(av[i]));
      const float sc = fp8_scale(am);
      float f[8];
      unpack_bf16x8(av[i], f);
      const u32x2 c = fp8_codes8(f, sc, __uint_as_float(am << 16));
      v8i32 aop;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        aop[2 * d] = __builtin_amdgcn_ds_bpermute(src + (d << 2), (int)c[0]);
        aop[2 * d + 1] = __builtin_amdgcn_ds_bpermute(src + (d << 2), (int)c[1]);
      }
      if (!live) aop = v8i32{0, 0, 0, 0, 0, 0, 0, 0};
      const v8i32 bop = {(int)bw[i][0][0], (int)bw[i][0][1], (int)bw[i][0][2], (int)bw[i][0][3],
                         (int)bw[i][1][0], (int)bw[i][1][1], (int)bw[i][1][2], (int)bw[i][1][3]};
      const v4f32 d = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aop, bop, v4f32{0.0f, 0.0f, 0.0f, 0.0f}, 0,
                                                                       0, 0, 127, 0, 127);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // result row 4 kb + j: its scale sits in every lane 16 (4 kb + j) + x (rows past 3 give 0)
        const int row = 4 * kb + j;
        const float sa = __uint_as_float((uint32_t)__builtin_amdgcn_ds_bpermute((16 * min(row, 3)) << 2,
                                                                               (int)__float_as_uint(sc)));
        const float ts = row < R ? sa * sw[i] : 0.0f;
        acc[0][j] = __builtin_fmaf(d[j], ts, acc[0][j]);
      }
    }
  } else {
    // lanes of rows past M read row M-1 (their results are not stored)
    const u32x4* arow[MT];
    const float* asrow[MT];   // quantized activations: the row's scales, block stride a_gs
    int crow[MT][2];          // AQ == 2: code rows 8j + lane/8 of the tile
    int64_t a_gs = 1;
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const int64_t m = min(m0 + 16 * t + (lane & 15), G.M - 1);
      if constexpr (AQ != 0) {
#pragma unroll
        for (int j = 0; j < 2; ++j) crow[t][j] = min(m0 + 16 * t + 8 * j + (lane >> 3), G.M - 1);
        arow[t] = reinterpret_cast<const u32x4*>(G.aq + m * G.K);
        const ScaleWalk sw = act_scale_walk(G.a_layout, m, G.K >> 7, G.M);
        asrow[t] = G.as + sw.row_part;
        a_gs = sw.g_stride;
      } else {
        arow[t] = reinterpret_cast<const u32x4*>(G.a + m * G.lda);
      }
    }
    constexpr int AV = AQ ? 2 : 4;   // 16-byte loads per operand: 32 codes, or 32 bf16
    for (int s0 = s_lo; s0 < s_hi; s0 += SW) {
      u32x4 bw[SW][2];
      float sw[SW];
      u32x4 av[SW][MT][AV];
      float sav[SW][MT];
      // unconditional loads, as in the FP4 kernel
#pragma unroll
      for (int i = 0; i < SW; ++i) {
        const int st = min(s0 + i, s_hi - 1);   // wave-uniform
        bw[i][0] = wq[st * wstep];
        bw[i][1] = wq[st * wstep + whalf];
        sw[i] = wsrow[st];
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          if constexpr (AQ == 1) {
            av[i][t][0] = arow[t][st * 8 + kb * 2];       // 32 e4m3fn codes
            av[i][t][1] = arow[t][st * 8 + kb * 2 + 1];
            sav[i][t] = asrow[t][st * a_gs];
          } else if constexpr (AQ == 2) {
            // the step's 128 code bytes of rows 8j + lane/8: lane L holds bytes 16 (L%8) .. +15
#pragma unroll
            for (int j = 0; j < 2; ++j)
              av[i][t][j] = reinterpret_cast<const u32x4*>(G.aq)[(int64_t)crow[t][j] * (G.K >> 4) + st * 8 + (lane & 7)];
            sav[i][t] = asrow[t][st * a_gs];
          } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) av[i][t][j] = arow[t][st * 16 + kb * 4 + j];   // 32 bf16
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);   // the whole batch in flight first, as in the FP4 kernel
#pragma unroll
      for (int i = 0; i < SW; ++i) {
        const bool live = s0 + i < s_hi;   // a dead step adds zero products, as in the FP4 kernel
        const v8i32 bop = {(int)bw[i][0][0], (int)bw[i][0][1], (int)bw[i][0][2], (int)bw[i][0][3],
                           (int)bw[i][1][0], (int)bw[i][1][1], (int)bw[i][1][2], (int)bw[i][1][3]};
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          float sc;
          v8i32 aop;
          if constexpr (AQ == 1) {
            sc = sav[i][t];
            aop = v8i32{(int)av[i][t][0][0], (int)av[i][t][0][1], (int)av[i][t][0][2], (int)av[i][t][0][3],
                        (int)av[i][t][1][0], (int)av[i][t][1][1], (int)av[i][t][1][2], (int)av[i][t][1][3]};
          } else if constexpr (AQ == 2) {
            // bytes 32 kb .. +31 of row r = lane%16: lanes 8 (r%8) + 2 kb and + 1 of load r/8
            sc = sav[i][t];
            const int src = (((lane & 7) << 3) + 2 * kb) << 2;
#pragma unroll
            for (int d = 0; d < 8; ++d) {
              const int a = src + ((d >> 2) << 2);
              const int lo = __builtin_amdgcn_ds_bpermute(a, (int)av[i][t][0][d & 3]);
              const int hi = __builtin_amdgcn_ds_bpermute(a, (int)av[i][t][1][d & 3]);
              aop[d] = (lane & 8) ? hi : lo;
            }
          } else {
            // the row's 128-group spans the four lanes l%16 + 16q
            uint32_t am = max(max(amax8(av[i][t][0]), amax8(av[i][t][1])), max(amax8(av[i][t][2]), amax8(av[i][t][3])));
            am = max(am, (uint32_t)__shfl_xor((int)am, 16));
            am = max(am, (uint32_t)__shfl_xor((int)am, 32));
            sc = fp8_scale(am);
            aop = fp8_codes32(av[i][t], sc, am);
          }
          if (!live) aop = v8i32{0, 0, 0, 0, 0, 0, 0, 0};
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

  gemm_reduce_store<MT, 1>(acc, lds, wave, waves, lane, tile * 16, m0, G.out, G.ldc, G.M);
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
