// rmsq_kernel.h - the fused residual-add + RMSNorm + per-group quantization
// kernel for gfx950.
//
// Sources, cited by title:
//   [FRQ] "fused rmsnorm quant fp8 work"
//   [ARQ] "[AMD] Add fused all-reduce RMSNorm per-group quant for Qwen3.5 FP8"
//   [ATF] "[Feat] Support input_rmsnorm_quant & qknorm_quant fused for Atom
//          dpsk v2 model"
//   [ATT] "[Triton] DS FP4/FP8 Triton fusion and GEMM optimization"
//
// Mapping. One workgroup per token row, 64*W threads (W waves, runtime),
// each lane owning J chunks of 8 bf16 (16 bytes): chunk c = j*64*W + lane.
// Short rows are packed instead, several waves per workgroup: one row per
// wave (chunk c = j*64 + lane), or rows of at most 32 chunks one per group of
// 16 or 32 lanes (one chunk per lane).
// All of a row's loads are issued before any arithmetic; the row then stays
// in registers across the one reduction, and every output is stored once.
// Loads and stores are 16-byte and coalesced across the wave. A 128-element
// FP8 group is 16 consecutive chunks, i.e. one 16-lane DPP row, so its amax
// is four DPP row rotations; a 32-element MXFP4 group is one lane quad.
//
// Numerics (results equal the double-precision definition bit for bit):
//  * h = bf16(x + r): the fp32 sum rounds to the same bf16 as the exact sum.
//  * sum of h^2 in fp64 (each square exact), DPP tree within the wave, then
//    the waves' partial sums in a fixed pairwise tree through LDS,
//    inv = 1/sqrt(ss/N + eps) in fp64 with correctly rounded divide / sqrt;
//    fl32(inv) comes from a Newton-refined reciprocal square root that is
//    close enough to decide it, and inv itself is formed only where an
//    element is redone in fp64.
//  * y = (h*g) * inv: h*g is exact in fp32 while it stays in the normal
//    range; the product is first taken in fp32 with fl32(inv), whose error
//    against the fp64 product lies within half an ulp on one side and 1.5 on
//    the other (the side of inv - fl32(inv)); only when its low half is the
//    bf16 rounding midpoint or that side's neighbour of it (two values per
//    row), or h*g is denormal or infinite, is the element redone: a midpoint
//    case is decided in fp32 from the sign of y - midpoint corrected by the
//    product's exact residual and inv's low part, and ties, near ties and the
//    rest are redone as fp64 h*g*inv rounded once to bf16.
//  * FP8 scale s = fl32(amax/448), correctly rounded; codes through the
//    hardware convert of yb * r, with r the reciprocal of s rounded up or
//    down: the sign of fma(s, 448, -amax) says on which side of every
//    rounding midpoint yb/s lies (for bf16 yb and amax, 448 yb / amax is a
//    midpoint exactly or far from one), so one bracket gives the codes of
//    yb/s; a group whose scale is exact takes the even code of the two
//    brackets, and groups with a tiny scale round the double quotient.
//  * MXFP4 scale byte from the bf16 exponent of amax; codes through the
//    hardware scaled convert straight from the packed bf16 (exact division
//    by 2^e, then e2m1 rounding).
#pragma once

#include "rmsq_device.h"

namespace rmsq {

struct Problem {
  // what the loads need, first (one 48-byte run)
  const uint16_t* x;
  const uint16_t* gamma;
  const uint16_t* r;      // residual in, or null
  int64_t ldx, ldr;       // row strides in elements
  int32_t N, M;
  // the rest
  uint16_t* h;            // residual out (null exactly when r is null)
  uint8_t* q;
  void* scale;
  uint16_t* yb;           // bf16 side-output, or null
  int64_t ldb;
  int32_t layout;         // scale layout: 0 row-major, 1 32-row tiles (MXFP4), 2 column-major
  float eps;
  double rn;              // 1/N rounded to nearest (host division)
  int32_t lanes_log2;     // rows packed by lanes: 2^k lanes per row (k = 4, 5 or 6)
};

constexpr int kMaxProblems = 4;
constexpr int kMaxWaves = 16;
// Long per-lane rows (J >= 7 chunks) keep up to ~120 VGPRs of row data live;
// they are launched with at most 4 waves per row so the register budget is
// not cut to 128 by a 1024-thread bound.
constexpr int max_waves(int J) { return J >= 7 ? 4 : kMaxWaves; }
// Launch description. The scalars are also passed as the kernel's leading
// int arguments, which the library is built to have preloaded into SGPRs at
// wave launch (gfx950 kernel-argument preloading), so only the selected
// problem's fields are read from the argument block.
struct Launch {
  int32_t count;
  int32_t rows;           // launch units over all problems: rows, or waves with packed rows
  int32_t row_group_log2; // 2^k consecutive rows (packed: workgroups) kept together on one
                          // XCD (0 = dispatch order)
  int32_t splits_log2;    // 2^k workgroups per row: each computes the row's statistics
                          // and normalizes / quantizes its own share of the row
  int32_t row_begin[kMaxProblems];  // first launch unit of each problem (increasing)
  Problem p[kMaxProblems];
};

// Rows packed by lanes: problem p fills the launch waves from row_begin[p]
// on, 2^(6-lt) rows per wave with lt = its lanes_log2. Lane l of the
// problem's wave u works on row (u << (6 - lt)) + (l >> lt), as lane
// l & (2^lt - 1) of that row.
__device__ __forceinline__ int32_t packed_row(int32_t u, int lt, int lane) { return (u << (6 - lt)) + (lane >> lt); }

// Workgroups are dispatched round-robin over the 8 XCDs, each with its own
// L2. With g = 2^lg > 1, every run of g consecutive rows is processed on one
// XCD (rows of 8*g consecutive workgroups are interleaved at g-row
// granularity), so scale bytes of neighbouring rows that share a cache line -
// a 224-byte scale row, or the 32 rows of a tiled MXFP4 scale block - are
// written from a single L2 instead of being merged from several. The mapping
// is a bijection on each block of 8*g rows; a ragged tail keeps dispatch order.
__device__ __forceinline__ int32_t row_of_block(int32_t b, int32_t rows, int32_t lg) {
  const int32_t x = b & 7, k = b >> 3;
  const int32_t mapped = ((((k >> lg) << 3) + x) << lg) + (k & ((1 << lg) - 1));
  // a select, not a branch: the launch scalars are then all needed up front
  return ((lg == 0) | (b >= (rows >> (lg + 3)) << (lg + 3))) ? b : mapped;
}

// RES: every problem of the launch has a residual (otherwise none has), so
// the loads of x, r and gamma form one straight block with no branch.
// PACK: how rows map to lanes.
//   kPackNone   the workgroup's waves share one row (LDS for the reduction);
//   kPackWave   rows short enough for one wave (J*64 chunks) are packed one
//               per wave, blockDim/64 consecutive rows per workgroup, with no
//               LDS and no barrier;
//   kPackLanes  (J = 1) likewise, but one row per group of T = 16, 32 or 64
//               lanes, per problem: rows of 128 or 256 elements fill a wave
//               4 or 2 at a time instead of leaving 48 or 32 lanes idle (the
//               row index is then per lane, which costs the one-per-wave
//               layout a few percent, so it stays separate).
// TAIL: how the rows of the launch end (T lanes per row, no row splits
// except with kRagged):
//   kExact    every row has exactly J*T chunks and every lane group of a
//             packed launch has a row, so no lane needs a bound (the usual
//             shapes: 7168 = 2 x 7 waves or 1 x 14, 1536 = 3 x 1, 512 = 1 x 1);
//   kUniform  every row has a whole number of chunk steps (a multiple of T
//             chunks, at most J*T) and every lane group has a row: steps past
//             a row's end are skipped by the whole wave, with a scalar test,
//             and their loads read zeros through the row's buffer resources
//             without touching memory (rows packed one per wave only: the MLA
//             latents, 1536 and 512 wide, in one launch);
//   kRagged   anything else: lanes past the row end clamp their chunk index
//             (read zeros, packed one per wave), and lane groups past a
//             problem's last row reload that row and store nothing.
enum Tail { kRagged = 0, kExact = 1, kUniform = 2 };
enum Pack { kPackNone = 0, kPackWave = 1, kPackLanes = 2 };

// Packed rows of 3 chunks per lane (the 1536-wide MLA latent rows), and of 4
// when quantized without a residual and bounded (the MLA latents in 4-chunk
// steps), are launched 8 waves per workgroup; held to
// 64 VGPRs, 8 waves fit on each SIMD, so four such workgroups per compute
// unit and a 4096 + 4096-row launch is resident at once (at 72 VGPRs only
// three fit and a third of the grid waits for a second round). The other
// 4-chunk variants do not fit that budget without spilling.
constexpr int min_waves_per_simd(int FMT, int J, bool packed, bool res, int tail) {
  return packed && (J == 3 || (J == 4 && !res && FMT != 2 && tail != kExact)) ? 8 : 1;
}

template <int FMT, int J, bool RES, int PACK, int TAIL>
__global__ void __launch_bounds__(64 * max_waves(J), min_waves_per_simd(FMT, J, PACK != kPackNone, RES, TAIL))
rmsq_fused_kernel(int32_t count, int32_t rows, int32_t lg, int32_t slg, int32_t rb1, int32_t rb2, int32_t rb3,
                  int32_t threads, int32_t blocks, const Launch L) {
  // the ints repeat L's scalars (count, rows, row_group_log2, splits_log2,
  // row_begin[1..3]) and the launch's blockDim.x and gridDim.x
  // Short per-lane rows (the usual shapes) keep h as fp32 and fetch gamma
  // together with x and r; long ones keep h packed and fetch gamma late, to
  // stay within the register budget.
  constexpr bool kShort = J <= 4;
  constexpr bool kPacked = PACK != kPackNone;
  static_assert(PACK != kPackLanes || J == 1, "rows packed by lanes take one chunk per lane");
  // Packed rows of 3 or 4 chunks per lane (held to 64 VGPRs) unpack h again
  // in phase 2 rather than keep 24 or 32 fp32 copies across the reduction.
  constexpr bool kKeepH = kShort && !(kPacked && J >= 3);
  // The fp64 path decides midpoint-window elements in fp32 first where its
  // latency bounds the launch: one chunk per lane (decode, short prefills,
  // rows packed by lanes) and rows packed one per wave up to 3 chunks (the
  // MLA latents), except 3 chunks with exact tails (held to 64 VGPRs, where
  // the larger block spills). Rows over several waves with more chunks are
  // bandwidth-bound; there the larger block cost the prefill batch 3% (it
  // moves the memory-bound code around the branch) and gains nothing.
  constexpr bool kSplitExact = J == 1 || (kPacked && J <= 3 && !(J == 3 && TAIL == kExact));
  __shared__ double red[kMaxWaves];

  // Neighbouring row groups run on different XCDs at the same time. (Giving
  // each XCD one contiguous block of M/8 rows instead was measured 12%
  // slower on the prefill workload.)
  int32_t row, split = 0;   // the launch unit: a row, or with packed rows a wave
  if constexpr (kPacked) {
    const int32_t wave = __builtin_amdgcn_readfirstlane((int32_t)(threadIdx.x >> 6));
    row = row_of_block((int32_t)blockIdx.x, blocks, lg) * (threads >> 6) + wave;
    if (row >= rows) return;   // the whole wave leaves: nothing below synchronizes
  } else {
    // Row splits (slg > 0): blocks in runs of 8 rows x 2^slg splits, block =
    // (row / 8) * 8 * 2^slg + split * 8 + row % 8, so a row's splits share an
    // XCD (block % 8) and its L2 serves their repeated reads of the row. Rows
    // are padded to a multiple of 8; padding blocks leave at once. Without
    // splits the host may group rows per XCD (lg > 0); the two are exclusive.
    const int32_t b = (int32_t)blockIdx.x;
    split = slg > 0 ? (b >> 3) & ((1 << slg) - 1) : 0;
    row = slg > 0 ? ((b >> (3 + slg)) << 3) | (b & 7) : row_of_block(b, rows, lg);
    if (row >= rows) return;   // the whole workgroup leaves before any barrier
  }
  // problems are consecutive ranges of launch units (row_begin increasing)
  const int pi = (count > 1 && row >= rb1) + (count > 2 && row >= rb2) + (count > 3 && row >= rb3);
  const Problem& P = L.p[pi];
  // The record's fields that the loads need, read together before anything
  // branches on them: one scalar round trip. (The row-split bounds below use
  // N; read where first used, the compiler fetched N alone, waited, and only
  // then fetched the pointers and strides - a second round trip on the
  // critical path of the short launches.)
  const uint16_t* const px = P.x;
  const uint16_t* const pg = P.gamma;
  const uint16_t* const pr = RES ? P.r : nullptr;
  const int64_t ldx = P.ldx, ldr = RES ? P.ldr : 0;
  const int32_t N = P.N, M = P.M;
  asm volatile("" ::"s"(px), "s"(pg), "s"(pr), "s"(ldx), "s"(ldr), "s"(N), "s"(M));
  const int32_t u = row - (pi == 0 ? 0 : pi == 1 ? rb1 : pi == 2 ? rb2 : rb3);
  const int lt = PACK == kPackLanes ? P.lanes_log2 : 6;
  const int T = PACK == kPackLanes ? 1 << lt : kPacked ? 64 : threads;
  const int tid = kPacked ? (int)(threadIdx.x & (T - 1)) : (int)threadIdx.x;
  int64_t m = u;
  bool live = true;   // packed by lanes: this lane group has a row of the problem
  if constexpr (PACK == kPackLanes) {
    const int32_t r = packed_row(u, lt, threadIdx.x & 63);
    live = r < M;
    m = live ? r : M - 1;
  }
  const int C = N >> 3;
  // What a lane loads at step j: the row's chunk j*T + tid, clamped to the
  // row's last step (kUniform: a wave-uniform offset, so the lane offset tid
  // is shared by every step) or to its last chunk (kRagged). Rows packed one
  // per wave read through buffer resources over the row instead: a chunk
  // past the row's end (a whole step of a shorter row in a kUniform launch,
  // the tail lanes of a ragged one) then reads zeros and touches no memory,
  // where the clamped form re-read a kilobyte per step from the caches, and
  // the loads take the row as a scalar base with one shared lane offset.
  // Rows over several waves keep plain indexing, which measured 0.15% faster
  // on the bandwidth-bound shapes than a scalar-base form.
  const int jl = TAIL == kUniform ? C / T - 1 : 0;
  auto at = [&](const u32x4* row, int j) {
    if constexpr (TAIL == kUniform) return row + min(j, jl) * T + tid;
    return row + (TAIL == kExact ? j * T + tid : min(j * T + tid, C - 1));
  };
  auto load = [&](const u32x4* row, int j) { return *at(row, j); };
  auto load_nt = [&](const u32x4* row, int j) { return __builtin_nontemporal_load(at(row, j)); };
  // (each step has its own resource, starting at the step and ending at the
  // row's end, so that the range check rests on the lane offset alone)
  auto load_buf = [&](const void* row, int j, auto policy) {
    const int done = j * T * 16;
    const __amdgpu_buffer_rsrc_t rs =
        buffer_rsrc(reinterpret_cast<const char*>(row) + done, C * 16 > done ? C * 16 - done : 0);
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, tid * 16, 0, decltype(policy)::value));
  };
  // ---- loads: x, gamma (short rows), then r, all issued before any use ---
  // (of the issue orders measured, this one was fastest on both the
  // bandwidth-bound and the latency-bound shapes)
  // A ragged row clamps its chunk index instead of guarding the loads: lanes
  // past the row end re-read the last chunk (the address of a live lane of
  // the same instruction, so no extra traffic; rows packed one per wave read
  // zeros there instead) and their h is zeroed before the sum of squares;
  // their stores are skipped.
  const u32x4* xrow = reinterpret_cast<const u32x4*>(px + m * ldx);
  const u32x4* rrow = RES ? reinterpret_cast<const u32x4*>(pr + m * ldr) : nullptr;
  const u32x4* grow = reinterpret_cast<const u32x4*>(pg);
  u32x4 xv[J], rv[RES ? J : 1], gv[kShort ? J : 1];
  if constexpr (PACK == kPackWave) {
#pragma unroll
    for (int j = 0; j < J; ++j) xv[j] = load_buf(xrow, j, std::integral_constant<int, kBufNontemporal>{});
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < J; ++j) gv[j] = load_buf(grow, j, std::integral_constant<int, 0>{});
  } else {
#pragma unroll
    for (int j = 0; j < J; ++j) xv[j] = load_nt(xrow, j);
    if constexpr (kShort) {
#pragma unroll
      for (int j = 0; j < J; ++j) gv[j] = load(grow, j);
    }
  }
  // keep the loads in this order: the scheduler may otherwise interleave
  // gamma's or r's with x's, or hoist x's unpacking (and the wait for x)
  // above them
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (RES) {
    if constexpr (PACK == kPackWave) {
#pragma unroll
      for (int j = 0; j < J; ++j) rv[j] = load_buf(rrow, j, std::integral_constant<int, kBufNontemporal>{});
    } else {
#pragma unroll
      for (int j = 0; j < J; ++j) rv[j] = load_nt(rrow, j);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  // chunks this workgroup normalizes and stores: all of them, or with row
  // splits a range whose ends fall on group boundaries (16 chunks FP8, 4 MXFP4)
  int lo = 0, hi = live ? C : 0;
  if (!kPacked && slg > 0) {
    constexpr int q = FMT == 0 ? 16 : FMT == 1 ? 4 : 1;
    lo = ((split * (C / q)) >> slg) * q;
    hi = split + 1 == (1 << slg) ? C : (((split + 1) * (C / q)) >> slg) * q;
  }

  // Every other field of the problem record this row needs, read now: their
  // scalar loads then overlap the row's vector loads instead of stalling the
  // statistics and the stores later (each late scalar load costs a memory
  // round trip on the row's critical path, which is what bounds the short
  // launches).
  const float eps = P.eps;
  const double rn = P.rn;
  const int32_t layout = P.layout;
  uint16_t* const hbase = RES ? P.h : nullptr;
  uint16_t* const ybase = P.yb;
  uint8_t* const qbase = FMT == 2 ? nullptr : P.q;
  void* const sbase = FMT == 2 ? nullptr : P.scale;
  const int64_t ldb = P.ldb;
  asm volatile("" ::"s"(eps), "s"(rn), "s"(layout), "s"(M), "s"(hbase), "s"(ybase), "s"(qbase), "s"(sbase), "s"(ldb));

  // ---- phase 1: h = x + r (stored after the reduction, with the other outputs)
  if constexpr (RES) {
#pragma unroll
    for (int j = 0; j < J; ++j) {
      u32x4 s;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        s[i] = pack_bf16(bf16_lo(xv[j][i]) + bf16_lo(rv[j][i]), bf16_hi(xv[j][i]) + bf16_hi(rv[j][i]));
      xv[j] = s;
    }
  }
  // xv now holds h (packed bf16); sum of squares over the live chunks
  float hf[kKeepH ? J : 1][8];
  double ss = 0.0;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    if (TAIL != kExact && j > 0 && j * T >= C) break;   // the rest lie past the row end for the whole workgroup
    u32x4 hw = xv[j];
    if (TAIL == kRagged && j * T + tid >= C) hw = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a = bf16_lo(hw[i]), b = bf16_hi(hw[i]);
      if constexpr (kKeepH) {
        hf[j][2 * i] = a;
        hf[j][2 * i + 1] = b;
      }
      ss = __builtin_fma((double)a, (double)a, ss);
      ss = __builtin_fma((double)b, (double)b, ss);
    }
  }
  ss = PACK == kPackLanes ? lanes_sum(ss, lt) : wave_sum(ss);
  const int nw = T >> 6;
  if (!kPacked && nw > 1) {
    // The waves' sums in a fixed pairwise tree over all 16 slots, four adds
    // deep (one dependent chain of nw adds was on the critical path of the
    // short launches); the slots past the last wave hold zero, which adds
    // exactly.
    if ((tid & 63) == 0) red[tid >> 6] = ss;
    if (tid >= nw && tid < kMaxWaves) red[tid] = 0.0;
    __syncthreads();
    double t[kMaxWaves / 2];
#pragma unroll
    for (int k = 0; k < kMaxWaves / 2; ++k) t[k] = red[2 * k] + red[2 * k + 1];
#pragma unroll
    for (int n = kMaxWaves / 4; n >= 1; n /= 2) {
#pragma unroll
      for (int k = 0; k < n; ++k) t[k] = t[2 * k] + t[2 * k + 1];
    }
    ss = t[0];
  }
  // ss / N, correctly rounded, from the correctly rounded reciprocal rn: the
  // product q0 is within an ulp of the quotient, its residual ss - q0 * N is
  // exact in one fma, and one more fma with rn rounds the corrected quotient
  // to nearest (Markstein's quotient refinement).
  const double nd = (double)N;
  const double q0 = ss * rn;
  const double ms = __builtin_fma(__builtin_fma(-q0, nd, ss), rn, q0);
  const double denom = ms + (double)eps;
  // fl32 of the inverse norm; the fp64 value itself is formed only where an
  // element is redone in fp64. Rows whose inverse norm leaves the
  // comfortable fp32 range take the exact path for every element.
  bool row_exact;
  float inv_lo;
  const float inv32 = inv_norm32(denom, row_exact, inv_lo);
  // one row per wave or per workgroup: the window offset is wave-uniform
  const uint32_t win = PACK == kPackLanes ? bf16_window_offset(inv_lo)
                                          : __builtin_amdgcn_readfirstlane(bf16_window_offset(inv_lo));
  // (The empty asm keeps the compiler from hoisting the loop-invariant fp64
  // inverse out of the rare block that calls this.)
  const auto inv64 = [denom] {
    double d = denom;
    asm volatile("" : "+v"(d));
    return inv_norm64(d);
  };

  // ---- phase 2: normalize, bf16, group scale, codes -----------------------
  u32x4* ybrow = ybase ? reinterpret_cast<u32x4*>(ybase + m * ldb) : nullptr;
  u32x4* hrow = RES ? reinterpret_cast<u32x4*>(hbase + m * ldr) : nullptr;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int c = j * T + tid;
    if (TAIL == kUniform && j * T >= C) continue;   // a whole step past the row end (wave-uniform)
    if (TAIL == kRagged && (c < lo || c >= hi)) continue;
    u32x4 g;
    if constexpr (kShort) g = gv[j];
    else g = grow[c];
    float hv[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      hv[2 * i] = kKeepH ? hf[kKeepH ? j : 0][2 * i] : bf16_lo(xv[j][i]);
      hv[2 * i + 1] = kKeepH ? hf[kKeepH ? j : 0][2 * i + 1] : bf16_hi(xv[j][i]);
    }
    uint32_t am;
    const u32x4 yw = norm_bf16x8<kSplitExact>(hv, xv[j], g, inv32, inv_lo, win, inv64, row_exact, am);
    // All stores of a row go out after its reduction: keeping the residual
    // write next to the others measured 3% faster than writing it as soon as
    // it is formed.
    if constexpr (RES) __builtin_nontemporal_store(xv[j], hrow + c);
    if (ybrow) __builtin_nontemporal_store(yw, ybrow + c);

    if constexpr (FMT == 2) continue;   // norm only: no quantization

    if constexpr (FMT == 0) {
      // FP8 e4m3fn, group 128 = one 16-lane DPP row
      float v[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = bf16_lo(yw[i]);
        v[2 * i + 1] = bf16_hi(yw[i]);
      }
      const uint32_t gam = max16(am);
      const float sc = fp8_scale(gam);
      const u32x2 qw = fp8_codes8(v, sc, __uint_as_float(gam << 16));
      u32x2* qrow = reinterpret_cast<u32x2*>(qbase + m * (int64_t)N);
      __builtin_nontemporal_store(qw, qrow + c);
      if ((tid & 15) == 0) {
        const int64_t g = c >> 4;
        reinterpret_cast<float*>(sbase)[layout == 2 ? g * M + m : m * (N >> 7) + g] = sc;
      }
    } else if constexpr (FMT == 1) {
      // MXFP4 e2m1, group 32 = one lane quad
      const uint32_t byte = mx_scale_byte(max4(am));
      const uint32_t w = fp4_codes8(yw, byte);
      uint32_t* qrow = reinterpret_cast<uint32_t*>(qbase + m * (int64_t)(N >> 1));
      __builtin_nontemporal_store(w, qrow + c);
      if ((tid & 3) == 0) {
        const int64_t gcount = N >> 5, gi = c >> 2;
        const int64_t off = layout == 0   ? m * gcount + gi
                            : layout == 1 ? (m >> 5) * (32 * gcount) + gi * 32 + (m & 31)
                                          : gi * M + m;
        reinterpret_cast<uint8_t*>(sbase)[off] = (uint8_t)byte;
      }
    }
  }
}

// ------------------------------------------------------------------------
// Standalone dynamic per-group quantization of bf16 rows (the separate quant
// kernel of the unfused chain: [ARQ, kernel count table] lists it as the
// dynamic per-group scaled quant kernel, [ARQ, Fallback order] as the
// separate per-1x128 quant). Same group arithmetic as the fused kernel.
// Grid: x = row, y = block of 64*W chunks of that row, one chunk per lane.

struct QuantArgs {
  const uint16_t* x;   // bf16 rows
  int64_t ldx;
  uint8_t* q;
  void* scale;
  int32_t M, N;
  int32_t layout;
};

template <int FMT>
__global__ void __launch_bounds__(256) rmsq_group_quant_kernel(const QuantArgs A) {
  const int64_t m = blockIdx.x;
  const int C = A.N >> 3;
  const int c = (int)blockIdx.y * (int)blockDim.x + (int)threadIdx.x;
  if (c >= C) return;   // whole groups exit together: C is a multiple of the group's lanes
  const u32x4 yw = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(A.x + m * A.ldx) + c);
  const uint32_t am = amax8(yw);
  if constexpr (FMT == 0) {
    float v[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_lo(yw[i]);
      v[2 * i + 1] = bf16_hi(yw[i]);
    }
    const uint32_t gam = max16(am);
    const float sc = fp8_scale(gam);
    const u32x2 qw = fp8_codes8(v, sc, __uint_as_float(gam << 16));
    __builtin_nontemporal_store(qw, reinterpret_cast<u32x2*>(A.q + m * (int64_t)A.N) + c);
    if ((threadIdx.x & 15) == 0) {
      const int64_t g = c >> 4;
      reinterpret_cast<float*>(A.scale)[A.layout == 2 ? g * A.M + m : m * (A.N >> 7) + g] = sc;
    }
  } else {
    const uint32_t byte = mx_scale_byte(max4(am));
    const uint32_t w = fp4_codes8(yw, byte);
    __builtin_nontemporal_store(w, reinterpret_cast<uint32_t*>(A.q + m * (int64_t)(A.N >> 1)) + c);
    if ((threadIdx.x & 3) == 0) {
      const int64_t gcount = A.N >> 5, gi = c >> 2;
      const int64_t off = A.layout == 0   ? m * gcount + gi
                          : A.layout == 1 ? (m >> 5) * (32 * gcount) + gi * 32 + (m & 31)
                                          : gi * A.M + m;
      reinterpret_cast<uint8_t*>(A.scale)[off] = (uint8_t)byte;
    }
  }
}

}  // namespace rmsq
