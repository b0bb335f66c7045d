// rmsq_abi.hip - C ABI of librmsq: argument validation, device check, launch
// configuration and kernel dispatch. Declarations and the contract are in
// include/rmsq.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "rmsq.h"
#include "rmsq_abi_common.h"
#include "rmsq_kernel.h"

namespace rmsq_abi {

thread_local char g_err[512];

rmsq_status fail(rmsq_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

rmsq_status check_overlaps(const Range* rs, int nr) {
  for (int i = 0; i < nr; ++i) {
    if (!rs[i].output) continue;
    for (int k = 0; k < nr; ++k) {
      if (k == i || (k < i && rs[k].output)) continue;
      const Range &a = rs[i], &b = rs[k];
      if (a.lo >= b.hi || b.lo >= a.hi) continue;
      // in-place residual: residual_out is exactly residual_in of the same problem
      if (a.problem == b.problem && a.kind == 2 && b.kind == 1 && a.lo == b.lo && a.hi == b.hi) continue;
      return fail(RMSQ_ERR_INVALID_ARG, "output buffer %d of problem %d overlaps buffer %d of problem %d", a.kind,
                  a.problem, b.kind, b.problem);
    }
  }
  return RMSQ_OK;
}

namespace {
// gfx950 check, cached per device.
std::atomic<int8_t> g_arch_ok[64];
}  // namespace

bool device_is_gfx950(int dev) {
  if (dev < 0) return false;
  if (dev < 64) {
    const int8_t c = g_arch_ok[dev].load(std::memory_order_relaxed);
    if (c) return c > 0;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return false;
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < 64) g_arch_ok[dev].store(ok ? 1 : -1, std::memory_order_relaxed);
  return ok;
}

}  // namespace rmsq_abi

namespace {

using namespace rmsq_abi;

size_t scale_bytes(int64_t M, int64_t N, int32_t group, int32_t fmt, int32_t layout) {
  if (M < 0 || N <= 0 || group <= 0 || N % group) return 0;
  const int64_t G = N / group;
  if (fmt == RMSQ_FMT_FP8_E4M3FN && group == 128 &&
      (layout == RMSQ_SCALE_ROW_MAJOR || layout == RMSQ_SCALE_COL_MAJOR))
    return (size_t)(M * G * 4);
  if (fmt == RMSQ_FMT_MXFP4_E2M1 && group == 32) {
    if (layout == RMSQ_SCALE_ROW_MAJOR || layout == RMSQ_SCALE_COL_MAJOR) return (size_t)(M * G);
    if (layout == RMSQ_SCALE_TILED32) return (size_t)(((M + 31) / 32) * 32 * G);
  }
  return 0;
}

// What a problem asks for: the fused operation, the norm alone (bf16
// output, no quantization), or the quantization alone (x is the bf16 input).
enum class Mode { kFused, kNormOnly, kQuantOnly };

// Validate one problem and append its buffers' byte ranges.
rmsq_status check_problem(const rmsq_problem& p, int idx, int32_t fmt0, Mode mode, Range* rs, int* nr) {
  const bool quant = mode != Mode::kNormOnly, norm = mode != Mode::kQuantOnly;
  int32_t group = 8;
  if (quant) {
    if (p.fmt != RMSQ_FMT_FP8_E4M3FN && p.fmt != RMSQ_FMT_MXFP4_E2M1)
      return fail(RMSQ_ERR_UNSUPPORTED, "problem %d: unknown fmt %d", idx, p.fmt);
    if (p.fmt != fmt0) return fail(RMSQ_ERR_INVALID_ARG, "problem %d: all problems must share fmt", idx);
    group = p.fmt == RMSQ_FMT_FP8_E4M3FN ? 128 : 32;
    if (p.group != group)
      return fail(RMSQ_ERR_UNSUPPORTED, "problem %d: group %d unsupported for fmt %d (need %d)", idx, p.group, p.fmt,
                  group);
    if (p.scale_layout != RMSQ_SCALE_ROW_MAJOR && p.scale_layout != RMSQ_SCALE_TILED32 &&
        p.scale_layout != RMSQ_SCALE_COL_MAJOR)
      return fail(RMSQ_ERR_INVALID_ARG, "problem %d: unknown scale layout %d", idx, p.scale_layout);
    if (p.scale_layout == RMSQ_SCALE_TILED32 && p.fmt != RMSQ_FMT_MXFP4_E2M1)
      return fail(RMSQ_ERR_UNSUPPORTED, "problem %d: the tiled scale layout is for MXFP4 only", idx);
  }
  if (p.M < 0) return fail(RMSQ_ERR_INVALID_ARG, "problem %d: M = %lld < 0", idx, (long long)p.M);
  if (p.N <= 0 || p.N % group)
    return fail(RMSQ_ERR_INVALID_ARG, "problem %d: N = %lld not a positive multiple of %d", idx, (long long)p.N, group);
  if (p.N > RMSQ_N_MAX) return fail(RMSQ_ERR_UNSUPPORTED, "problem %d: N = %lld > %d", idx, (long long)p.N, RMSQ_N_MAX);
  if (p.M > INT32_MAX) return fail(RMSQ_ERR_UNSUPPORTED, "problem %d: M = %lld too large", idx, (long long)p.M);
  if (norm && (!std::isfinite(p.eps) || p.eps < 0.0f))
    return fail(RMSQ_ERR_INVALID_ARG, "problem %d: eps must be finite and >= 0", idx);
  const int64_t ldx = p.ldx ? p.ldx : p.N, ldr = p.ldr ? p.ldr : p.N, ldb = p.ldb ? p.ldb : p.N;
  if (ldx < p.N || ldx % 8 || (norm && p.residual_in && (ldr < p.N || ldr % 8)) ||
      (norm && p.out_bf16 && (ldb < p.N || ldb % 8)))
    return fail(RMSQ_ERR_INVALID_ARG, "problem %d: row strides must be multiples of 8 and >= N", idx);
  if (p.M == 0) return RMSQ_OK;  // nothing is read or written; pointers may be NULL
  if (norm && (p.residual_in == nullptr) != (p.residual_out == nullptr))
    return fail(RMSQ_ERR_INVALID_ARG, "problem %d: residual_in and residual_out must both be set or both be NULL", idx);
  if (!p.x || (norm && !p.gamma) || (quant && (!p.out_q || !p.out_scale)))
    return fail(RMSQ_ERR_INVALID_ARG, "problem %d: x, gamma, out_q and out_scale must be non-NULL", idx);
  if (mode == Mode::kNormOnly && !p.out_bf16)
    return fail(RMSQ_ERR_INVALID_ARG, "problem %d: the norm alone needs out_bf16", idx);
  if (!aligned(p.x, 16) || (norm && (!aligned(p.gamma, 16) || (p.residual_in && !aligned(p.residual_in, 16)) ||
                                     (p.residual_out && !aligned(p.residual_out, 16)) ||
                                     (p.out_bf16 && !aligned(p.out_bf16, 16)))))
    return fail(RMSQ_ERR_INVALID_ARG, "problem %d: bf16 pointers must be 16-byte aligned", idx);
  if (quant && !aligned(p.out_q, p.fmt == RMSQ_FMT_FP8_E4M3FN ? 8 : 4))
    return fail(RMSQ_ERR_INVALID_ARG, "problem %d: out_q misaligned", idx);
  if (quant && p.fmt == RMSQ_FMT_FP8_E4M3FN && !aligned(p.out_scale, 4))
    return fail(RMSQ_ERR_INVALID_ARG, "problem %d: out_scale must be 4-byte aligned", idx);

  auto add = [&](const void* ptr, int64_t bytes, bool out, int kind) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(ptr);
    rs[(*nr)++] = Range{a, a + (uintptr_t)bytes, out, idx, kind};
  };
  const int64_t M = p.M, N = p.N;
  add(p.x, ((M - 1) * ldx + N) * 2, false, 0);
  if (norm) {
    if (p.residual_in) {
      add(p.residual_in, ((M - 1) * ldr + N) * 2, false, 1);
      add(p.residual_out, ((M - 1) * ldr + N) * 2, true, 2);
    }
    add(p.gamma, N * 2, false, 3);
    if (p.out_bf16) add(p.out_bf16, ((M - 1) * ldb + N) * 2, true, 6);
  }
  if (quant) {
    add(p.out_q, M * (p.fmt == RMSQ_FMT_FP8_E4M3FN ? N : N / 2), true, 4);
    add(p.out_scale, (int64_t)scale_bytes(M, N, p.group, p.fmt, p.scale_layout), true, 5);
  }
  return RMSQ_OK;
}

// Launch shape: chunk-steps per lane J (compiled set) and waves per row W.
// Measured on MI355X: spreading a row over several waves with 2-4 chunks per
// lane sustains the traffic far better than long per-lane rows (one wave per
// 7168-wide row leaves the HBM queues bursty), while a single chunk per lane
// pays the per-wave fixed cost of the norm (reduction, fp64 inverse square
// root) too often. Rule: the first J of 2, 3, 4, 1 whose W stays <= 8 with
// at most 20% idle lanes (7168 -> J 2 x 7 waves, 1536 -> J 3 x 1 wave);
// then relax the wave limit, then take anything that fits. With at most two
// rows per compute unit each row's latency counts most: there the most waves
// win (J 1 x 14 waves for 64 rows of 7168: 6.3 us against 6.8 us for J 2 x 7;
// 512 rows 8.42 against 8.63 us; from 768 rows J 2 x 7 is faster again:
// 10.9 against 12.4 us). Rows of at most 64 chunks take one chunk per lane:
// packed, they then share a wave 16, 32 or 64 lanes each.
constexpr int kJs[] = {2, 3, 4, 1, 7, 8, 14};
constexpr int kJsFewRows[] = {1, 2, 3, 4, 7, 8, 14};
constexpr int kWaveRowsPerBlock = 8;
constexpr int kMaxSplits = 8;

void pick_shape(int64_t C, int64_t rows, int* J_out, int* W_out) {
  if (C <= 64) {
    *J_out = 1;
    *W_out = 1;
    return;
  }
  const bool few = rows <= 2 * kComputeUnits;
  for (int pass = 0; pass < 3; ++pass) {
    for (int k = 0; k < 7; ++k) {
      const int J = few ? kJsFewRows[k] : kJs[k];
      const int64_t W = (C + 64 * J - 1) / (64 * J);
      if (W > rmsq::max_waves(J)) continue;
      const int64_t slots = W * 64 * J;
      if (pass < 2 && (slots - C) * 5 > slots) continue;
      if (pass == 0 && W > (few ? rmsq::kMaxWaves : 8)) continue;
      *J_out = J;
      *W_out = (int)W;
      return;
    }
  }
  *J_out = 4;
  *W_out = rmsq::kMaxWaves;
}

// The fused kernel's arguments: the launch scalars (preloaded into SGPRs),
// then the launch description.
#define RMSQ_LAUNCH_ARGS(L)                                                                                  \
  (L).count, (L).rows, (L).row_group_log2, (L).splits_log2, (L).row_begin[1], (L).row_begin[2], (L).row_begin[3], \
      (int32_t)block.x, (int32_t)grid.x, (L)

// The exact and uniform tails are used for J <= 4 only: the long per-lane
// shapes (very wide rows) keep their bounds, which also keeps them within the
// register budget; the uniform tail is compiled for rows packed one per wave
// only (with one chunk per lane it coincides with the exact one).
template <int FMT, bool RES, int TAIL>
void launch_res(const rmsq::Launch& L, int J, int pack, const dim3 grid, const dim3 block, hipStream_t stream) {
  using rmsq::rmsq_fused_kernel;
  constexpr int kPackedTail = TAIL;
  constexpr int kRowTail = TAIL == rmsq::kUniform ? rmsq::kRagged : TAIL;
  if (pack == rmsq::kPackLanes) {   // one chunk per lane, 16 to 64 lanes per row
    hipLaunchKernelGGL((rmsq_fused_kernel<FMT, 1, RES, rmsq::kPackLanes, kRowTail>), grid, block, 0, stream,
                       RMSQ_LAUNCH_ARGS(L));
    return;
  }
  if (pack == rmsq::kPackWave) {   // one row per wave (J <= 4 only)
    constexpr int P = rmsq::kPackWave;
    switch (J) {
      case 4: hipLaunchKernelGGL((rmsq_fused_kernel<FMT, 4, RES, P, kPackedTail>), grid, block, 0, stream, RMSQ_LAUNCH_ARGS(L)); break;
      case 3: hipLaunchKernelGGL((rmsq_fused_kernel<FMT, 3, RES, P, kPackedTail>), grid, block, 0, stream, RMSQ_LAUNCH_ARGS(L)); break;
      case 2: hipLaunchKernelGGL((rmsq_fused_kernel<FMT, 2, RES, P, kPackedTail>), grid, block, 0, stream, RMSQ_LAUNCH_ARGS(L)); break;
      default: hipLaunchKernelGGL((rmsq_fused_kernel<FMT, 1, RES, P, kPackedTail>), grid, block, 0, stream, RMSQ_LAUNCH_ARGS(L)); break;
    }
    return;
  }
  constexpr int N = rmsq::kPackNone;
  switch (J) {
    case 14: hipLaunchKernelGGL((rmsq_fused_kernel<FMT, 14, RES, N, rmsq::kRagged>), grid, block, 0, stream, RMSQ_LAUNCH_ARGS(L)); break;
    case 8: hipLaunchKernelGGL((rmsq_fused_kernel<FMT, 8, RES, N, rmsq::kRagged>), grid, block, 0, stream, RMSQ_LAUNCH_ARGS(L)); break;
    case 7: hipLaunchKernelGGL((rmsq_fused_kernel<FMT, 7, RES, N, rmsq::kRagged>), grid, block, 0, stream, RMSQ_LAUNCH_ARGS(L)); break;
    case 4: hipLaunchKernelGGL((rmsq_fused_kernel<FMT, 4, RES, N, kRowTail>), grid, block, 0, stream, RMSQ_LAUNCH_ARGS(L)); break;
    case 3: hipLaunchKernelGGL((rmsq_fused_kernel<FMT, 3, RES, N, kRowTail>), grid, block, 0, stream, RMSQ_LAUNCH_ARGS(L)); break;
    case 2: hipLaunchKernelGGL((rmsq_fused_kernel<FMT, 2, RES, N, kRowTail>), grid, block, 0, stream, RMSQ_LAUNCH_ARGS(L)); break;
    default: hipLaunchKernelGGL((rmsq_fused_kernel<FMT, 1, RES, N, kRowTail>), grid, block, 0, stream, RMSQ_LAUNCH_ARGS(L)); break;
  }
}

// One launch of up to four problems with the shape chosen for it; they
// either all have a residual or none has (the caller splits a mixed set).
// R > 1: packed rows, W is 1 and a workgroup has R waves, each holding one
// row (pack = kPackWave) or, with one chunk per lane, one row per
// 2^lanes_log2 lanes (kPackLanes; L.rows then counts waves).
struct Plan {
  rmsq::Launch L;
  int J, W, R;
  int pack;       // rmsq::Pack
  int64_t rows;   // rows over the launch's problems
  dim3 grid, block;
};

// The launch's grid: one workgroup per row (R > 1: per R waves; with row
// splits, per split of a row, the rows padded to a multiple of 8).
void plan_grid(Plan& P) {
  const rmsq::Launch& L = P.L;
  const int64_t padded = (L.rows + 7) / 8 * 8;
  const int64_t blocks = P.R > 1 ? (L.rows + P.R - 1) / P.R : L.splits_log2 > 0 ? padded << L.splits_log2 : L.rows;
  P.grid = dim3((unsigned)blocks);
  P.block = dim3((unsigned)(64 * (P.R > 1 ? P.R : P.W)));
}

// Lanes holding one row of problem i: 64 x W, or packed 2^lanes_log2.
int64_t row_lanes(const Plan& P, int i) { return P.R > 1 ? int64_t{1} << P.L.p[i].lanes_log2 : 64 * P.W; }


// How the launch's rows end (rmsq::Tail): every row exactly fills its J x T
// lanes (T lanes per row) - exact; packed rows that are all a whole number of
// T-lane steps - uniform; otherwise ragged. Packed launches whose last wave
// of a problem is partly empty, and row splits, are ragged.
int launch_tail(const Plan& P) {
  const rmsq::Launch& L = P.L;
  if (L.splits_log2 != 0 || P.J > 4) return rmsq::kRagged;
  bool exact = true, uniform = P.R > 1;
  for (int i = 0; i < L.count; ++i) {
    const int64_t C = L.p[i].N >> 3, T = row_lanes(P, i);
    const bool full = P.pack != rmsq::kPackLanes || L.p[i].M % (64 / T) == 0;
    exact &= C == P.J * T && full;
    uniform &= C % T == 0 && C <= P.J * T && full;
  }
  return exact ? rmsq::kExact : uniform ? rmsq::kUniform : rmsq::kRagged;
}

template <int FMT>
rmsq_status launch_fmt(const Plan& P, hipStream_t stream) {
  const rmsq::Launch& L = P.L;
  const int tail = launch_tail(P);
  const bool res = L.p[0].r != nullptr;
  if (tail == rmsq::kExact) {
    if (res) launch_res<FMT, true, rmsq::kExact>(L, P.J, P.pack, P.grid, P.block, stream);
    else launch_res<FMT, false, rmsq::kExact>(L, P.J, P.pack, P.grid, P.block, stream);
  } else if (tail == rmsq::kUniform) {
    if (res) launch_res<FMT, true, rmsq::kUniform>(L, P.J, P.pack, P.grid, P.block, stream);
    else launch_res<FMT, false, rmsq::kUniform>(L, P.J, P.pack, P.grid, P.block, stream);
  } else {
    if (res) launch_res<FMT, true, rmsq::kRagged>(L, P.J, P.pack, P.grid, P.block, stream);
    else launch_res<FMT, false, rmsq::kRagged>(L, P.J, P.pack, P.grid, P.block, stream);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(RMSQ_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return RMSQ_OK;
}

bool compiled_J(int J) {
  for (int k : kJs)
    if (k == J) return true;
  return false;
}

// The optional per-call launch hint, checked before anything is planned.
rmsq_status check_hint(const rmsq_launch_hint* h) {
  if (!h) return RMSQ_OK;
  if ((h->chunks_per_lane == 0) != (h->waves_per_row == 0))
    return fail(RMSQ_ERR_INVALID_ARG, "hint: chunks_per_lane and waves_per_row are set together (or both 0)");
  if (h->chunks_per_lane != 0 &&
      (!compiled_J(h->chunks_per_lane) || h->waves_per_row < 1 || h->waves_per_row > rmsq::max_waves(h->chunks_per_lane)))
    return fail(RMSQ_ERR_INVALID_ARG, "hint: no launch shape of %d chunks per lane x %d waves", h->chunks_per_lane,
                h->waves_per_row);
  if (h->row_group < 0 || h->row_group > 64)
    return fail(RMSQ_ERR_INVALID_ARG, "hint: row_group %d outside 0..64", h->row_group);
  if (h->waves_per_workgroup < 0 || h->waves_per_workgroup > rmsq::kMaxWaves)
    return fail(RMSQ_ERR_INVALID_ARG, "hint: waves_per_workgroup %d outside 0..%d", h->waves_per_workgroup,
                rmsq::kMaxWaves);
  if (h->row_splits < 0 || h->row_splits > kMaxSplits)
    return fail(RMSQ_ERR_INVALID_ARG, "hint: row_splits %d outside 0..%d", h->row_splits, kMaxSplits);
  if (h->lanes_per_row != 0 && h->lanes_per_row != 16 && h->lanes_per_row != 32 && h->lanes_per_row != 64)
    return fail(RMSQ_ERR_INVALID_ARG, "hint: lanes_per_row %d is not 0, 16, 32 or 64", h->lanes_per_row);
  return RMSQ_OK;
}

// Validate the problems and plan their launches (one for the problems with
// a residual, one for those without; a set that mixes the two takes two
// launches, in that order). Everything here is host arithmetic on the
// arguments: no HIP call, no state outside *plans.
rmsq_status plan(const rmsq_problem* ps, int32_t count, Mode mode, const rmsq_launch_hint* hint, Plan plans[2],
                 int* np_out) {
  g_err[0] = 0;
  *np_out = 0;
  if (!ps) return fail(RMSQ_ERR_INVALID_ARG, "problems is NULL");
  if (count < 1 || count > RMSQ_MAX_PROBLEMS)
    return fail(RMSQ_ERR_INVALID_ARG, "count = %d outside 1..%d", count, RMSQ_MAX_PROBLEMS);
  if (const rmsq_status s = check_hint(hint); s != RMSQ_OK) return s;
  const rmsq_launch_hint h = hint ? *hint : rmsq_launch_hint{0, 0, 0, 0, 0, 0};
  Range rs[RMSQ_MAX_PROBLEMS * 7];
  int nr = 0;
  for (int i = 0; i < count; ++i) {
    const rmsq_status s = check_problem(ps[i], i, ps[0].fmt, mode, rs, &nr);
    if (s != RMSQ_OK) return s;
  }
  if (const rmsq_status s = check_overlaps(rs, nr); s != RMSQ_OK) return s;

  int np = 0;
  for (int with_res = 1; with_res >= 0; --with_res) {
    Plan& P = plans[np];
    P = Plan{};
    rmsq::Launch& L = P.L;
    int64_t rows = 0, Cmax = 0;
    int n = 0;
    for (int i = 0; i < count; ++i) {
      const rmsq_problem& p = ps[i];
      if (p.M == 0 || (p.residual_in != nullptr) != (with_res == 1)) continue;
      rmsq::Problem& d = L.p[n++];
      d.x = static_cast<const uint16_t*>(p.x);
      d.r = static_cast<const uint16_t*>(p.residual_in);
      d.h = static_cast<uint16_t*>(p.residual_out);
      d.gamma = static_cast<const uint16_t*>(p.gamma);
      d.q = mode == Mode::kNormOnly ? nullptr : static_cast<uint8_t*>(p.out_q);
      d.scale = mode == Mode::kNormOnly ? nullptr : p.out_scale;
      d.yb = static_cast<uint16_t*>(p.out_bf16);
      d.ldx = p.ldx ? p.ldx : p.N;
      d.ldr = p.ldr ? p.ldr : p.N;
      d.ldb = p.ldb ? p.ldb : p.N;
      d.M = (int32_t)p.M;
      d.N = (int32_t)p.N;
      L.row_begin[n - 1] = (int32_t)rows;
      d.layout = p.scale_layout;
      d.eps = p.eps;
      d.rn = 1.0 / (double)p.N;
      rows += p.M;
      if (p.N / 8 > Cmax) Cmax = p.N / 8;
    }
    if (n == 0) continue;
    if (rows > INT32_MAX) return fail(RMSQ_ERR_UNSUPPORTED, "total rows %lld exceed the grid limit", (long long)rows);
    L.count = n;
    L.rows = (int32_t)rows;

    int J, W;
    pick_shape(Cmax, rows, &J, &W);
    if (h.chunks_per_lane != 0) {
      if ((int64_t)h.chunks_per_lane * h.waves_per_row * 64 < Cmax)
        return fail(RMSQ_ERR_INVALID_ARG, "hint: %d chunks per lane x %d waves do not cover rows of %lld elements",
                    h.chunks_per_lane, h.waves_per_row, (long long)Cmax * 8);
      J = h.chunks_per_lane;
      W = h.waves_per_row;
    }
    // Row grouping per XCD (measured): 16 rows when a problem writes tiled or
    // column-major scales (neighbouring rows' scales share lines there; half a
    // 32-row tile per XCD keeps each line in few L2s, +1% for tiled); plain
    // dispatch order otherwise, which was fastest for row-major scales.
    bool grouped = false;
    for (int i = 0; i < n; ++i) grouped |= L.p[i].layout != RMSQ_SCALE_ROW_MAJOR;
    int lg = grouped ? 4 : 0;
    if (h.row_group > 0) {
      lg = 0;
      while ((2 << lg) <= h.row_group) ++lg;   // largest power of two <= the hint
    }
    // Rows that fit one wave are packed several per workgroup once there are
    // enough of them to fill the machine (a CU holds only so many
    // workgroups, so one-wave workgroups leave wave slots empty).
    int R = 1;
    if (W == 1 && J <= 4) R = h.waves_per_workgroup > 0 ? h.waves_per_workgroup
                                                       : (rows >= 4 * kComputeUnits ? kWaveRowsPerBlock : 1);
    int lgR = 0;
    while ((2 << lgR) <= R) ++lgR;
    L.row_group_log2 = R > 1 ? (lg > lgR ? lg - lgR : 0) : lg;   // groups of workgroups when packed
    // Fewer rows than compute units: split each row over several workgroups
    // (each recomputes the row's sum of squares, bit-identically, and does
    // the normalize / quantize work for its share), so every CU works.
    // Not with an in-place residual: a split would read the residual row
    // while another split of the same row overwrites it with h.
    bool in_place = false;
    for (int i = 0; i < n; ++i) in_place |= L.p[i].r != nullptr && L.p[i].r == L.p[i].h;
    L.splits_log2 = 0;
    if (R == 1 && !in_place) {
      int S = 1;
      if (h.row_splits > 0)
        while (S * 2 <= h.row_splits) S *= 2;   // largest power of two <= the hint
      else
        while (S < kMaxSplits && rows * S * 2 <= kComputeUnits) S *= 2;
      const int64_t q = mode == Mode::kNormOnly ? 1 : ps[0].fmt == RMSQ_FMT_FP8_E4M3FN ? 16 : 4;
      int64_t Cmin = Cmax;
      for (int i = 0; i < n; ++i) Cmin = std::min<int64_t>(Cmin, L.p[i].N / 8);
      while (S > 1 && Cmin / q < S) S /= 2;   // at least one group per split
      while ((1 << L.splits_log2) < S) ++L.splits_log2;
      if (S > 1) L.row_group_log2 = 0;
    }
    // Packed rows of one chunk per lane: each problem's rows take 2^k lanes
    // (16, 32 or 64), the fewest that hold the row unless the hint fixes
    // them, so a wave holds 2^(6-k) rows and their statistics share one
    // instruction sequence (128-wide rows: four per wave). Measured against
    // one row per wave (16384 rows, MI355X): 5.3 against 9.0 us for rows of
    // 128, 8.0 against 12.7 us for rows of 256 with a residual. The launch
    // then counts waves: problem i fills waves row_begin[i] ... (its last one
    // possibly part empty). Wider rows, and more chunks per lane, keep one
    // row per wave.
    P.rows = rows;
    P.pack = R > 1 ? rmsq::kPackWave : rmsq::kPackNone;
    for (int i = 0; i < n; ++i) L.p[i].lanes_log2 = 6;
    if (h.lanes_per_row > 0 && h.lanes_per_row < 64 && R > 1 && J != 1)
      return fail(RMSQ_ERR_INVALID_ARG, "hint: %d lanes per row needs one chunk per lane (the launch has %d)",
                  h.lanes_per_row, J);
    if (R > 1 && J == 1) {
      bool lanes = false;
      for (int i = 0; i < n; ++i) {
        rmsq::Problem& d = L.p[i];
        const int64_t C = d.N / 8;
        int lt = 4;
        if (h.lanes_per_row > 0) {
          while ((1 << lt) < h.lanes_per_row) ++lt;
          if (C > int64_t{1} << lt)
            return fail(RMSQ_ERR_INVALID_ARG, "hint: %d lanes per row do not hold rows of %lld elements",
                        h.lanes_per_row, (long long)C * 8);
        } else {
          while (lt < 6 && C > int64_t{1} << lt) ++lt;
        }
        d.lanes_log2 = lt;
        lanes |= lt < 6;
      }
      if (lanes) {
        P.pack = rmsq::kPackLanes;
        int64_t waves = 0;
        for (int i = 0; i < n; ++i) {
          L.row_begin[i] = (int32_t)waves;
          waves += (L.p[i].M + (64 >> L.p[i].lanes_log2) - 1) >> (6 - L.p[i].lanes_log2);
        }
        L.rows = (int32_t)waves;
      }
    }
    P.J = J;
    P.W = W;
    P.R = R;
    plan_grid(P);
    // the dispatch counts work-items per dimension in 32 bits
    if ((uint64_t)P.grid.x * P.block.x > UINT32_MAX)
      return fail(RMSQ_ERR_UNSUPPORTED, "%lld rows of %lld elements need %llu work-items in one launch, beyond 2^32",
                  (long long)rows, (long long)Cmax * 8, (unsigned long long)P.grid.x * P.block.x);
    ++np;
  }
  *np_out = np;
  return RMSQ_OK;
}

rmsq_status run(const rmsq_problem* ps, int32_t count, Mode mode, const rmsq_launch_hint* hint, void* stream) {
  Plan plans[2];
  int np = 0;
  if (const rmsq_status s = plan(ps, count, mode, hint, plans, &np); s != RMSQ_OK) return s;
  if (np == 0) return RMSQ_OK;   // every problem has M == 0
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || !device_is_gfx950(dev))
    return fail(RMSQ_ERR_UNSUPPORTED, "current HIP device is not a gfx950 GPU");
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int k = 0; k < np; ++k) {
    const rmsq_status st = mode == Mode::kNormOnly               ? launch_fmt<2>(plans[k], s)
                           : ps[0].fmt == RMSQ_FMT_FP8_E4M3FN ? launch_fmt<0>(plans[k], s)
                                                                : launch_fmt<1>(plans[k], s);
    if (st != RMSQ_OK) return st;
  }
  return RMSQ_OK;
}

// The quantization alone on bf16 rows: grid x = row, y = blocks of 128
// chunks, one 8-element chunk per lane.
rmsq_status run_quant(const rmsq_problem& p, void* stream) {
  g_err[0] = 0;
  Range rs[4];
  int nr = 0;
  if (const rmsq_status st = check_problem(p, 0, p.fmt, Mode::kQuantOnly, rs, &nr); st != RMSQ_OK) return st;
  if (const rmsq_status st = check_overlaps(rs, nr); st != RMSQ_OK) return st;
  if (p.M == 0) return RMSQ_OK;
  // one workgroup of 128 work-items per row (and per 1024 elements of it);
  // the dispatch counts work-items per dimension in 32 bits
  if (p.M > (int64_t)(UINT32_MAX / 128))
    return fail(RMSQ_ERR_UNSUPPORTED, "quant: M = %lld rows need more than 2^32 work-items in one launch",
                (long long)p.M);
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || !device_is_gfx950(dev))
    return fail(RMSQ_ERR_UNSUPPORTED, "current HIP device is not a gfx950 GPU");
  rmsq::QuantArgs A;
  A.x = static_cast<const uint16_t*>(p.x);
  A.ldx = p.ldx ? p.ldx : p.N;
  A.q = static_cast<uint8_t*>(p.out_q);
  A.scale = p.out_scale;
  A.M = (int32_t)p.M;
  A.N = (int32_t)p.N;
  A.layout = p.scale_layout;
  const int64_t C = p.N / 8;
  const dim3 grid((unsigned)p.M, (unsigned)((C + 127) / 128)), block(128);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p.fmt == RMSQ_FMT_FP8_E4M3FN)
    hipLaunchKernelGGL(rmsq::rmsq_group_quant_kernel<0>, grid, block, 0, s, A);
  else
    hipLaunchKernelGGL(rmsq::rmsq_group_quant_kernel<1>, grid, block, 0, s, A);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(RMSQ_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return RMSQ_OK;
}

}  // namespace

extern "C" {

rmsq_status rmsnorm_quant_group(const void* x, const void* residual_in, const void* gamma, float eps, int64_t M,
                                int64_t N, int32_t group, int32_t fmt, void* out_q, void* out_scale,
                                void* residual_out, void* out_bf16_or_null, void* stream) {
  rmsq_problem p;
  std::memset(&p, 0, sizeof p);
  p.x = x;
  p.residual_in = residual_in;
  p.residual_out = residual_out;
  p.gamma = gamma;
  p.eps = eps;
  p.M = M;
  p.N = N;
  p.group = group;
  p.fmt = fmt;
  p.scale_layout = RMSQ_SCALE_ROW_MAJOR;
  p.out_q = out_q;
  p.out_scale = out_scale;
  p.out_bf16 = out_bf16_or_null;
  return run(&p, 1, Mode::kFused, nullptr, stream);
}

rmsq_status rmsnorm_quant_group_multi(const rmsq_problem* problems, int32_t count, void* stream) {
  return run(problems, count, Mode::kFused, nullptr, stream);
}

rmsq_status rmsnorm_quant_group_multi_ex(const rmsq_problem* problems, int32_t count, const rmsq_launch_hint* hint,
                                         void* stream) {
  return run(problems, count, Mode::kFused, hint, stream);
}

rmsq_status rmsq_plan_launch(const rmsq_problem* problems, int32_t count, const rmsq_launch_hint* hint,
                             rmsq_launch_plan* out) {
  if (!out) return fail(RMSQ_ERR_INVALID_ARG, "plan output is NULL");
  std::memset(out, 0, sizeof *out);
  Plan plans[2];
  int np = 0;
  if (const rmsq_status s = plan(problems, count, Mode::kFused, hint, plans, &np); s != RMSQ_OK) return s;
  out->launches = np;
  for (int k = 0; k < np; ++k) {
    const Plan& P = plans[k];
    rmsq_launch_info& d = out->launch[k];
    d.problems = P.L.count;
    d.rows = (int32_t)P.rows;
    d.chunks_per_lane = P.J;
    d.waves_per_row = P.W;
    d.waves_per_workgroup = P.R;
    d.row_splits = 1 << P.L.splits_log2;
    d.row_group = 1 << P.L.row_group_log2;
    d.workgroups = (int64_t)P.grid.x;
    d.threads_per_workgroup = (int32_t)P.block.x;
    d.residual = P.L.p[0].r != nullptr;
    d.tail = launch_tail(P);
    for (int i = 0; i < P.L.count; ++i) d.lanes_per_row[i] = (int32_t)row_lanes(P, i);
  }
  return RMSQ_OK;
}

rmsq_status add_rmsnorm(const void* x, const void* residual_in, const void* gamma, float eps, int64_t M, int64_t N,
                        void* residual_out, void* out_bf16, void* stream) {
  rmsq_problem p;
  std::memset(&p, 0, sizeof p);
  p.x = x;
  p.residual_in = residual_in;
  p.residual_out = residual_out;
  p.gamma = gamma;
  p.eps = eps;
  p.M = M;
  p.N = N;
  p.out_bf16 = out_bf16;
  return run(&p, 1, Mode::kNormOnly, nullptr, stream);
}

rmsq_status dynamic_per_group_scaled_quant(const void* x, int64_t M, int64_t N, int32_t group, int32_t fmt,
                                           int32_t scale_layout, void* out_q, void* out_scale, void* stream) {
  rmsq_problem p;
  std::memset(&p, 0, sizeof p);
  p.x = x;
  p.M = M;
  p.N = N;
  p.group = group;
  p.fmt = fmt;
  p.scale_layout = scale_layout;
  p.out_q = out_q;
  p.out_scale = out_scale;
  return run_quant(p, stream);
}

int32_t rmsq_device_supported(int32_t device) {
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || device < 0 || device >= n) return 0;
  return device_is_gfx950(device) ? 1 : 0;
}

size_t rmsq_scale_bytes(int64_t M, int64_t N, int32_t group, int32_t fmt, int32_t scale_layout) {
  return scale_bytes(M, N, group, fmt, scale_layout);
}

const char* rmsq_status_string(rmsq_status s) {
  switch (s) {
    case RMSQ_OK: return "RMSQ_OK";
    case RMSQ_ERR_INVALID_ARG: return "RMSQ_ERR_INVALID_ARG";
    case RMSQ_ERR_UNSUPPORTED: return "RMSQ_ERR_UNSUPPORTED";
    case RMSQ_ERR_HIP: return "RMSQ_ERR_HIP";
    default: return "RMSQ_UNKNOWN_STATUS";
  }
}

const char* rmsq_last_error(void) { return g_err; }

int32_t rmsq_query_shape(int64_t N, int64_t rows, int32_t* J, int32_t* W) {
  if (N <= 0 || N % 8 || N > RMSQ_N_MAX || rows < 0 || !J || !W) return RMSQ_ERR_INVALID_ARG;
  int j, w;
  pick_shape(N / 8, rows, &j, &w);
  *J = j;
  *W = w;
  return RMSQ_OK;
}

}  // extern "C"
