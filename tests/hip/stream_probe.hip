// stream_probe.hip - test-only bandwidth probes: plain streams (read, write,
// copy) and the fused kernel's exact traffic pattern with no arithmetic, to
// measure the achievable HBM ceiling of the GPU. Grid-stride loops, bounds
// checked; n16 counts 16-byte elements.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rmsq.h"
#include "rmsq_kernel.h"

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <bool NT>
__device__ __forceinline__ u32x4 ld16(const u32x4* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}
template <bool NT, typename T>
__device__ __forceinline__ void st(T v, T* p) {
  if constexpr (NT) __builtin_nontemporal_store(v, p);
  else *p = v;
}

template <bool NT>
__global__ void k_read(const u32x4* a, int64_t n16, uint32_t* sink) {
  uint32_t acc = 0;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n16; i += (int64_t)gridDim.x * blockDim.x) {
    const u32x4 v = ld16<NT>(a + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;   // keeps the loads alive; practically never stores
}

template <bool NT>
__global__ void k_write(u32x4* a, int64_t n16) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n16; i += (int64_t)gridDim.x * blockDim.x)
    st<NT>(u32x4{(uint32_t)i, 1u, 2u, 3u}, a + i);
}

template <bool NT>
__global__ void k_copy(const u32x4* a, u32x4* b, int64_t n16) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n16; i += (int64_t)gridDim.x * blockDim.x)
    st<NT>(ld16<NT>(a + i), b + i);
}

// The fused kernel's traffic per 8-element chunk: read x and r (16 B each),
// write h and yb (16 B each) and codes (8 B). Grid-stride over chunks.
template <bool NT>
__global__ void k_mix(const u32x4* x, const u32x4* r, u32x4* h, u32x4* yb, u32x2* q, int64_t n16) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n16; i += (int64_t)gridDim.x * blockDim.x) {
    const u32x4 a = ld16<NT>(x + i), b = ld16<NT>(r + i);
    const u32x4 s = a + b;
    st<NT>(s, h + i);
    st<NT>(s ^ a, yb + i);
    st<NT>(u32x2{s[0] ^ s[1], s[2] ^ s[3]}, q + i);
  }
}

// The fused MXFP4 kernel's traffic per 8-element chunk: read x and r (16 B
// each), write h (16 B) and the packed codes (4 B). Grid-stride over chunks.
__global__ void k_mix_fp4(const u32x4* x, const u32x4* r, u32x4* h, uint32_t* q, int64_t n16) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n16; i += (int64_t)gridDim.x * blockDim.x) {
    const u32x4 a = __builtin_nontemporal_load(x + i), b = __builtin_nontemporal_load(r + i);
    const u32x4 s = a + b;
    __builtin_nontemporal_store(s, h + i);
    __builtin_nontemporal_store(s[0] ^ s[1] ^ s[2] ^ s[3], q + i);
  }
}

// Same traffic with the fused kernel's mapping: one workgroup of 64*W lanes
// per row of C chunks, J chunks per lane (chunk c = j*64*W + lane), all loads
// of a row issued before any store; SYNC adds the workgroup barrier the norm's
// cross-wave reduction needs between the two phases.
template <int J, bool SYNC>
__global__ void __launch_bounds__(1024) k_mix_rows(const u32x4* x, const u32x4* r, u32x4* h, u32x4* yb, u32x2* q,
                                                   int32_t M, int32_t C) {
  const int64_t m = blockIdx.x;
  if (m >= M) return;
  const int t = threadIdx.x, T = blockDim.x;
  u32x4 a[J], b[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int c = j * T + t;
    if (c < C) {
      a[j] = __builtin_nontemporal_load(x + m * C + c);
      b[j] = __builtin_nontemporal_load(r + m * C + c);
    }
  }
  if (SYNC) __syncthreads();
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int c = j * T + t;
    if (c < C) {
      const u32x4 s = a[j] + b[j];
      __builtin_nontemporal_store(s, h + m * C + c);
      __builtin_nontemporal_store(s ^ a[j], yb + m * C + c);
      __builtin_nontemporal_store(u32x2{s[0] ^ s[1], s[2] ^ s[3]}, q + m * C + c);
    }
  }
}

// Persistent variant: G workgroups loop over rows m = blockIdx.x, +G, ...,
// with the next row's loads issued before the current row's stores.
template <int J>
__global__ void __launch_bounds__(1024) k_mix_rows_persist(const u32x4* x, const u32x4* r, u32x4* h, u32x4* yb,
                                                           u32x2* q, int32_t M, int32_t C) {
  const int t = threadIdx.x, T = blockDim.x;
  u32x4 a[J], b[J], na[J], nb[J];
  int64_t m = blockIdx.x;
  if (m >= M) return;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int c = j * T + t;
    if (c < C) {
      a[j] = __builtin_nontemporal_load(x + m * C + c);
      b[j] = __builtin_nontemporal_load(r + m * C + c);
    }
  }
  for (; m < M; m += gridDim.x) {
    const int64_t n = m + gridDim.x;
    if (n < M) {
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int c = j * T + t;
        if (c < C) {
          na[j] = __builtin_nontemporal_load(x + n * C + c);
          nb[j] = __builtin_nontemporal_load(r + n * C + c);
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int c = j * T + t;
      if (c < C) {
        const u32x4 s = a[j] + b[j];
        __builtin_nontemporal_store(s, h + m * C + c);
        __builtin_nontemporal_store(s ^ a[j], yb + m * C + c);
        __builtin_nontemporal_store(u32x2{s[0] ^ s[1], s[2] ^ s[3]}, q + m * C + c);
        a[j] = na[j];
        b[j] = nb[j];
      }
    }
  }
}

// Cache-policy variants through buffer instructions (raw buffers, bounds
// checked by the descriptor: out-of-range lanes read 0 and drop stores).
// Policy bits: 1 = sc0, 2 = nt, 16 = sc1.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, 0x00020000);
}

template <int LP, int SP>
__global__ void k_mix_pol(const u32x4* x, const u32x4* r, u32x4* h, u32x4* yb, u32x2* q, int64_t n16) {
  const __amdgpu_buffer_rsrc_t rx = rsrc(x, n16 * 16), rr = rsrc(r, n16 * 16), rh = rsrc(h, n16 * 16),
                               ry = rsrc(yb, n16 * 16), rq = rsrc(q, n16 * 8);
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n16; i += (int64_t)gridDim.x * blockDim.x) {
    const int off = (int)(i * 16);
    const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, LP);
    const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(rr, off, 0, LP);
    const u32x4 s = a + b;
    __builtin_amdgcn_raw_buffer_store_b128(s, rh, off, 0, SP);
    __builtin_amdgcn_raw_buffer_store_b128(s ^ a, ry, off, 0, SP);
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{s[0] ^ s[1], s[2] ^ s[3]}, rq, (int)(i * 8), 0, SP);
  }
}

// Row-mapped (W waves, 2 chunks per lane, C chunks per row) with the policies.
template <int LP, int SP>
__global__ void __launch_bounds__(1024) k_rows_pol(const u32x4* x, const u32x4* r, u32x4* h, u32x4* yb, u32x2* q,
                                                   int32_t M, int32_t C) {
  const int64_t m = blockIdx.x;
  if (m >= M) return;
  const int t = threadIdx.x, T = blockDim.x;
  const int64_t rb = m * C * 16;
  const __amdgpu_buffer_rsrc_t rx = rsrc(x + m * C, C * 16), rr = rsrc(r + m * C, C * 16),
                               rh = rsrc(h + m * C, C * 16), ry = rsrc(yb + m * C, C * 16), rq = rsrc(q + m * C, C * 8);
  (void)rb;
  u32x4 a[2], b[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int c = j * T + t;
    a[j] = __builtin_amdgcn_raw_buffer_load_b128(rx, c * 16, 0, LP);
    b[j] = __builtin_amdgcn_raw_buffer_load_b128(rr, c * 16, 0, LP);
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int c = j * T + t;
    const u32x4 s = a[j] + b[j];
    __builtin_amdgcn_raw_buffer_store_b128(s, rh, c * 16, 0, SP);
    __builtin_amdgcn_raw_buffer_store_b128(s ^ a[j], ry, c * 16, 0, SP);
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{s[0] ^ s[1], s[2] ^ s[3]}, rq, c * 8, 0, SP);
  }
}

// The fused kernel's memory skeleton for one launch plan, with no arithmetic:
// the same grid, row / split / packed-wave mapping, loads (x, gamma, r, in the
// same order, 16 bytes per lane), one cross-wave exchange through LDS with the
// workgroup barrier, and the same stores (h, bf16 rows, codes, one scale per
// group) - the values stored are bit mixes of the inputs. Its time is the
// floor of a launch of that plan: what is left when the statistics, the
// normalization and the quantization cost nothing.
template <int FMT, int J, bool RES, int PACK>
__global__ void __launch_bounds__(64 * rmsq::max_waves(J))
k_plan_floor(int32_t count, int32_t rows, int32_t lg, int32_t slg, int32_t rb1, int32_t rb2, int32_t rb3,
             int32_t threads, int32_t blocks, const rmsq::Launch L) {
  constexpr bool WAVE_ROWS = PACK != rmsq::kPackNone;
  __shared__ uint32_t red[rmsq::kMaxWaves];
  int32_t row, split = 0;
  if constexpr (WAVE_ROWS) {
    const int32_t wave = __builtin_amdgcn_readfirstlane((int32_t)(threadIdx.x >> 6));
    row = rmsq::row_of_block((int32_t)blockIdx.x, blocks, lg) * (threads >> 6) + wave;
    if (row >= rows) return;
  } else {
    const int32_t b = (int32_t)blockIdx.x;
    split = slg > 0 ? (b >> 3) & ((1 << slg) - 1) : 0;
    row = slg > 0 ? ((b >> (3 + slg)) << 3) | (b & 7) : rmsq::row_of_block(b, rows, lg);
    if (row >= rows) return;
  }
  const int pi = (count > 1 && row >= rb1) + (count > 2 && row >= rb2) + (count > 3 && row >= rb3);
  const rmsq::Problem& P = L.p[pi];
  const int32_t u = row - (pi == 0 ? 0 : pi == 1 ? rb1 : pi == 2 ? rb2 : rb3);
  const int lt = PACK == rmsq::kPackLanes ? P.lanes_log2 : 6;
  const int T = PACK == rmsq::kPackLanes ? 1 << lt : WAVE_ROWS ? 64 : threads;
  const int tid = WAVE_ROWS ? (int)(threadIdx.x & (T - 1)) : (int)threadIdx.x;
  int64_t m = u;
  bool live = true;
  if constexpr (PACK == rmsq::kPackLanes) {
    const int32_t r = rmsq::packed_row(u, lt, threadIdx.x & 63);
    live = r < P.M;
    m = live ? r : P.M - 1;
  }
  const int C = P.N >> 3;
  int lo = 0, hi = live ? C : 0;
  if (!WAVE_ROWS && slg > 0) {
    constexpr int q = FMT == 0 ? 16 : 4;
    lo = ((split * (C / q)) >> slg) * q;
    hi = split + 1 == (1 << slg) ? C : (((split + 1) * (C / q)) >> slg) * q;
  }
  const u32x4* xrow = reinterpret_cast<const u32x4*>(P.x + m * P.ldx);
  const u32x4* rrow = RES ? reinterpret_cast<const u32x4*>(P.r + m * P.ldr) : nullptr;
  const u32x4* grow = reinterpret_cast<const u32x4*>(P.gamma);
  u32x4 xv[J], rv[RES ? J : 1], gv[J];
  if constexpr (PACK == rmsq::kPackWave) {
    // as the kernel: one buffer resource per step, from the step to the
    // row's end (steps and lanes past it read zeros, no memory)
    auto ld = [&](const u32x4* row, int j, auto policy) {
      const int done = j * T * 16;
      const __amdgpu_buffer_rsrc_t rs =
          rmsq::buffer_rsrc(reinterpret_cast<const char*>(row) + done, C * 16 > done ? C * 16 - done : 0);
      return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, tid * 16, 0, decltype(policy)::value));
    };
#pragma unroll
    for (int j = 0; j < J; ++j) xv[j] = ld(xrow, j, std::integral_constant<int, rmsq::kBufNontemporal>{});
#pragma unroll
    for (int j = 0; j < J; ++j) gv[j] = ld(grow, j, std::integral_constant<int, 0>{});
    if constexpr (RES) {
#pragma unroll
      for (int j = 0; j < J; ++j) rv[j] = ld(rrow, j, std::integral_constant<int, rmsq::kBufNontemporal>{});
    }
  } else {
#pragma unroll
    for (int j = 0; j < J; ++j) xv[j] = __builtin_nontemporal_load(xrow + min(j * T + tid, C - 1));
#pragma unroll
    for (int j = 0; j < J; ++j) gv[j] = grow[min(j * T + tid, C - 1)];
    if constexpr (RES) {
#pragma unroll
      for (int j = 0; j < J; ++j) rv[j] = __builtin_nontemporal_load(rrow + min(j * T + tid, C - 1));
    }
  }
  uint32_t acc = 0;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    if (RES) xv[j] += rv[j];
    acc ^= xv[j][0] ^ xv[j][3];
  }
  const int nw = T >> 6;
  if (!WAVE_ROWS && nw > 1) {
    if ((tid & 63) == 0) red[tid >> 6] = acc;
    __syncthreads();
    acc = red[(tid >> 6) ^ 1];
  }
  u32x4* ybrow = P.yb ? reinterpret_cast<u32x4*>(P.yb + m * P.ldb) : nullptr;
  u32x4* hrow = RES ? reinterpret_cast<u32x4*>(P.h + m * P.ldr) : nullptr;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int c = j * T + tid;
    if (c < lo || c >= hi) continue;
    if constexpr (RES) __builtin_nontemporal_store(xv[j], hrow + c);
    const u32x4 y = xv[j] ^ gv[j];
    if (ybrow) __builtin_nontemporal_store(y, ybrow + c);
    if constexpr (FMT == 0) {
      __builtin_nontemporal_store(u32x2{y[0] ^ y[1], y[2] ^ acc}, reinterpret_cast<u32x2*>(P.q + m * (int64_t)P.N) + c);
      if ((tid & 15) == 0)
        reinterpret_cast<uint32_t*>(P.scale)[P.layout == 2 ? (c >> 4) * P.M + m : m * (P.N >> 7) + (c >> 4)] = y[3];
    } else {
      __builtin_nontemporal_store(y[0] ^ y[1] ^ acc, reinterpret_cast<uint32_t*>(P.q + m * (int64_t)(P.N >> 1)) + c);
      if ((tid & 3) == 0) {
        const int64_t gcount = P.N >> 5, gi = c >> 2;
        const int64_t off = P.layout == 0   ? m * gcount + gi
                            : P.layout == 1 ? (m >> 5) * (32 * gcount) + gi * 32 + (m & 31)
                                            : gi * P.M + m;
        reinterpret_cast<uint8_t*>(P.scale)[off] = (uint8_t)y[3];
      }
    }
  }
}

__global__ void k_empty(int* p) {
  if (p && threadIdx.x == 1024) p[0] = 0;   // never true: blocks are at most 1024 threads
}

static int st_rc() { return hipGetLastError() == hipSuccess ? 0 : 3; }

// exported: the library is built with hidden visibility
#pragma GCC visibility push(default)
extern "C" {
// kind: 0 read, 1 write, 2 copy, 3 FP8 mix, 4 MXFP4 mix (nontemporal only); nt: nontemporal
// hints; blocks/threads: launch shape.
int stream_probe(int kind, int nt, const void* a, void* b, void* c, void* d, void* e, int64_t n16, int blocks,
                 int threads, void* stream) {
  if (n16 <= 0 || blocks <= 0 || threads <= 0 || threads > 1024) return 1;
  hipStream_t s = (hipStream_t)stream;
  const dim3 g(blocks), t(threads);
  switch (kind * 2 + (nt ? 1 : 0)) {
    case 0: hipLaunchKernelGGL(k_read<false>, g, t, 0, s, (const u32x4*)a, n16, (uint32_t*)b); break;
    case 1: hipLaunchKernelGGL(k_read<true>, g, t, 0, s, (const u32x4*)a, n16, (uint32_t*)b); break;
    case 2: hipLaunchKernelGGL(k_write<false>, g, t, 0, s, (u32x4*)b, n16); break;
    case 3: hipLaunchKernelGGL(k_write<true>, g, t, 0, s, (u32x4*)b, n16); break;
    case 4: hipLaunchKernelGGL(k_copy<false>, g, t, 0, s, (const u32x4*)a, (u32x4*)b, n16); break;
    case 5: hipLaunchKernelGGL(k_copy<true>, g, t, 0, s, (const u32x4*)a, (u32x4*)b, n16); break;
    case 6: hipLaunchKernelGGL(k_mix<false>, g, t, 0, s, (const u32x4*)a, (const u32x4*)b, (u32x4*)c, (u32x4*)d, (u32x2*)e, n16); break;
    case 7: hipLaunchKernelGGL(k_mix<true>, g, t, 0, s, (const u32x4*)a, (const u32x4*)b, (u32x4*)c, (u32x4*)d, (u32x2*)e, n16); break;
    case 9: hipLaunchKernelGGL(k_mix_fp4, g, t, 0, s, (const u32x4*)a, (const u32x4*)b, (u32x4*)c, (uint32_t*)e, n16); break;
    default: return 1;
  }
  return st_rc();
}

// The row-mapped mix: M rows of C chunks, W waves and J chunks per lane
// (J*64*W >= C), optional barrier; persist > 0 launches that many persistent
// workgroups instead of one per row.
int stream_probe_rows(const void* x, const void* r, void* h, void* yb, void* q, int32_t M, int32_t C, int32_t J,
                      int32_t W, int32_t sync, int32_t persist, void* stream) {
  if (M <= 0 || C <= 0 || W < 1 || W > 16 || (int64_t)J * W * 64 < C) return 1;
  const dim3 g(persist > 0 ? persist : M), t(64 * W);
  hipStream_t s = (hipStream_t)stream;
  const u32x4 *X = (const u32x4*)x, *R = (const u32x4*)r;
  u32x4 *H = (u32x4*)h, *Y = (u32x4*)yb;
  u32x2* Q = (u32x2*)q;
#define ROWS(JJ)                                                                         \
  if (J == JJ) {                                                                          \
    if (persist > 0) hipLaunchKernelGGL(k_mix_rows_persist<JJ>, g, t, 0, s, X, R, H, Y, Q, M, C); \
    else if (sync) hipLaunchKernelGGL((k_mix_rows<JJ, true>), g, t, 0, s, X, R, H, Y, Q, M, C); \
    else hipLaunchKernelGGL((k_mix_rows<JJ, false>), g, t, 0, s, X, R, H, Y, Q, M, C);     \
    return st_rc();                                                                       \
  }
  ROWS(1) ROWS(2) ROWS(4) ROWS(7) ROWS(14)
#undef ROWS
  return 1;
}
// Policy probes: lp, sp in {0, 1, 2, 3, 16, 17, 18, 19}; rows > 0 selects the
// row-mapped kernel with W = threads / 64 waves per row (2 chunks per lane).
#define POL_CASE(LP, SP)                                                                                  \
  if (lp == LP && sp == SP) {                                                                             \
    if (rows > 0)                                                                                         \
      hipLaunchKernelGGL((k_rows_pol<LP, SP>), dim3(rows), dim3(threads), 0, s, X, R, H, Y, Q, rows, C);  \
    else                                                                                                  \
      hipLaunchKernelGGL((k_mix_pol<LP, SP>), dim3(blocks), dim3(threads), 0, s, X, R, H, Y, Q, n16);     \
    return st_rc();                                                                                       \
  }
#define POL_ROW(LP) POL_CASE(LP, 0) POL_CASE(LP, 1) POL_CASE(LP, 2) POL_CASE(LP, 3) POL_CASE(LP, 16) POL_CASE(LP, 17) POL_CASE(LP, 18) POL_CASE(LP, 19)
int stream_probe_policy(int lp, int sp, const void* x, const void* r, void* h, void* yb, void* q, int64_t n16,
                        int blocks, int threads, int rows, int C, void* stream) {
  if (n16 <= 0 || threads <= 0 || threads > 1024 || n16 * 16 > 0x7FFFFFFF) return 1;
  if (rows > 0 && ((int64_t)rows * C != n16 || 2 * threads < C)) return 1;
  hipStream_t s = (hipStream_t)stream;
  const u32x4 *X = (const u32x4*)x, *R = (const u32x4*)r;
  u32x4 *H = (u32x4*)h, *Y = (u32x4*)yb;
  u32x2* Q = (u32x2*)q;
  POL_ROW(0) POL_ROW(1) POL_ROW(2) POL_ROW(3) POL_ROW(16) POL_ROW(17) POL_ROW(18) POL_ROW(19)
  return 1;
}
#undef POL_ROW
#undef POL_CASE
// The memory skeleton of one planned launch of the fused kernel (k_plan_floor):
// `problems` as for rmsnorm_quant_group_multi (already validated by the
// library's planner, which produced `info` for exactly these problems: the
// launch's problems are those with M > 0 whose residual presence matches
// info->residual, in order). FP8 or MXFP4 as the problems' fmt; J in 1..4.
int stream_probe_plan_floor(const rmsq_problem* ps, int32_t count, const rmsq_launch_info* info, void* stream) {
  if (!ps || !info || count < 1 || count > 4 || info->chunks_per_lane < 1 || info->chunks_per_lane > 4) return 1;
  rmsq::Launch L{};
  int n = 0;
  int64_t rows = 0;
  for (int i = 0; i < count; ++i) {
    const rmsq_problem& p = ps[i];
    if (p.M == 0 || (p.residual_in != nullptr) != (info->residual != 0)) continue;
    rmsq::Problem& d = L.p[n++];
    d.x = static_cast<const uint16_t*>(p.x);
    d.r = static_cast<const uint16_t*>(p.residual_in);
    d.h = static_cast<uint16_t*>(p.residual_out);
    d.gamma = static_cast<const uint16_t*>(p.gamma);
    d.q = static_cast<uint8_t*>(p.out_q);
    d.scale = p.out_scale;
    d.yb = static_cast<uint16_t*>(p.out_bf16);
    d.ldx = p.ldx ? p.ldx : p.N;
    d.ldr = p.ldr ? p.ldr : p.N;
    d.ldb = p.ldb ? p.ldb : p.N;
    d.M = (int32_t)p.M;
    d.N = (int32_t)p.N;
    d.layout = p.scale_layout;
    d.lanes_log2 = 6;
    L.row_begin[n - 1] = (int32_t)rows;
    rows += p.M;
  }
  if (n != info->problems || rows != info->rows) return 1;
  L.count = n;
  L.rows = (int32_t)rows;
  bool lanes = false;   // rows packed by lanes: the launch counts waves
  if (info->waves_per_workgroup > 1) {
    for (int i = 0; i < n; ++i) {
      const int32_t T = info->lanes_per_row[i];
      if (T != 16 && T != 32 && T != 64) return 1;
      L.p[i].lanes_log2 = T == 16 ? 4 : T == 32 ? 5 : 6;
      lanes |= T < 64;
    }
  }
  if (lanes) {
    if (info->chunks_per_lane != 1) return 1;
    int64_t waves = 0;
    for (int i = 0; i < n; ++i) {
      L.row_begin[i] = (int32_t)waves;
      waves += (L.p[i].M + (64 >> L.p[i].lanes_log2) - 1) >> (6 - L.p[i].lanes_log2);
    }
    L.rows = (int32_t)waves;
  }
  int lg = 0, slg = 0;
  while ((1 << lg) < info->row_group) ++lg;
  while ((1 << slg) < info->row_splits) ++slg;
  L.row_group_log2 = lg;
  L.splits_log2 = slg;
  const dim3 g((unsigned)info->workgroups), t((unsigned)info->threads_per_workgroup);
  const bool packed = info->waves_per_workgroup > 1, res = info->residual != 0, fp4 = ps[0].fmt == 1;
  hipStream_t s = (hipStream_t)stream;
#define FLOOR_ARGS L.count, L.rows, L.row_group_log2, L.splits_log2, L.row_begin[1], L.row_begin[2], L.row_begin[3], \
                   (int32_t)t.x, (int32_t)g.x, L
#define FLOOR_J(F, JJ, R)                                                                             \
  if (info->chunks_per_lane == JJ) {                                                                  \
    if (JJ == 1 && lanes) hipLaunchKernelGGL((k_plan_floor<F, 1, R, rmsq::kPackLanes>), g, t, 0, s, FLOOR_ARGS); \
    else if (packed) hipLaunchKernelGGL((k_plan_floor<F, JJ, R, rmsq::kPackWave>), g, t, 0, s, FLOOR_ARGS);      \
    else hipLaunchKernelGGL((k_plan_floor<F, JJ, R, rmsq::kPackNone>), g, t, 0, s, FLOOR_ARGS);                  \
    return st_rc();                                                                                   \
  }
#define FLOOR_F(F, R) FLOOR_J(F, 1, R) FLOOR_J(F, 2, R) FLOOR_J(F, 3, R) FLOOR_J(F, 4, R)
  if (!fp4 && res) { FLOOR_F(0, true) }
  if (!fp4 && !res) { FLOOR_F(0, false) }
  if (fp4 && res) { FLOOR_F(1, true) }
  if (fp4 && !res) { FLOOR_F(1, false) }
#undef FLOOR_F
#undef FLOOR_J
#undef FLOOR_ARGS
  return 1;
}
// An empty kernel: the launch-overhead floor of back-to-back launches.
int stream_probe_empty(int blocks, int threads, void* stream) {
  if (blocks <= 0 || threads <= 0 || threads > 1024) return 1;
  hipLaunchKernelGGL(k_empty, dim3(blocks), dim3(threads), 0, (hipStream_t)stream, (int*)nullptr);
  return st_rc();
}
}
#pragma GCC visibility pop
