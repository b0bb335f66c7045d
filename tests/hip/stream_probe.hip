// stream_probe.hip - test-only bandwidth probes: plain streams (read, write,
// copy) and the fused kernel's exact traffic pattern with no arithmetic, to
// measure the achievable HBM ceiling of the GPU. Grid-stride loops, bounds
// checked; n16 counts 16-byte elements.
#include <hip/hip_runtime.h>
#include <stdint.h>

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
// An empty kernel: the launch-overhead floor of back-to-back launches.
int stream_probe_empty(int blocks, int threads, void* stream) {
  if (blocks <= 0 || threads <= 0 || threads > 1024) return 1;
  hipLaunchKernelGGL(k_empty, dim3(blocks), dim3(threads), 0, (hipStream_t)stream, (int*)nullptr);
  return st_rc();
}
}
#pragma GCC visibility pop
