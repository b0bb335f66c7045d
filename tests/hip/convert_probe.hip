// convert_probe.hip - test-only library: runs the fused kernel's per-element
// number helpers (fp4_quant_amd/csrc/rmsq_device.h) and the raw gfx950
// convert instructions on arrays, so that tests can compare them with the CPU
// oracle over exhaustive and adversarial inputs. Every kernel is a bounds-
// checked grid-stride loop over n items.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rmsq_device.h"

using namespace rmsq;

#define GRID_LOOP(i, n) \
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < (n); i += (int64_t)gridDim.x * blockDim.x)

__global__ void k_norm_bf16(const float* hv, const float* gv, const double* inv, const uint8_t* row_exact,
                            uint16_t* out, uint16_t* am_out, int64_t n) {
  GRID_LOOP(k, n) {
    float h[8];
    u32x4 hp, g;
    for (int e = 0; e < 8; ++e) h[e] = hv[8 * k + e];
    for (int i = 0; i < 4; ++i) {   // h and gamma are bf16 values: their fp32 patterns' high halves
      hp[i] = (__float_as_uint(hv[8 * k + 2 * i]) >> 16) | (__float_as_uint(hv[8 * k + 2 * i + 1]) & 0xFFFF0000u);
      g[i] = (__float_as_uint(gv[8 * k + 2 * i]) >> 16) | (__float_as_uint(gv[8 * k + 2 * i + 1]) & 0xFFFF0000u);
    }
    uint32_t am;
    const float lo = (float)(inv[k] - (double)(float)inv[k]);
    const u32x4 w = norm_bf16x8(h, hp, g, (float)inv[k], lo, bf16_window_offset(lo), [&] { return inv[k]; },
                                row_exact[k] != 0, am);
    for (int e = 0; e < 8; ++e) out[8 * k + e] = (uint16_t)(w[e >> 1] >> ((e & 1) * 16));
    am_out[k] = (uint16_t)am;
  }
}

// the fused kernels' fl32 of the inverse norm of d, and their row test
__global__ void k_inv_norm(const double* d, float* inv32, uint8_t* row_exact, int64_t n) {
  GRID_LOOP(i, n) {
    bool ex;
    float lo;
    inv32[i] = inv_norm32(d[i], ex, lo);
    row_exact[i] = ex;
  }
}

__global__ void k_fp8_scale(const uint16_t* amax, float* s, int64_t n) {
  GRID_LOOP(i, n) s[i] = fp8_scale(amax[i]);
}

// codes of 8 values of a group with maximum magnitude amax[k] (bf16 bits),
// under the scale the kernels form for it
__global__ void k_fp8_codes(const float* v, const uint16_t* amax, uint8_t* out, int64_t n) {
  GRID_LOOP(k, n) {
    float x[8];
    for (int e = 0; e < 8; ++e) x[e] = v[8 * k + e];
    const uint32_t a = amax[k];
    const u32x2 q = fp8_codes8(x, fp8_scale(a), __uint_as_float(a << 16));
    for (int e = 0; e < 8; ++e) out[8 * k + e] = (uint8_t)(q[e >> 2] >> ((e & 3) * 8));
  }
}

__global__ void k_mx_byte(const uint16_t* amax, uint8_t* out, int64_t n) {
  GRID_LOOP(i, n) out[i] = (uint8_t)mx_scale_byte(amax[i]);
}

__global__ void k_fp4_codes(const uint16_t* v, const uint8_t* byte, uint32_t* out, int64_t n) {
  GRID_LOOP(k, n) {
    u32x4 w;
    for (int i = 0; i < 4; ++i) w[i] = (uint32_t)v[8 * k + 2 * i] | ((uint32_t)v[8 * k + 2 * i + 1] << 16);
    out[k] = fp4_codes8(w, byte[k]);
  }
}

__global__ void k_cvt_bf16(const float* in, uint16_t* out, int64_t n) {
  GRID_LOOP(i, n) out[i] = (uint16_t)(pack_bf16(in[i], 0.0f) & 0xFFFFu);
}

__global__ void k_cvt_fp8(const float* in, uint8_t* out, int64_t n) {  // n pairs
  GRID_LOOP(k, n) {
    const uint32_t w = cvt_fp8x2<true>(in[2 * k], in[2 * k + 1], cvt_fp8x2<false>(in[2 * k + 1], in[2 * k], 0u));
    out[4 * k + 0] = (uint8_t)w;          // low word: (b, a)
    out[4 * k + 1] = (uint8_t)(w >> 8);
    out[4 * k + 2] = (uint8_t)(w >> 16);  // high word: (a, b)
    out[4 * k + 3] = (uint8_t)(w >> 24);
  }
}

__global__ void k_cvt_fp4(const float* in, uint8_t* out, int64_t n) {  // n groups of 8
  GRID_LOOP(k, n) {
    const float* a = in + 8 * k;
    // the plain (fp32-input) hardware convert with scale 1
    uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, a[0], a[1], 1.0f, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, a[2], a[3], 1.0f, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, a[4], a[5], 1.0f, 2);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, a[6], a[7], 1.0f, 3);
    for (int b = 0; b < 4; ++b) out[4 * k + b] = (uint8_t)(w >> (8 * b));
  }
}

__global__ void k_f64_to_bf16(const double* in, uint16_t* out, int64_t n) {
  GRID_LOOP(i, n) out[i] = (uint16_t)bf16_from_f64(in[i]);
}

__global__ void k_fp8_exact(const float* v, const float* s, uint8_t* out, int64_t n) {
  GRID_LOOP(i, n) out[i] = (uint8_t)fp8_exact(v[i], s[i]);
}

__global__ void k_rcp(const float* s, float* out, int64_t n) {
  GRID_LOOP(i, n) out[i] = __builtin_amdgcn_rcpf(s[i]);
}

// Raw scaled converts of packed bf16 pairs (v_cvt_scalef32_pk_fp4_bf16 /
// v_cvt_scalef32_pk_fp8_bf16) with a per-pair fp32 scale operand: the tests
// pin down how the scale operand enters the result.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short s16x2_t __attribute__((ext_vector_type(2)));

__global__ void k_cvt_fp4_bf16_scaled(const uint32_t* pairs, const float* scale, uint8_t* out, int64_t n) {
  GRID_LOOP(k, n) {
    const uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(0u, __builtin_bit_cast(bf16x2_t, pairs[k]), scale[k], 0);
    out[k] = (uint8_t)w;
  }
}

__global__ void k_cvt_fp8_bf16_scaled(const uint32_t* pairs, const float* scale, uint16_t* out, int64_t n) {
  GRID_LOOP(k, n) {
    const s16x2_t w = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(s16x2_t{0, 0}, __builtin_bit_cast(bf16x2_t, pairs[k]),
                                                               scale[k], false);
    out[k] = (uint16_t)w[0];
  }
}

// One v_mfma_scale_f32_16x16x128_f8f6f4 with e2m1 A and B per wave, on raw
// lane registers from the host: wave w reads a, b [w][lane][4 dwords], the
// e8m0 scale registers sa, sb [w][lane] and writes d [w][lane][4]. One wave
// per 64-thread block; the tests pin the operand and result layouts.
typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef float v4f_t __attribute__((ext_vector_type(4)));

__global__ void k_mfma_scale_fp4(const uint32_t* a, const uint32_t* b, const uint32_t* sa, const uint32_t* sb, float* d,
                                 int64_t waves) {
  const int64_t w = blockIdx.x;
  if (w >= waves) return;
  const int l = threadIdx.x;
  const int64_t o = (w * 64 + l) * 4;
  v8i_t av = {(int)a[o], (int)a[o + 1], (int)a[o + 2], (int)a[o + 3], 0, 0, 0, 0};
  v8i_t bv = {(int)b[o], (int)b[o + 1], (int)b[o + 2], (int)b[o + 3], 0, 0, 0, 0};
  const v4f_t c = {0.0f, 0.0f, 0.0f, 0.0f};
  const v4f_t r = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 4, 4, 0, (int)sa[w * 64 + l], 0,
                                                                 (int)sb[w * 64 + l]);
  for (int i = 0; i < 4; ++i) d[o + i] = r[i];
}

// The same instruction with e4m3fn A and B (cbsz = blgp = 0): wave w reads
// a, b [w][lane][8 dwords] and the scale registers sa, sb [w][lane].
__global__ void k_mfma_scale_fp8(const uint32_t* a, const uint32_t* b, const uint32_t* sa, const uint32_t* sb, float* d,
                                 int64_t waves) {
  const int64_t w = blockIdx.x;
  if (w >= waves) return;
  const int l = threadIdx.x;
  const int64_t o = (w * 64 + l) * 8;
  v8i_t av, bv;
  for (int i = 0; i < 8; ++i) {
    av[i] = (int)a[o + i];
    bv[i] = (int)b[o + i];
  }
  const v4f_t c = {0.0f, 0.0f, 0.0f, 0.0f};
  const v4f_t r = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 0, 0, 0, (int)sa[w * 64 + l], 0,
                                                                 (int)sb[w * 64 + l]);
  for (int i = 0; i < 4; ++i) d[(w * 64 + l) * 4 + i] = r[i];
}

static int launch_status() { return hipGetLastError() == hipSuccess ? 0 : 3; }

#define GRID(n) dim3((unsigned)(((n) + 255) / 256 < 65536 ? ((n) + 255) / 256 : 65536)), dim3(256), 0, (hipStream_t)stream

// exported: the library is built with hidden visibility
#pragma GCC visibility push(default)
extern "C" {
int probe_norm_bf16(const float* h, const float* g, const double* inv, const uint8_t* ex, uint16_t* out,
                    uint16_t* am, int64_t n, void* stream) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(k_norm_bf16, GRID(n), h, g, inv, ex, out, am, n);
  return launch_status();
}
int probe_inv_norm(const double* d, float* inv32, uint8_t* ex, int64_t n, void* stream) {
  hipLaunchKernelGGL(k_inv_norm, GRID(n), d, inv32, ex, n);
  return (int)hipGetLastError();
}
int probe_fp8_scale(const uint16_t* a, float* s, int64_t n, void* stream) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(k_fp8_scale, GRID(n), a, s, n);
  return launch_status();
}
int probe_fp8_codes(const float* v, const uint16_t* amax, uint8_t* out, int64_t n, void* stream) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(k_fp8_codes, GRID(n), v, amax, out, n);
  return launch_status();
}
int probe_mx_byte(const uint16_t* a, uint8_t* out, int64_t n, void* stream) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(k_mx_byte, GRID(n), a, out, n);
  return launch_status();
}
int probe_fp4_codes(const uint16_t* v, const uint8_t* b, uint32_t* out, int64_t n, void* stream) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(k_fp4_codes, GRID(n), v, b, out, n);
  return launch_status();
}
int probe_cvt_bf16(const float* in, uint16_t* out, int64_t n, void* stream) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(k_cvt_bf16, GRID(n), in, out, n);
  return launch_status();
}
int probe_cvt_fp8(const float* in, uint8_t* out, int64_t n, void* stream) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(k_cvt_fp8, GRID(n), in, out, n);
  return launch_status();
}
int probe_cvt_fp4(const float* in, uint8_t* out, int64_t n, void* stream) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(k_cvt_fp4, GRID(n), in, out, n);
  return launch_status();
}
int probe_f64_to_bf16(const double* in, uint16_t* out, int64_t n, void* stream) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(k_f64_to_bf16, GRID(n), in, out, n);
  return launch_status();
}
int probe_rcp(const float* s, float* out, int64_t n, void* stream) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(k_rcp, GRID(n), s, out, n);
  return launch_status();
}
int probe_cvt_fp4_bf16_scaled(const uint32_t* pairs, const float* scale, uint8_t* out, int64_t n, void* stream) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(k_cvt_fp4_bf16_scaled, GRID(n), pairs, scale, out, n);
  return launch_status();
}
int probe_cvt_fp8_bf16_scaled(const uint32_t* pairs, const float* scale, uint16_t* out, int64_t n, void* stream) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(k_cvt_fp8_bf16_scaled, GRID(n), pairs, scale, out, n);
  return launch_status();
}
int probe_mfma_scale_fp4(const uint32_t* a, const uint32_t* b, const uint32_t* sa, const uint32_t* sb, float* d,
                         int64_t waves, void* stream) {
  if (waves <= 0) return 0;
  hipLaunchKernelGGL(k_mfma_scale_fp4, dim3((unsigned)waves), dim3(64), 0, (hipStream_t)stream, a, b, sa, sb, d, waves);
  return launch_status();
}
int probe_mfma_scale_fp8(const uint32_t* a, const uint32_t* b, const uint32_t* sa, const uint32_t* sb, float* d,
                         int64_t waves, void* stream) {
  if (waves <= 0) return 0;
  hipLaunchKernelGGL(k_mfma_scale_fp8, dim3((unsigned)waves), dim3(64), 0, (hipStream_t)stream, a, b, sa, sb, d, waves);
  return launch_status();
}
int probe_fp8_exact(const float* v, const float* s, uint8_t* out, int64_t n, void* stream) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(k_fp8_exact, GRID(n), v, s, out, n);
  return launch_status();
}
}
#pragma GCC visibility pop
