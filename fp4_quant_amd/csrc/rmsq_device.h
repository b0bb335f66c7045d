// rmsq_device.h - device-side number formats and cross-lane helpers for gfx950.
//
// Conversions go through the CDNA4 hardware convert instructions
// (v_cvt_pk_bf16_f32, v_cvt_pk_fp8_f32, v_cvt_scalef32_pk_fp4_bf16), all
// round-to-nearest-even. Where an fp32 intermediate could double-round, the
// value is first rounded to odd in fp32 (f64_to_f32_odd): rounding to odd
// with at least two extra bits and then to nearest even equals a single
// rounding to nearest even (Boldo & Melquiond, "When double rounding is odd").
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rmsq {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// bf16 halves of a packed dword, widened to fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two fp32 -> packed bf16, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// double -> float rounded to odd: the float neighbour of v with an odd last
// bit when v is not a float, v itself otherwise. Overflow gives the largest
// finite float, underflow the least subnormal (both odd), sign kept.
__device__ __forceinline__ float f64_to_f32_odd(double v) {
  float t = (float)v;                       // nearest even
  uint32_t b = __float_as_uint(t);
  double back = (double)t;
  if (back != v && (b & 1u) == 0u) b += (__builtin_fabs(v) > __builtin_fabs(back)) ? 1u : 0xFFFFFFFFu;
  return __uint_as_float(b);
}

// bf16 nearest-even of a double (one rounding): round to odd in fp32, then
// the hardware nearest-even bf16 convert. Returns the 16-bit pattern.
__device__ __forceinline__ uint32_t bf16_from_f64(double v) {
  return pack_bf16(f64_to_f32_odd(v), 0.0f) & 0xFFFFu;
}

// Two fp32 -> two e4m3fn bytes (a in the lower byte), nearest even, written
// into the low (HI_WORD false) or high 16 bits of `old` (v_cvt_pk_fp8_f32;
// gfx950 uses the OCP e4m3fn encoding). The caller keeps |v| < 464 so
// nothing saturates.
template <bool HI_WORD>
__device__ __forceinline__ uint32_t cvt_fp8x2(float a, float b, uint32_t old) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, HI_WORD);
}

// A packed pair of bf16 (low half = even element) -> two e2m1 nibbles (even
// element low) in byte SEL of `old`: v_cvt_scalef32_pk_fp4_bf16, which
// divides by 2^k, k taken from the exponent field of the fp32 scale operand
// (scale bits = e8m0 byte << 23, byte 0 meaning 2^-127), then rounds to
// nearest even and saturates at 6. Checked on the GPU for every e8m0 byte
// and every bf16 value up to twice the largest magnitude a group with that
// byte holds.
template <int SEL>
__device__ __forceinline__ uint32_t cvt_fp4x2_bf16(uint32_t pair, uint32_t byte, uint32_t old) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(old, __builtin_bit_cast(bf16x2, pair), __uint_as_float(byte << 23),
                                                  SEL);
}

// e4m3fn byte of the exact quotient v / s for the rare cases the fast path
// cannot decide: the quotient in double is within 2^-53 relative of the
// exact one, and a non-tie quotient of a bf16 value by an fp32 value sits at
// least 2^-29 relative away from every e4m3fn rounding midpoint, so rounding
// the double (to odd in fp32, then to nearest even in hardware) decides as
// the exact quotient would.
__device__ __forceinline__ uint32_t fp8_exact(float v, float s) {
  float t = f64_to_f32_odd((double)v / (double)s);
  return cvt_fp8x2<false>(t, t, 0u) & 0xFFu;
}

// ------------------------------------------------------- element blocks --
// The per-chunk arithmetic of the fused kernel, on 8 consecutive elements.

__device__ __forceinline__ bool near_bf16_midpoint(float y) {
  return ((__float_as_uint(y) & 0xFFFFu) - 0x7FFCu) <= 8u;
}

typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

// Classes of an fp32 product h * gamma that is not exact or not finite:
// NaN, +-infinity, +-denormal (v_cmp_class_f32 mask). A normal product of two
// bf16 (8 significant bits each) is exact in fp32.
constexpr int kInexactProduct = 0x001 | 0x002 | 0x004 | 0x010 | 0x080 | 0x200;

// bf16(h * g * inv) for 8 elements: h bf16 values (as fp32, and packed two
// per dword in hpk), g the 8 bf16 gammas packed two per dword, inv the fp64
// inverse norm and inv32 = fl32(inv). hg = h * g is exact in fp32 unless it
// leaves the normal range; then y = hg * inv32 is within 2 ulp of the fp64
// product h * g * inv, so its bf16 rounding is final unless y lies within 4
// ulp of a bf16 midpoint. Those elements, elements whose hg is denormal or
// infinite, and every element of a row_exact row are redone in fp64 from h
// and g (their product is exact there) with a single rounding. (A product
// that underflows to zero is harmless here: the caller flags rows with
// inv > 2^16, and below that a zero hg keeps the sign of a true result that
// rounds to zero in bf16 anyway.) The window test runs on packed 16-bit
// lanes: the low halves of two products side by side (v_perm_b32), plus
// 0x8004 modulo 2^16, fall in [0, 8] exactly for the products whose low 16
// bits lie in [0x7FFC, 0x8004]; the minimum over the 8 elements decides
// whether any of them needs the fp64 path.
__device__ __forceinline__ u32x4 norm_bf16x8(const float h[8], const u32x4 hpk, const u32x4 g, float inv32,
                                             double inv, bool row_exact) {
  u32x4 yw;
  u16x2 lo_min = {0xFFFFu, 0xFFFFu};
  bool odd = row_exact;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float hg0 = h[2 * i] * bf16_lo(g[i]), hg1 = h[2 * i + 1] * bf16_hi(g[i]);
    odd |= __builtin_amdgcn_classf(hg0, kInexactProduct) | __builtin_amdgcn_classf(hg1, kInexactProduct);
    const float y0 = hg0 * inv32, y1 = hg1 * inv32;
    const uint32_t lows = __builtin_amdgcn_perm(__float_as_uint(y1), __float_as_uint(y0), 0x05040100u);
    lo_min = __builtin_elementwise_min(lo_min, __builtin_bit_cast(u16x2, lows) + u16x2{0x8004u, 0x8004u});
    yw[i] = pack_bf16(y0, y1);
  }
  const bool need = odd | (min((uint32_t)lo_min[0], (uint32_t)lo_min[1]) <= 8u);
  if (__builtin_expect(need, 0)) {   // rare: keep the fast path's code contiguous
    // Rare: recompute the products here instead of keeping the fast path's
    // 16 intermediates alive across the branch (the empty asm hides that
    // they are the same values, so the compiler does not hold them in
    // registers for the whole phase).
    u32x4 gr = g, hr = hpk;
    float ir = inv32;
    asm volatile("" : "+v"(gr), "+v"(hr), "+v"(ir));
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float ge = (e & 1) ? bf16_hi(gr[e >> 1]) : bf16_lo(gr[e >> 1]);
      const float he = (e & 1) ? bf16_hi(hr[e >> 1]) : bf16_lo(hr[e >> 1]);
      const float hg = he * ge;
      if (row_exact | __builtin_amdgcn_classf(hg, kInexactProduct) | near_bf16_midpoint(hg * ir)) {
        const uint32_t b = bf16_from_f64((double)he * (double)ge * inv);
        const int sh = (e & 1) * 16;
        yw[e >> 1] = (yw[e >> 1] & ~(0xFFFFu << sh)) | (b << sh);
      }
    }
  }
  return yw;
}

// FP8 scale of a group from its amax (a bf16 magnitude pattern): amax / 448
// rounded once to fp32, 1.0 for an all-zero group. For amax >= 2^-100 the
// quotient is a normal fp32 and is formed as fl32(amax * fl64(1/448)): amax
// has 8 significant bits, so amax/448 = (A/7) 2^k, whose bits past any
// rounding position repeat with period 3 and never come within 2^-27
// (relative) of an fp32 midpoint unless 7 divides A and the quotient is
// exact; the fp64 product is within 2^-52 of the quotient, so its fp32
// rounding is the correctly rounded one. Smaller amax uses the IEEE fp32
// division (denormals kept).
__device__ __forceinline__ float fp8_scale(uint32_t amax_bits) {
  const float a = __uint_as_float(amax_bits << 16);
  if (__builtin_expect(amax_bits < 0x0D80u, 0)) return amax_bits == 0 ? 1.0f : a / 448.0f;
  return (float)((double)a * (1.0 / 448.0));
}

// e4m3fn codes of v[e] / s for 8 bf16 values v (as fp32) of one group, bytes
// in element order. rs = v_rcp_f32(s) is within 1 ulp of 1/s for every scale
// this kernel produces (s = fl32(amax/448) for a bf16 amax >= 2^-100; checked
// exhaustively on the GPU), so r_lo = rs - 4 ulp < 1/s < rs + 4 ulp = r_hi,
// and the nearest-even products v*r_lo and v*r_hi bracket v/s. Rounding to
// e4m3fn is monotone, so where both brackets give the same code that code is
// the rounding of v/s (also across the e4m3fn subnormal range); four codes
// are compared at once as a packed dword. Where they differ - quotients
// within a few ulp of a rounding midpoint, exact ties - the two codes are
// neighbours (the brackets are 8 fp32 ulp apart, e4m3fn codes at least 2^-4
// relative), and v/s is compared with the boundary B between them: B has few
// significant bits (1.ffff1 x 2^E in the normal range, (k + 1/2) 2^-9 in the
// subnormal one: min(4, E + 10) fraction bits at its exponent E), and |x_hi|
// exceeds it by less than the next such bit, so clearing |x_hi|'s lower
// fraction bits gives B exactly; fma(B, s, -|v|) rounds once, so its sign is
// that of B s - |v| and it is zero only at an exact tie (for s >= 2^-100 the
// difference is a multiple of 2^-140, representable), which takes the code
// with the even mantissa. With bf16 inputs this is not rare - exact ties come
// with every group whose amax mantissa is a multiple of 7 - so it must not
// cost a branch per element. MODE picks the form (each measured best where
// it is used): kFp8Straight, one straight block over the 8 elements (the
// fused kernel's short rows); kFp8Rounds, one differing element per lane per
// round, the wave looping while any lane has one left (the GEMMs, where each
// lane encodes 32 elements); kFp8PerElement, each differing element on the
// double-precision path under its own branch (the long-row kernels, short of
// registers). Groups whose scale is too small for a normal reciprocal take
// the double-precision path.
enum Fp8Fix { kFp8PerElement = 0, kFp8Straight = 1, kFp8Rounds = 2 };

// The rounding boundary between the neighbouring codes of x_hi's bracket and
// the decision against it: 1 when v/s lies above the boundary or on it with
// c_lo odd (then the code is c_lo + 1), else 0.
__device__ __forceinline__ uint32_t fp8_round_up(float v, float x_hi, float s, uint32_t c_lo) {
  const uint32_t xb = __float_as_uint(x_hi) & 0x7FFFFFFFu;
  const int keep = max(0, min(4, (int)(xb >> 23) - 117));
  const float B = __uint_as_float(xb & ~((1u << (23 - keep)) - 1u));
  const float t = __builtin_fmaf(B, s, -__builtin_fabsf(v));
  return (uint32_t)(t < 0.0f) | ((uint32_t)(t == 0.0f) & (c_lo & 1u));
}

template <int MODE = kFp8Straight>
__device__ __forceinline__ u32x2 fp8_codes8(const float v[8], float s) {
  const uint32_t rb = __float_as_uint(__builtin_amdgcn_rcpf(s));
  const float r_lo = __uint_as_float(rb - 4u), r_hi = __uint_as_float(rb + 4u);
  float lo[8], hi[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    lo[e] = v[e] * r_lo;
    hi[e] = v[e] * r_hi;
  }
  u32x2 qw, qh;
  qw[0] = cvt_fp8x2<true>(lo[2], lo[3], cvt_fp8x2<false>(lo[0], lo[1], 0u));
  qw[1] = cvt_fp8x2<true>(lo[6], lo[7], cvt_fp8x2<false>(lo[4], lo[5], 0u));
  qh[0] = cvt_fp8x2<true>(hi[2], hi[3], cvt_fp8x2<false>(hi[0], hi[1], 0u));
  qh[1] = cvt_fp8x2<true>(hi[6], hi[7], cvt_fp8x2<false>(hi[4], hi[5], 0u));
  const bool tiny = s < 0x1p-100f;
  if (MODE == kFp8PerElement || __builtin_expect(tiny, 0)) {
    if (__builtin_expect(tiny | (qw[0] != qh[0]) | (qw[1] != qh[1]), 0)) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int sh = (e & 3) * 8;
        if (tiny | ((((qw[e >> 2] ^ qh[e >> 2]) >> sh) & 0xFFu) != 0u)) {
          const uint32_t b = fp8_exact(v[e], s);
          qw[e >> 2] = (qw[e >> 2] & ~(0xFFu << sh)) | (b << sh);
        }
      }
    }
  } else if (__builtin_expect((qw[0] != qh[0]) | (qw[1] != qh[1]), 0)) {
    // c_hi = c_lo + 1 where the codes differ (neighbours of one sign, no carry)
    if constexpr (MODE == kFp8Straight) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int sh = (e & 3) * 8;
        const uint32_t c_lo = (qw[e >> 2] >> sh) & 0xFFu, c_hi = (qh[e >> 2] >> sh) & 0xFFu;
        qw[e >> 2] += ((c_lo != c_hi) ? fp8_round_up(v[e], hi[e], s, c_lo) : 0u) << sh;
      }
    } else {
      uint32_t dm = 0;   // elements whose bracket codes differ
#pragma unroll
      for (int e = 0; e < 8; ++e)
        dm |= (uint32_t)((((qw[e >> 2] ^ qh[e >> 2]) >> ((e & 3) * 8)) & 0xFFu) != 0u) << e;
      while (__any(dm != 0u)) {   // at most 8 rounds: each clears a bit of every lane that has one
        if (dm != 0u) {
          const int e = __builtin_ctz(dm);
          dm &= dm - 1u;
          float ve = v[0], he = hi[0];
#pragma unroll
          for (int k = 1; k < 8; ++k) {
            ve = e == k ? v[k] : ve;
            he = e == k ? hi[k] : he;
          }
          const int sh = (e & 3) * 8;
          const uint32_t up = fp8_round_up(ve, he, s, ((e < 4 ? qw[0] : qw[1]) >> sh) & 0xFFu);
          if (e < 4) qw[0] += up << sh;
          else qw[1] += up << sh;
        }
      }
    }
  }
  return qw;
}

// MXFP4 e8m0 scale byte of a group from its amax (bf16 magnitude pattern):
// e = floor(log2 amax) - 2 clamped to [-127, 127], byte = e + 127, which is
// the bf16 exponent field of amax minus 2 (0 for subnormal amax), and 127
// (scale 1) for an all-zero group.
__device__ __forceinline__ uint32_t mx_scale_byte(uint32_t amax_bits) {
  const uint32_t E = amax_bits >> 7;
  return amax_bits == 0 ? 127u : (E >= 2u ? E - 2u : 0u);
}

// e2m1 codes of yb[e] / 2^(byte-127) for 8 bf16 values packed two per dword
// (the division by a power of two is exact), packed two per byte with the
// even element in the low nibble.
__device__ __forceinline__ uint32_t fp4_codes8(const u32x4 yw, uint32_t byte) {
  uint32_t w = cvt_fp4x2_bf16<0>(yw[0], byte, 0u);
  w = cvt_fp4x2_bf16<1>(yw[1], byte, w);
  w = cvt_fp4x2_bf16<2>(yw[2], byte, w);
  w = cvt_fp4x2_bf16<3>(yw[3], byte, w);
  return w;
}

// ---------------------------------------------------------------- lanes --
// Rotate within each row of 16 lanes (DPP row_ror).
template <int N>
__device__ __forceinline__ uint32_t row_ror(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x120 + N, 0xF, 0xF, false);
}
// Swap within quads: lane i reads lane i^1 (quad_perm [1,0,3,2]) or i^2 ([2,3,0,1]).
__device__ __forceinline__ uint32_t quad_xor1(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t quad_xor2(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);
}

// max over the 16 lanes of a DPP row; every lane of the row gets the result.
__device__ __forceinline__ uint32_t max16(uint32_t v) {
  v = max(v, row_ror<8>(v));
  v = max(v, row_ror<4>(v));
  v = max(v, row_ror<2>(v));
  v = max(v, row_ror<1>(v));
  return v;
}
// max over a quad of lanes.
__device__ __forceinline__ uint32_t max4(uint32_t v) {
  v = max(v, quad_xor1(v));
  v = max(v, quad_xor2(v));
  return v;
}

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, CTRL, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), CTRL, 0xF, 0xF, false);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ double readlane_f64(double v, int lane) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, lane);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), lane);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Sum over the 64 lanes of a (fully active) wave in a fixed order: DPP
// rotations within each 16-lane row (addition is commutative, so every lane of
// a row ends with the same value), then the four row sums in a fixed tree.
// The result is wave-uniform.
__device__ __forceinline__ double wave_sum(double v) {
  v += dpp_f64<0x128>(v);
  v += dpp_f64<0x124>(v);
  v += dpp_f64<0x122>(v);
  v += dpp_f64<0x121>(v);
  return (readlane_f64(v, 0) + readlane_f64(v, 16)) + (readlane_f64(v, 32) + readlane_f64(v, 48));
}

// Largest |value| of eight packed bf16 (four dwords), as a bf16 magnitude
// pattern: integer max of (bits & 0x7FFF) orders bf16 magnitudes exactly.
__device__ __forceinline__ uint32_t amax8(u32x4 w) {
  const u16x2 a = __builtin_bit_cast(u16x2, w[0] & 0x7FFF7FFFu), b = __builtin_bit_cast(u16x2, w[1] & 0x7FFF7FFFu);
  const u16x2 c = __builtin_bit_cast(u16x2, w[2] & 0x7FFF7FFFu), d = __builtin_bit_cast(u16x2, w[3] & 0x7FFF7FFFu);
  const u16x2 m = __builtin_elementwise_max(__builtin_elementwise_max(a, b), __builtin_elementwise_max(c, d));
  return max((uint32_t)m[0], (uint32_t)m[1]);
}

}  // namespace rmsq
