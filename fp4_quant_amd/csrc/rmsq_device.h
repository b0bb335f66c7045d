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

// A value the caller never reads, for the operands an instruction requires
// but overwrites: the bits of a packed convert's destination that its next
// convert replaces, and the "old" value of a DPP move whose every lane
// receives a source lane. Left undefined, it costs no register initialization.
__device__ __forceinline__ uint32_t any_u32() { return __builtin_nondeterministic_value(0u); }

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
  return cvt_fp8x2<false>(t, t, any_u32()) & 0xFFu;
}

// ------------------------------------------------------- element blocks --
// The per-chunk arithmetic of the fused kernel, on 8 consecutive elements.

// Low 16 bits of an fp32 within 2 of 0x8000: at most 2 ulps from a bf16
// rounding midpoint of its binade. It contains both windows a row can have
// (below), so the direct fp64 block redoes every element the fast path left
// undecided without keeping the row's window at hand.
__device__ __forceinline__ bool near_bf16_midpoint(float y) {
  return ((__float_as_uint(y) & 0xFFFFu) - 0x7FFEu) <= 4u;
}

// The window of a row, from the sign of inv_lo (inv - inv32 rounded): low
// halves {0x7FFF, 0x8000} when inv32 <= inv, {0x8000, 0x8001} when inv32 > inv.
// Returned as the pair offset that maps the window to {0, 1}: (low 16 bits +
// offset) mod 2^16 <= 1, two 16-bit lanes per dword.
__device__ __forceinline__ uint32_t bf16_window_offset(float inv_lo) {
  return 0x80018001u - (__float_as_uint(inv_lo) >> 31) * 0x00010001u;
}

typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

// Largest |value| of eight packed bf16 (four dwords), as a bf16 magnitude
// pattern: integer max of (bits & 0x7FFF) orders bf16 magnitudes exactly.
__device__ __forceinline__ uint32_t amax8(u32x4 w) {
  const u16x2 a = __builtin_bit_cast(u16x2, w[0] & 0x7FFF7FFFu), b = __builtin_bit_cast(u16x2, w[1] & 0x7FFF7FFFu);
  const u16x2 c = __builtin_bit_cast(u16x2, w[2] & 0x7FFF7FFFu), d = __builtin_bit_cast(u16x2, w[3] & 0x7FFF7FFFu);
  const u16x2 m = __builtin_elementwise_max(__builtin_elementwise_max(a, b), __builtin_elementwise_max(c, d));
  return max((uint32_t)m[0], (uint32_t)m[1]);
}

// A raw buffer resource over `bytes` bytes at p (untyped 32-bit data
// format, no stride): a buffer load whose lane offset is at or past `bytes`
// returns zeros and touches no memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* p, int32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, bytes, 0x00020000);
}
constexpr int kBufNontemporal = 2;   // cache-policy operand of the buffer loads: nt

// The inverse norm inv = 1 / sqrt(d), d = ss/N + eps, as the definition forms
// it in fp64: a correctly rounded square root, then a correctly rounded
// division (0 when d is 0, and for an infinite d). About 30 fp64
// instructions, two of them transcendental; the kernels need it only where
// an element is redone in fp64.
__device__ __forceinline__ double inv_norm64(double d) { return d > 0.0 ? 1.0 / __builtin_sqrt(d) : 0.0; }

// What every element needs from the inverse norm: inv32 = fl32(inv) and
// whether the row takes the exact path for all its elements (inv > 2^16,
// where an h * gamma that underflows to zero in fp32 could still have a
// nonzero bf16 result, or inv < 2^-100), without forming inv itself.
//
// z = 1/sqrt(d) is refined from v_rsq_f64 by two Newton steps
// z' = z + (z/2)(1 - (d z) z), each taking a relative error e to at most
// 1.5 e^2 plus 1.5 units of fp64 rounding (2^-53): from any start within
// 2^-14 (v_rsq_f64 is far closer) to within 2^-27, then within 2^-52.4.
// inv rounds twice, so it is within 2^-52 (1 + 2^-52) of 1/sqrt(d), and
// |z - inv| < 2^-51 z. Rounding to nearest is monotone, so fl32(z) = fl32(inv)
// unless an fp32 rounding midpoint lies within 2^-51 z of z: in z's binade
// [2^k, 2^k+1) the midpoints are where the 29 mantissa bits below fp32
// precision read 2^28, and one unit of those bits is at least 2^-53 z, so
// that can only happen when they lie within 4 of 2^28. Within 32 of it
// (about one row in 10^7) and for d outside (0, inf), inv is formed in full.
// The row test on z is widened by 2^-48 (relative) so that it also holds
// for inv. inv_lo = fl32(z - inv32) is returned too: inv32 + inv_lo is then
// within 2^-51 z + 2^-48 z of inv, which the fp64 path uses to decide most
// elements in fp32.
__device__ __forceinline__ float inv_norm32(double d, bool& row_exact, float& inv_lo) {
  double z = __builtin_amdgcn_rsq(d);
  z = __builtin_fma(0.5 * z, __builtin_fma(-(d * z), z, 1.0), z);
  z = __builtin_fma(0.5 * z, __builtin_fma(-(d * z), z, 1.0), z);
  const uint32_t t = (uint32_t)__double_as_longlong(z) & 0x1FFFFFFFu;
  if (__builtin_expect((t - (0x10000000u - 32u) <= 64u) | !(d > 0.0 && d < __builtin_inf()), 0)) z = inv_norm64(d);
  row_exact = z > 0x1.ffffffffffffcp15 || (z != 0.0 && z < 0x1.0000000000010p-100);
  const float inv32 = (float)z;
  inv_lo = (float)(z - (double)inv32);
  return inv32;
}

// Classes of an fp32 product h * gamma that is not exact or not finite:
// NaN, +-infinity, +-denormal (v_cmp_class_f32 mask). A normal product of two
// bf16 (8 significant bits each) is exact in fp32.
constexpr int kInexactProduct = 0x001 | 0x002 | 0x004 | 0x010 | 0x080 | 0x200;

// bf16(h * g * inv) for 8 elements: h bf16 values (as fp32, and packed two
// per dword in hpk), g the 8 bf16 gammas packed two per dword, inv the fp64
// inverse norm (returned by inv64(), which only the rare fp64 path calls),
// inv32 = fl32(inv) and inv_lo with inv32 + inv_lo within 2^-47.8 inv of inv,
// off the row's window offset (bf16_window_offset(inv_lo)). hg = h * g is
// exact in fp32 unless it leaves the normal range. With a = hg * inv32 and
// inv = inv32 (1 + e), |e| <= 2^-24, the exact product is a + a e, where
// |a e| is under one ulp of y's binade (|a| < 2^24 ulps), and y = fl32(a) is
// within half an ulp of a: |hg inv| - |y| lies in [-1/2, 3/2) ulps when
// e >= 0 and in (-3/2, 1/2] when e <= 0. A y whose low 16 bits are below
// 0x7FFF or above 0x8000 (e >= 0), or below 0x8000 or above 0x8001 (e <= 0),
// therefore rounds to bf16 as the exact product does, and as the fp64 product
// (within 2^-53 of it). The sign of inv_lo picks the window; where it differs
// from that of e, |e| < 2^-50 and either window holds. Elements in the
// window, elements whose hg is denormal or infinite, and every element of a
// row_exact row are redone from h and g (their product is exact there) with a
// single rounding. (A product that underflows to zero is harmless here: the
// caller flags rows with inv > 2^16, and below that a zero hg keeps the sign
// of a true result that rounds to zero in bf16 anyway.) The window test runs
// on packed 16-bit lanes: the low halves of two products side by side
// (v_perm_b32), plus off modulo 2^16, fall in [0, 1] exactly for the window's
// two values; the minimum over the 8 elements decides whether any of them
// needs the rare path.
//
// am: the largest |result| as a bf16 magnitude pattern (what amax8 gives for
// the returned words). Rounding to nearest is monotone and symmetric, so on
// the fast path it is the bf16 of the largest |y| (one v_max3_f32 with
// absolute-value operands per pair, one convert); the fp64 path takes it from
// the final words.
template <bool SPLIT = true, class Inv64>
__device__ __forceinline__ u32x4 norm_bf16x8(const float h[8], const u32x4 hpk, const u32x4 g, float inv32,
                                             float inv_lo, uint32_t off, Inv64 inv64, bool row_exact,
                                             uint32_t& am) {
  u32x4 yw;
  u16x2 lo_min = {0xFFFFu, 0xFFFFu};
  u16x2 tw[4];   // per pair: (low 16 bits + off) mod 2^16, at most 1 in the window
  bool odd = row_exact;
  float ymax;
  // the class mask as a scalar operand (a literal would be rematerialized in
  // a vector register for every call)
  int cls = kInexactProduct;
  asm("" : "+s"(cls));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float hg0 = h[2 * i] * bf16_lo(g[i]), hg1 = h[2 * i + 1] * bf16_hi(g[i]);
    odd |= __builtin_amdgcn_classf(hg0, cls) | __builtin_amdgcn_classf(hg1, cls);
    const float y0 = hg0 * inv32, y1 = hg1 * inv32;
    const uint32_t lows = __builtin_amdgcn_perm(__float_as_uint(y1), __float_as_uint(y0), 0x05040100u);
    tw[i] = __builtin_bit_cast(u16x2, lows) + __builtin_bit_cast(u16x2, off);
    lo_min = __builtin_elementwise_min(lo_min, tw[i]);
    ymax = i == 0 ? __builtin_fmaxf(__builtin_fabsf(y0), __builtin_fabsf(y1))
                  : __builtin_fmaxf(__builtin_fmaxf(ymax, __builtin_fabsf(y0)), __builtin_fabsf(y1));
    yw[i] = pack_bf16(y0, y1);
  }
  am = pack_bf16(ymax, 0.0f);
  const bool need = odd | (min((uint32_t)lo_min[0], (uint32_t)lo_min[1]) <= 1u);
  if (__builtin_expect(need, 0)) {   // rare: keep the fast path's code contiguous
    // Rare: recompute the products here instead of keeping the fast path's
    // 16 intermediates alive across the branch (the empty asm hides that
    // they are the same values, so the compiler does not hold them in
    // registers for the whole phase).
    //
    // In a wave with no flagged row or product, an element taken for its
    // midpoint window (2^-100 <= |y| < 2^127) is decided in fp32 first (SPLIT):
    // with M the bf16 midpoint next to y = fl32(hg inv32) (the same upper 16
    // bits, low half 0x8000), D = (y - M) + (t1 + t2), t1 = fma(hg, inv32, -y)
    // the product's exact residual and t2 = hg inv_lo, equals hg inv - M to
    // within 2^-45.9 |y| before its own last rounding, which keeps its sign
    // (inv32 + inv_lo within 2^-47.8 inv of inv; t2 and t1 + t2 round once,
    // to within 2^-48 |y| and 2^-47 |y|; y - M and t1 are exact), and the
    // definition's fp64 Y lies within 2^-53 |y| of hg inv. So where
    // |D| > 2^-45 |M| (|M| within 2^-7 of |y|) the
    // sign of D says on which side of M Y lies: the upper bf16 (away from
    // zero) when D has y's sign, the lower otherwise. The rest - ties, near
    // ties, extreme magnitudes - are redone in fp64 from h and g (their
    // product is exact there) with a single rounding of h g inv, and only then
    // is inv formed (about 30 dependent fp64 instructions that the waves
    // entering this block, the last to finish a launch, would otherwise all
    // wait for). Waves with a flagged lane, and kernels that keep the
    // smaller code (SPLIT false: where the larger block would spill, or on
    // bandwidth-bound rows, where it gains nothing), take the direct block:
    // inv formed at once, every element needing it redone in fp64.
    if (SPLIT && !__builtin_amdgcn_ballot_w64(odd)) {
      // No lane has a flagged product or row: only window elements, read off
      // the fast path's test values, so that a section costs one compare
      // (the waves entering this block finish last, and its length is what
      // the short launches wait for). A flagged lane anywhere in the wave
      // takes the direct block below.
      u32x4 gr = g, hr = hpk;
      float ir = inv32, il = inv_lo;
      asm volatile("" : "+v"(gr), "+v"(hr), "+v"(ir), "+v"(il));
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if ((uint32_t)tw[e >> 1][e & 1] <= 1u) {
          const float ge = (e & 1) ? bf16_hi(gr[e >> 1]) : bf16_lo(gr[e >> 1]);
          const float he = (e & 1) ? bf16_hi(hr[e >> 1]) : bf16_lo(hr[e >> 1]);
          const float hg = he * ge;
          const float y = hg * ir;
          uint32_t b;
          bool done = false;
          const float ay = __builtin_fabsf(y);
          if (ay >= 0x1p-100f && ay < 0x1p127f) {
            const float M = __uint_as_float((__float_as_uint(y) & 0xFFFF0000u) | 0x8000u);
            const float D = (y - M) + (__builtin_fmaf(hg, ir, -y) + hg * il);
            if (__builtin_fabsf(D) > 0x1p-45f * __builtin_fabsf(M)) {
              b = (__float_as_uint(y) >> 16) + ((__float_as_uint(D) ^ __float_as_uint(y)) >> 31 ? 0u : 1u);
              done = true;
            }
          }
          if (!done) b = bf16_from_f64((double)he * (double)ge * inv64());
          const int sh = (e & 1) * 16;
          yw[e >> 1] = (yw[e >> 1] & ~(0xFFFFu << sh)) | (b << sh);
        }
      }
    } else {
      double inv = inv64();
      u32x4 gr = g, hr = hpk;
      float ir = inv32;
      asm volatile("" : "+v"(gr), "+v"(hr), "+v"(ir), "+v"(inv));
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
    am = amax8(yw);
  }
  return yw;
}

// FP8 scale of a group from its amax (a bf16 magnitude pattern): amax / 448
// rounded once to fp32, 1.0 for an all-zero group. For amax >= 2^-100 it is
// formed in fp32 by one division refinement step: q0 = fl32(amax * c) with
// c = fl32(1/448) is within an ulp of the quotient, the residual
// amax - 448 q0 is exact in one fma, and q0 + residual * c rounded once (a
// second fma) is the correctly rounded amax / 448 - for every bf16 amax in
// that range, checked exhaustively (a CPU test, and the GPU probe of this
// function). (amax has 8 significant bits, so amax/448 = (A/7) 2^k, whose
// bits past any rounding position repeat with period 3 and never come within
// 2^-27 (relative) of an fp32 midpoint unless 7 divides A and the quotient is
// exact.) Smaller amax uses the IEEE fp32 division (denormals kept).
__device__ __forceinline__ float fp8_scale(uint32_t amax_bits) {
  const float a = __uint_as_float(amax_bits << 16);
  if (__builtin_expect(amax_bits < 0x0D80u, 0)) return amax_bits == 0 ? 1.0f : a / 448.0f;
  constexpr float c = 1.0f / 448.0f;
  const float q0 = a * c;
  return __builtin_fmaf(__builtin_fmaf(-q0, 448.0f, a), c, q0);
}

// e4m3fn codes of v[e] / s for 8 bf16 values v (as fp32) of one group with
// maximum magnitude amax and scale s = fp8_scale(amax) = fl32(amax / 448),
// bytes in element order.
//
// Bracket: rs = v_rcp_f32(s) is within 1 ulp of 1/s for every scale this
// library forms (checked exhaustively on the GPU), so r_lo = rs - 4 ulp <
// 1/s < rs + 4 ulp = r_hi and the nearest-even products v*r_lo and v*r_hi
// bracket v/s within 2^-20. Rounding to e4m3fn is monotone, so where both
// give the same code that code is the rounding of v/s (also across the
// e4m3fn subnormal range). Four codes are compared at once as a dword.
//
// Where they differ, v/s lies within 2^-20 of a rounding midpoint B. v/s is
// R * amax / (448 s) with R = 448 v / amax and |amax / (448 s) - 1| <= 2^-24,
// and for bf16 v and amax, R is either exactly a midpoint or at least 2^-12
// (relative) away from every one (checked for every (v, amax) pair on the
// CPU): so R = B exactly, and v/s = B * amax / (448 s) sits above B when
// 448 s < amax, below it when 448 s > amax, and on it - a tie, which takes
// the even code - when 448 s = amax (amax's mantissa a multiple of 7). The
// sign of fma(s, 448, -amax) is that of the exact difference (a nonzero
// difference is at least 2^-123, no underflow to zero), so one fma per group
// decides every element of it: off a midpoint both brackets agree, and on
// one the upper bracket gives the upper code and the lower the lower. So a
// group with 448 s < amax takes the codes of v*r_hi, one with 448 s > amax
// those of v*r_lo - one product and half a convert per element - and only a
// group with an exact scale (448 s = amax, about one in seven) needs both:
// the two codes are then neighbours of one sign where they differ, c_hi =
// c_lo + 1 in each differing byte, and the even one of the pair is
// (c_lo + c_hi + (c_lo & 1)) / 2 in every byte (where they agree too), one
// v_lerp_u8 per four codes.
// Groups whose scale is below 2^-100 (no normal reciprocal) take the
// double-precision path element by element.
__device__ __forceinline__ u32x2 fp8_codes8(const float v[8], float s, float amax) {
  u32x2 qw;
  if (__builtin_expect(s < 0x1p-100f, 0)) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int sh = (e & 3) * 8;
      const uint32_t b = fp8_exact(v[e], s);
      qw[e >> 2] = e & 3 ? (qw[e >> 2] & ~(0xFFu << sh)) | (b << sh) : b;
    }
    return qw;
  }
  const uint32_t rb = __float_as_uint(__builtin_amdgcn_rcpf(s));
  const float t = __builtin_fmaf(s, 448.0f, -amax);
  const float r = __uint_as_float(rb + (t < 0.0f ? 4u : -4u));   // r_hi or r_lo
  float p[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) p[e] = v[e] * r;
  // The first convert of each dword writes its low half; the high half it
  // keeps is replaced by the second, so the register it starts from is any
  // value that dies here (one of its own operands): no initialization.
  qw[0] = cvt_fp8x2<true>(p[2], p[3], cvt_fp8x2<false>(p[0], p[1], __float_as_uint(p[1])));
  qw[1] = cvt_fp8x2<true>(p[6], p[7], cvt_fp8x2<false>(p[4], p[5], __float_as_uint(p[5])));
  if (t == 0.0f) {   // exact scale: ties take the even code
    const float r_hi = __uint_as_float(rb + 4u);
    float h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) h[e] = v[e] * r_hi;
    u32x2 qh;
    qh[0] = cvt_fp8x2<true>(h[2], h[3], cvt_fp8x2<false>(h[0], h[1], __float_as_uint(h[1])));
    qh[1] = cvt_fp8x2<true>(h[6], h[7], cvt_fp8x2<false>(h[4], h[5], __float_as_uint(h[5])));
#pragma unroll
    for (int k = 0; k < 2; ++k) qw[k] = __builtin_amdgcn_lerp(qw[k], qh[k], qw[k]);
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
  uint32_t w = cvt_fp4x2_bf16<0>(yw[0], byte, any_u32());
  w = cvt_fp4x2_bf16<1>(yw[1], byte, w);
  w = cvt_fp4x2_bf16<2>(yw[2], byte, w);
  w = cvt_fp4x2_bf16<3>(yw[3], byte, w);
  return w;
}

// ---------------------------------------------------------------- lanes --
// Rotate within each row of 16 lanes (DPP row_ror).
template <int N>
__device__ __forceinline__ uint32_t row_ror(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)any_u32(), (int)v, 0x120 + N, 0xF, 0xF, false);
}
// Swap within quads: lane i reads lane i^1 (quad_perm [1,0,3,2]) or i^2 ([2,3,0,1]).
__device__ __forceinline__ uint32_t quad_xor1(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)any_u32(), (int)v, 0xB1, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t quad_xor2(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)any_u32(), (int)v, 0x4E, 0xF, 0xF, false);
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

// DPP row rotation of a double (both halves): lane i of each 16-lane row
// reads lane (i + N) mod 16 of that row. Every lane must be active; with
// bound_ctrl and all rows and banks enabled every lane is written, so no old
// value is needed (and none is copied in).
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)b, CTRL, 0xF, 0xF, true);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(b >> 32), CTRL, 0xF, 0xF, true);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// v + (the same lane of the neighbouring 16-lane row): rows 0 and 1 both get
// r0 + r1, rows 2 and 3 both get r2 + r3 (v_permlane16_swap exchanges the odd
// rows of its first operand with the even rows of its second; with both
// operands v the two results hold r0 r0 r2 r2 and r1 r1 r3 r3).
__device__ __forceinline__ double add_rows16(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const auto lo = __builtin_amdgcn_permlane16_swap((uint32_t)b, (uint32_t)b, false, false);
  const auto hi = __builtin_amdgcn_permlane16_swap((uint32_t)(b >> 32), (uint32_t)(b >> 32), false, false);
  return __builtin_bit_cast(double, ((uint64_t)hi[0] << 32) | lo[0]) +
         __builtin_bit_cast(double, ((uint64_t)hi[1] << 32) | lo[1]);
}

// v + (the same lane of the other 32-lane half): v_permlane32_swap exchanges
// rows 2-3 of its first operand with rows 0-1 of its second, so with both
// operands v the results hold r0 r1 r0 r1 and r2 r3 r2 r3.
__device__ __forceinline__ double add_halves32(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const auto lo = __builtin_amdgcn_permlane32_swap((uint32_t)b, (uint32_t)b, false, false);
  const auto hi = __builtin_amdgcn_permlane32_swap((uint32_t)(b >> 32), (uint32_t)(b >> 32), false, false);
  return __builtin_bit_cast(double, ((uint64_t)hi[0] << 32) | lo[0]) +
         __builtin_bit_cast(double, ((uint64_t)hi[1] << 32) | lo[1]);
}

// Sum over each aligned group of 2^lt lanes (lt = 4, 5 or 6) of a fully
// active wave, in a fixed order: DPP rotations within each 16-lane row
// (addition is commutative, so every lane of a row ends with the same value),
// then rows 0+1 and 2+3, then the two pairs. Every lane gets its group's sum,
// bit-identical across the group.
__device__ __forceinline__ double lanes_sum(double v, int lt) {
  v += dpp_f64<0x128>(v);
  v += dpp_f64<0x124>(v);
  v += dpp_f64<0x122>(v);
  v += dpp_f64<0x121>(v);
  if (lt >= 5) v = add_rows16(v);
  if (lt >= 6) v = add_halves32(v);
  return v;
}

// Sum over the 64 lanes of a wave: (r0 + r1) + (r2 + r3) of the row sums.
__device__ __forceinline__ double wave_sum(double v) { return lanes_sum(v, 6); }

}  // namespace rmsq
