"""The fused kernel rounds y = h * gamma * inv to bf16 from the fp32 product
y32 = fl32(fl32(h * gamma) * inv32), inv32 = fl32(inv), and redoes the element
only when the low 16 bits of y32 fall in a window of two values that each row
picks from the sign of inv_lo = fl32(z - inv32) (z the refined reciprocal
square root, within 2^-51 z of inv): {0x7FFF, 0x8000} when inv_lo >= 0,
{0x8000, 0x8001} when inv_lo < 0.

The bound behind that window: h * gamma is exact in fp32 (two 8-bit
significands). With a = hg * inv32 and eps = (inv - inv32) / inv32
(|eps| <= 2^-24), the exact product is a (1 + eps), and |a| eps is under one
ulp of y32's binade (|a| < 2^24 ulps); y32 = fl32(a) is within half an ulp
of a. So |hg inv| - |y32| lies in [-1/2, 3/2) ulps when eps >= 0 and in
(-3/2, 1/2] when eps <= 0: a y32 below 0x7FFF or above 0x8000 (eps >= 0), or
below 0x8000 or above 0x8001 (eps <= 0), rounds to the same bf16 as the
exact product, and as the double product the definition rounds (within
2^-53 of it). Where inv_lo has the other sign than eps, |eps| < 2^-50 and
either window holds.

This CPU test checks that with the same IEEE binary32 / binary64 operations:
random bf16 pairs with products in the normal range; double inverse norms
chosen to put the exact product within a few fp32 ulps of a bf16 midpoint
(every mantissa, the top of the binade oversampled, where an ulp is smallest
relative to the value); random inverse norms; and inverse norms within a few
fp64 ulps of an fp32 value (eps near zero, where z may put inv_lo on the
other side). Every sample outside its row's window must round like the double
product; the signed error must stay in the interval for its sign of eps and
come near its far end; and both window values must catch products that round
the other way, so that neither can be dropped."""
import subprocess

SRC = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static uint64_t s = 0x2545F4914F6CDD1Dull;
static uint64_t rnd(void) { s ^= s << 13; s ^= s >> 7; s ^= s << 17; return s; }
static float f_bits(uint32_t b) { float f; memcpy(&f, &b, 4); return f; }
static uint32_t bits_f(float f) { uint32_t b; memcpy(&b, &f, 4); return b; }
static uint64_t bits_d(double d) { uint64_t b; memcpy(&b, &d, 8); return b; }

/* bf16 of a normal-range float, round to nearest even */
static uint32_t bf16_of_float(float f) {
  const uint32_t b = bits_f(f);
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}
/* bf16 of a normal-range double, round to nearest even (on the double's bits) */
static uint32_t bf16_of_double(double d) {
  uint64_t b = bits_d(d);
  const uint64_t sign = b >> 63;
  b &= 0x7FFFFFFFFFFFFFFFull;
  b = (b + ((1ull << 44) - 1) + ((b >> 45) & 1ull)) >> 45;   /* 1 + 11 + 7 bits */
  const uint64_t e = (b >> 7) - 1023 + 127, m = b & 0x7F;   /* carries went into e */
  return (uint32_t)((sign << 15) | (e << 7) | m);
}
/* a random bf16 of magnitude 2^(elo .. elo + span - 1), either sign */
static float rnd_bf16(int elo, int span) {
  const uint32_t e = (uint32_t)(127 + elo + (int)(rnd() % (uint64_t)span));
  return f_bits(((uint32_t)(rnd() & 1) << 31) | (e << 23) | ((uint32_t)(rnd() & 0x7F) << 16));
}

int main(void) {
  long n = 0, bad = 0, in_window = 0, just_outside = 0, caught_mid = 0, caught_side = 0, flipped = 0;
  long n_pos = 0, n_neg = 0;
  /* signed error (|exact| - |y32|) in ulps of y32's binade, by the sign of eps */
  double pos_min = 9, pos_max = -9, neg_min = 9, neg_max = -9;
  for (long k = 0; k < 6000000; ++k) {
    const float h = rnd_bf16(-20, 40), g = rnd_bf16(-8, 16);
    const float hg = h * g;                               /* exact: normal range */
    double inv;
    const int kind = (int)(k % 8);
    if (kind == 0) {                                      /* random inverse norm */
      inv = ldexp(1.0 + (double)(rnd() >> 11) * 0x1p-53, (int)(rnd() % 40) - 20);
    } else {                                              /* aim at a bf16 midpoint */
      const uint32_t m = (kind == 1) ? 0x7Fu : (uint32_t)(rnd() & 0x7F);
      const int e = (int)(rnd() % 40) - 20;
      const double mid = ldexp(1.0 + ((double)m + 0.5) / 128.0, e);   /* 1.m + half a bf16 ulp */
      inv = mid / fabs((double)hg);
      const double ulp32 = ldexp(1.0, e - 23);
      if (kind == 7) {
        /* eps near zero: an fp32 inverse norm, moved by a few fp64 ulps */
        inv = (double)(float)inv * (1.0 + ((double)(int64_t)(rnd() % 9) - 4.0) * 0x1p-53);
      } else {
        /* move the product by up to +-6 fp32 ulps of its binade */
        inv += ((double)(int64_t)(rnd() % 24001) - 12000.0) / 2000.0 * ulp32 / fabs((double)hg);
      }
    }
    /* the kernel's z: within 3 units of 2^-53 (relative) of inv */
    const double z = inv * (1.0 + ((double)(int64_t)(rnd() % 7) - 3.0) * 0x1p-53);
    const float inv32 = (float)inv;
    const float inv_lo = (float)(z - (double)inv32);
    const int neg = signbit(inv_lo) != 0;
    if ((inv < (double)inv32) != neg && inv != (double)inv32) ++flipped;
    const uint32_t wlo = neg ? 0x8000u : 0x7FFFu;         /* the row's window {wlo, wlo + 1} */

    const float y32 = hg * inv32;
    const double yo = (double)hg * inv;
    const uint32_t L = bits_f(y32) & 0xFFFFu;
    ++n;
    {   /* the exact product to 64 bits (long double), signed in magnitude */
      int ey;
      frexpf(y32, &ey);
      const long double ex = (long double)hg * (long double)inv;
      const double err = (double)((fabsl(ex) - fabsl((long double)y32)) / ldexpl(1.0L, ey - 24));
      if (inv >= (double)inv32) {
        ++n_pos;
        if (err < pos_min) pos_min = err;
        if (err > pos_max) pos_max = err;
      } else {
        ++n_neg;
        if (err < neg_min) neg_min = err;
        if (err > neg_max) neg_max = err;
      }
    }
    const int differs = bf16_of_float(y32) != bf16_of_double(yo);
    if (L == wlo || L == wlo + 1) {                       /* the kernel takes the exact path */
      ++in_window;
      if (differs) {
        if (L == 0x8000u) ++caught_mid;
        else ++caught_side;
      }
      continue;
    }
    if (L == wlo - 1 || L == wlo + 2) ++just_outside;
    if (differs) {
      if (bad < 5) printf("h=%a g=%a inv=%a y32=%a L=%x window=%x\n", h, g, inv, y32, L, wlo);
      ++bad;
    }
  }
  printf("checked %ld mismatches %ld window %ld just_outside %ld caught_mid %ld caught_side %ld flipped %ld "
         "n_pos %ld n_neg %ld pos_min %.6f pos_max %.6f neg_min %.6f neg_max %.6f\n", n, bad, in_window,
         just_outside, caught_mid, caught_side, flipped, n_pos, n_neg, pos_min, pos_max, neg_min, neg_max);
  return bad != 0;
}
"""


def test_norm_midpoint_window_per_row(tmp_path):
    src = tmp_path / "window.c"
    exe = tmp_path / "window"
    src.write_text(SRC)
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-o", str(exe), str(src), "-lm"],
                   check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    print(out.stdout)
    assert out.returncode == 0, out.stdout
    f = dict(zip(out.stdout.split()[0::2], out.stdout.split()[1::2]))
    assert int(f["mismatches"]) == 0
    assert int(f["window"]) > 50_000 and int(f["just_outside"]) > 50_000
    assert int(f["n_pos"]) > 1_000_000 and int(f["n_neg"]) > 1_000_000
    # the rows whose inv_lo sign differs from that of eps are exercised
    assert int(f["flipped"]) > 1000
    # both window values are needed: each catches products that round the other way
    assert int(f["caught_mid"]) > 0 and int(f["caught_side"]) > 0
    # the signed error stays in the interval the window is derived from, and
    # comes near its far end (so the window cannot shift toward the midpoint)
    tiny = 2.0 ** -20
    assert -0.5 - tiny <= float(f["pos_min"]) and float(f["pos_max"]) < 1.5
    assert -1.5 < float(f["neg_min"]) and float(f["neg_max"]) <= 0.5 + tiny
    assert float(f["pos_max"]) > 1.3 and float(f["neg_min"]) < -1.3
