"""The row statistics divide the sum of squares by N without a division: with
rn = 1/N rounded to nearest (computed once on the host), q0 = ss * rn is
within an ulp of ss / N, the residual ss - q0 * N is exact in one fma, and
fma(residual, rn, q0) is the correctly rounded quotient (Markstein's quotient
refinement). The kernel relies on this equalling IEEE division bit for bit;
this CPU test checks it with the same IEEE binary64 operations (C's
correctly rounded fma and division) for every row width the library accepts
and, per width, random sums of squares over the whole exponent range plus
sums whose quotient lies within a few ulps of a rounding midpoint."""
import os
import subprocess

SRC = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static uint64_t s = 0x9E3779B97F4A7C15ull;
static uint64_t rnd(void) { s ^= s << 13; s ^= s >> 7; s ^= s << 17; return s; }
static double from_bits(uint64_t b) { double d; memcpy(&d, &b, 8); return d; }

int main(void) {
  long bad = 0, n = 0, near = 0;
  for (int N = 8; N <= 32768; N += 8) {
    const double nd = (double)N, rn = 1.0 / nd;
    for (int k = 0; k < 600; ++k) {
      double ss;
      if (k < 400) {                       /* random positive doubles, exponents -900..900 */
        const uint64_t e = 123 + rnd() % 1800;
        ss = from_bits((e << 52) | (rnd() & 0xFFFFFFFFFFFFFull));
      } else {                             /* quotients next to a rounding midpoint */
        const uint64_t e = 900 + rnd() % 250;
        const double q = from_bits((e << 52) | (rnd() & 0xFFFFFFFFFFFFFull));
        const double half = (nextafter(q, INFINITY) - q) / 2;   /* half an ulp of q */
        /* N * (q + half), the midpoint times N: N*q = p + err exactly, and
           N * half is exact (a power of two times N <= 2^15) */
        const double p = nd * q, err = fma(nd, q, -p);
        ss = p + (err + nd * half);
        for (int d = (int)(rnd() % 5) - 2; d > 0; --d) ss = nextafter(ss, INFINITY);
        for (int d = (int)(rnd() % 5) - 2; d < 0; ++d) ss = nextafter(ss, 0.0);
      }
      const double q0 = ss * rn;
      const double got = fma(fma(-q0, nd, ss), rn, q0);
      const double want = ss / nd;
      ++n;
      {   /* how close the quotient is to a midpoint, in ulps (long double) */
        const long double ex = (long double)ss / (long double)nd;
        const long double ul = (long double)(nextafter(want, INFINITY) - want);
        long double f = (ex - (long double)want) / ul;
        if (f < 0) f = -f;
        if (f > 0.49L && f < 0.51L) ++near;
      }
      if (memcmp(&got, &want, 8) != 0) {
        if (bad < 5) printf("N=%d ss=%a got=%a want=%a\n", N, ss, got, want);
        ++bad;
      }
    }
  }
  printf("checked %ld mismatches %ld near %ld\n", n, bad, near);
  return bad != 0;
}
"""


def test_refined_quotient_equals_division(tmp_path):
    src = tmp_path / "q.c"
    src.write_text(SRC)
    exe = tmp_path / "q"
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", str(src), "-o", str(exe), "-lm"],
                   check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout
    assert "mismatches 0" in r.stdout
    near = int(r.stdout.split("near")[1])
    assert near > 20000, r.stdout     # tens of thousands of quotients within 0.01 ulp of a midpoint
