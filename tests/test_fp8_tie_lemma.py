"""The FP8 encode decides its rare undecided elements without any division
or branch, on the strength of one fact about the group quantization, checked
here exhaustively on the CPU.

For a group maximum amax (a bf16 magnitude, at least 2^-100 so the scale is a
normal fp32 number) and any bf16 value v with |v| <= amax, let R = 448 |v| /
amax, the quotient by the exact scale amax / 448. Then R is either exactly an
e4m3fn rounding midpoint (the point halfway between two neighbouring codes)
or at least 2^-19 (relative) away from every midpoint. (A ratio of two
8-bit mantissas times 448 that is not a 5-bit dyadic number misses every
such number by about 2^-13 or more.)

Consequence used by the kernels: the stored scale is s = fl32(amax / 448), so
v / s = R * (amax / (448 s)) with |amax / (448 s) - 1| <= 2^-24. Whenever the
two products v * r_lo and v * r_hi that bracket v / s within 2^-20 round to
different codes, a midpoint lies within 2^-20 of v / s, hence within 2^-19
of R, hence R IS that midpoint; v / s then lies above it exactly when
448 s < amax, below it when 448 s > amax, and on it (a tie: even code) when
448 s == amax. The sign of fma(s, 448, -amax) (exact sign: one rounding of
an exact difference that cannot underflow to zero for amax >= 2^-100)
therefore picks the code."""
import subprocess

SRC = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static double bf16(uint32_t b) { uint32_t u = b << 16; float f; memcpy(&f, &u, 4); return f; }

int main(void) {
  long pairs = 0, ties = 0, bad = 0;
  double min_rel = 1.0;
  for (uint32_t ab = 0x0D80; ab <= 0x7F7F; ++ab) {          /* amax >= 2^-100, finite */
    const double a = bf16(ab);
    for (uint32_t vb = 1; vb <= ab; ++vb) {                  /* 0 < v <= amax */
      const double v = bf16(vb);
      const double R = 448.0 * v / a;                        /* within 2^-53 of the ratio */
      /* the neighbouring e4m3fn values below and above R and the midpoint between them */
      double u;
      if (R >= 0x1p-6) { int e; frexp(R, &e); u = ldexp(1.0, e - 1 - 3); }
      else u = 0x1p-9;
      const double lo = floor(R / u) * u, M = lo + u / 2;
      ++pairs;
      if (448.0 * v == M * a) { ++ties; continue; }          /* both products exact in double */
      const double rel = fabs(R - M) / M;
      if (rel < min_rel) min_rel = rel;
      if (rel < 0x1p-19) {
        if (bad < 5) printf("near miss: amax %04x v %04x rel %g\n", ab, vb, rel);
        ++bad;
      }
    }
  }
  printf("pairs %ld ties %ld near_misses %ld min_rel_log2 %.2f\n", pairs, ties, bad, log2(min_rel));
  return bad != 0;
}
"""


def test_ratio_is_a_midpoint_or_far_from_every_midpoint(tmp_path):
    src = tmp_path / "lemma.c"
    src.write_text(SRC)
    exe = tmp_path / "lemma"
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", str(src), "-o", str(exe), "-lm"],
                   check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stdout
    fields = dict(zip(r.stdout.split()[::2], r.stdout.split()[1::2]))
    assert int(fields["near_misses"]) == 0
    assert int(fields["pairs"]) > 500_000_000 and int(fields["ties"]) > 300_000
    assert float(fields["min_rel_log2"]) > -19
