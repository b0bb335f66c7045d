"""The kernels form the FP8 group scale s = fl32(amax / 448) in fp32 without a
division: q0 = fl32(amax * c) with c = fl32(1/448), then
s = fma(fma(-q0, 448, amax), c, q0). This CPU test checks, for every bf16
amax from 2^-100 to the largest finite one (the range the kernels use it
for; smaller amax take the IEEE division), that the result is bit for bit
the correctly rounded quotient, computed here as the double quotient
rounded to fp32 (the quotient never lies within 2^-27 of an fp32 midpoint
unless it is exact, so the double rounding cannot differ) and also with
C's correctly rounded float division. The GPU probe test of fp8_scale checks
the kernels' own instructions over the same values."""
import subprocess

SRC = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>
static float fb(uint32_t b) { float f; memcpy(&f, &b, 4); return f; }
static uint32_t bf(float f) { uint32_t b; memcpy(&b, &f, 4); return b; }
int main(void) {
  const float c = 1.0f / 448.0f;
  long bad = 0, n = 0, exact = 0;
  for (uint32_t ab = 0x0D80; ab <= 0x7F7F; ++ab) {
    const float a = fb(ab << 16);
    const float want = (float)((double)a / 448.0);
    const float want2 = a / 448.0f;
    const float q0 = a * c;
    const float s = fmaf(fmaf(-q0, 448.0f, a), c, q0);
    ++n;
    if ((double)s * 448.0 == (double)a) ++exact;
    if (bf(s) != bf(want) || bf(s) != bf(want2)) {
      if (bad < 5) printf("a=%a want=%a got=%a\n", a, want, s);
      ++bad;
    }
  }
  printf("checked %ld mismatches %ld exact %ld\n", n, bad, exact);
  return bad != 0;
}
"""


def test_fp32_scale_refinement_is_correctly_rounded(tmp_path):
    src, exe = tmp_path / "scale.c", tmp_path / "scale"
    src.write_text(SRC)
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-o", str(exe), str(src), "-lm"], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    print(out.stdout)
    assert out.returncode == 0, out.stdout
    f = dict(zip(out.stdout.split()[0::2], out.stdout.split()[1::2]))
    assert int(f["checked"]) == 0x7F7F - 0x0D80 + 1 and int(f["mismatches"]) == 0
    assert int(f["exact"]) > 1000      # the amax with a mantissa that 7 divides: exact quotients
