"""CPU check of the arithmetic identity the NVFP4 quantizer's fast path uses.

With S = (8 + m) / 8 * 2^e (any E4M3 value times a power-of-two global
scale) and r = RN(1 / S), the FMA sequence q = RN(x r), e = RN(q S - x),
y = RN(q - e r) equals RN(x / S) for every fp32 x.  Scaling by powers of two
is exact, so it suffices to run every fp32 significand of both signs over
two binades (x in [1, 4), which covers quotients on both sides of a binade
edge) against the 8 possible E4M3 significands; a few exponents of S are
included as a sanity check.  Signed zeros are covered by the GPU packing
tests (the host compiler may refold the sequence without regard to the sign
of a zero result)."""
import os
import shutil
import subprocess
import tempfile

import pytest

SRC = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>
static float f(uint32_t u) { float x; memcpy(&x, &u, 4); return x; }
static uint32_t bits(float x) { uint32_t u; memcpy(&u, &x, 4); return u; }
int main(void) {
  long bad = 0, total = 0;
  const int exps[3] = {-9, 0, 9};
  for (int m = 0; m < 8; m++)
    for (int k = 0; k < 3; k++) {
      const float S = ldexpf((8.0f + m) / 8.0f, exps[k]);
      const float r = 1.0f / S;
      for (int sgn = 0; sgn < 2; sgn++)
        for (uint32_t u = 0x3F800000u; u < 0x40800000u; u++) {
          const float x = f(u | (sgn ? 0x80000000u : 0u));
          const float q = x * r;
          const float e = fmaf(q, S, -x);
          const float y = fmaf(-e, r, q);
          const float z = x / S;
          total++;
          if (bits(y) != bits(z)) bad++;
        }
    }
  printf("%ld %ld\n", total, bad);
  return 0;
}
"""


def _has_fma() -> bool:
    try:
        with open("/proc/cpuinfo") as f:
            return " fma " in f.read()
    except OSError:
        return False


@pytest.mark.skipif(shutil.which("gcc") is None or not _has_fma(), reason="needs gcc and a host CPU with FMA")
def test_fma_corrected_quotient_is_correctly_rounded():
    with tempfile.TemporaryDirectory() as d:
        src, exe = os.path.join(d, "q.c"), os.path.join(d, "q")
        with open(src, "w") as f:
            f.write(SRC)
        subprocess.run(["gcc", "-O2", "-mfma", "-ffp-contract=off", "-fno-fast-math", src, "-o", exe, "-lm"],
                       check=True)
        out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout.split()
    total, bad = int(out[0]), int(out[1])
    assert total == 8 * 3 * 2 * (1 << 24)
    assert bad == 0
