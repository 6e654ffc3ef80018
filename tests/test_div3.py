"""The quantizers' division of a group's range by 3 (device.h div3):
q0 = d * RN(1/3), r = fma(-3, q0, d), fminf(fma(r, RN(1/3), q0), d).  The
claim is that this equals the correctly rounded d / 3 for every
non-negative fp32 d, +inf included.  Checked here for all 2^31 + 1 bit
patterns from +0 to +inf by a small C program (the host's fmaf and
division are IEEE fp32 with round-to-nearest and denormals kept, as on the
device); the GPU side is pinned end to end by the bit-exact parity tests,
whose oracle divides."""
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
static float f32(uint32_t u) { float x; memcpy(&x, &u, 4); return x; }
static uint32_t bits(float x) { uint32_t u; memcpy(&u, &x, 4); return u; }
static float div3(float d) {
  const float y = 0x1.555556p-2f;
  const float q0 = d * y;
  const float r = fmaf(-3.0f, q0, d);
  return fminf(fmaf(r, y, q0), d);
}
int main(void) {
  unsigned long long bad = 0;
#pragma omp parallel for reduction(+ : bad) schedule(static)
  for (long long u = 0; u <= 0x7F800000LL; ++u) {
    const float d = f32((uint32_t)u);
    if (bits(div3(d)) != bits(d / 3.0f)) ++bad;
  }
  printf("mismatches %llu\n", bad);
  return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_div3_equals_division_for_every_nonnegative_float():
    with tempfile.TemporaryDirectory() as d:
        src, exe = os.path.join(d, "div3.c"), os.path.join(d, "div3")
        with open(src, "w") as f:
            f.write(SRC)
        subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", src, "-o", exe,
                        "-lm"], check=True)
        out = subprocess.run([exe], check=True, capture_output=True, text=True, timeout=600).stdout
    assert out.strip() == "mismatches 0", out
