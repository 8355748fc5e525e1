"""The NVFP4 kernels' division-free quotients, checked on the CPU.

Per 16-group the NVFP4 steps need m = g / v and kf = v / g, rounded to
nearest-even fp32, where v is the value of an E4M3 scale byte and g the
per-tensor multiplier ("[Transform] [Quantization] Add QuTLASS support to
vLLM", Purpose; the NVFP4 call shape in the review of
bench_nvfp4_qutlass.py).  For g in [2^-60, 2^60] the kernels compute them
without a division:

  m  = q + (g - q v) y  (two fmas),  q = g y,  y = an approximate 1 / v
  kf = fp32(fp64(v) * (1 / fp64(g)))

and g / 6 (per tensor) in the same form as m.  The argument that these
are the correctly rounded quotients rests on v (and 6) having at most 4
significant bits.  This test compiles the same formulas in C (no
contraction: every product and fma rounds where the kernel's does), with y
taken as the correctly rounded reciprocal moved by up to 3 ulp either way
(the hardware reciprocal is within 1 ulp), and compares them bit for bit
with fp32 division over every nonzero finite scale byte and a spread of
g values, the ends of the range included.
"""
import os
import subprocess
import tempfile

C_SRC = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float e4m3_value(unsigned b) {           /* non-negative E4M3 byte */
  unsigned e = (b >> 3) & 15u, f = b & 7u;
  return e ? ldexpf((float)(8u + f), (int)e - 10) : ldexpf((float)f, -9);
}
static uint32_t bits(float x) { uint32_t u; memcpy(&u, &x, 4); return u; }
static uint64_t state = 0x9E3779B97F4A7C15ull;   /* splitmix64 */
static uint64_t next(void) {
  uint64_t z = (state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

int main(int argc, char **argv) {
  long n = atol(argv[1]), checked = 0, bad = 0;
  for (long i = 0; i < n + 4; ++i) {
    float g;
    if (i == n) g = 0x1p-60f;
    else if (i == n + 1) g = 0x1p60f;
    else if (i == n + 2) g = nextafterf(0x1p60f, 0.0f);
    else if (i == n + 3) g = 1.0f;
    else {
      uint64_t r = next();
      int ex = (int)(r % 121) - 60;                 /* 2^-60 .. 2^60 */
      float mant = 1.0f + (float)((r >> 8) & 0x7FFFFF) * 0x1p-23f;
      g = ldexpf(mant, ex);
      if (g > 0x1p60f) g = 0x1p60f;
    }
    const double ig = 1.0 / (double)g;
    {                                               /* c6 = g / 6, same form */
      float y = 1.0f / 6.0f;
      for (int k = 0; k < 3; ++k) y = nextafterf(y, 0.0f);
      for (int d = -3; d <= 3; ++d) {
        const float q = g * y;
        const float c6 = fmaf(fmaf(-q, 6.0f, g), y, q);
        if (bits(c6) != bits(g / 6.0f)) { ++bad; if (bad < 5) printf("c6 g=%a d=%d\n", g, d); }
        y = nextafterf(y, INFINITY);
        ++checked;
      }
    }
    for (unsigned b = 1; b < 127; ++b) {
      const float v = e4m3_value(b);
      const float want_m = g / v, want_kf = v / g;
      const float kf = (float)((double)v * ig);
      if (bits(kf) != bits(want_kf)) { ++bad; if (bad < 5) printf("kf g=%a v=%a\n", g, v); }
      float y = 1.0f / v;
      for (int k = 0; k < 3; ++k) y = nextafterf(y, 0.0f);
      for (int d = -3; d <= 3; ++d) {
        const float q = g * y;
        const float m = fmaf(fmaf(-q, v, g), y, q);
        if (bits(m) != bits(want_m)) { ++bad; if (bad < 5) printf("m g=%a v=%a d=%d\n", g, v, d); }
        y = nextafterf(y, INFINITY);
        ++checked;
      }
    }
  }
  printf("checked %ld bad %ld\n", checked, bad);
  return bad != 0;
}
"""


def test_division_free_quotients_are_correctly_rounded():
    with tempfile.TemporaryDirectory() as d:
        src, exe = os.path.join(d, "q.c"), os.path.join(d, "q")
        with open(src, "w") as f:
            f.write(C_SRC)
        # -ffp-contract=off: q = g * y must round on its own, as in the kernel
        subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", src, "-o", exe, "-lm"])
        r = subprocess.run([exe, "200000"], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout
    assert "bad 0" in r.stdout, r.stdout
