"""The arithmetic shortcuts of the FP8 / INT8 append kernels, checked on the host over their whole
input space (no GPU, no library): the kernels replace the two correctly rounded fp32 divisions
of the row quantiser (scale = max|x| / M, then x / scale) by

- scale: s0 = a * RN(1/M), then one residual step s0 - (s0 M - a) RN(1/M);
- quotient: q = x * r with r any reciprocal within one ulp of 1/s, then one residual step
  q - (q s - x) r,

and claim that the stored scale is the correctly rounded a / M for every bf16 row maximum a, and
that the code of the quotient (E4M3FN round-to-nearest-even for M = 448, nearest integer with
ties to even for M = 127) is the code of the correctly rounded x / s for every bf16 x with
|x| <= a and s in [2^-80, 2^80] (outside that range the kernels divide). The GPU append tests
compare the kernels bit for bit with the oracle on sampled rows; this test is what covers the
rest of the inputs.

By default every bf16 row maximum is checked for the scale, and the quotient over all 128
mantissas of a in several binades (the quotient's code depends on the ratio of x and a only,
so these cover every ratio, including the ones that fall in the E4M3FN subnormal range);
SEG_ATTN_EXHAUSTIVE=1 runs every (x, a) pair (about two minutes)."""
import os
import shutil
import subprocess

import pytest

_SRC = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
static float bf(uint32_t b) { uint32_t u = b << 16; float f; memcpy(&f, &u, 4); return f; }
static uint32_t bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* The 127 non-negative finite E4M3FN values in code order (bias 7, 3 mantissa bits,
   subnormals at exponent field 0, code 0x7F is NaN and excluded). */
static double e4m3[127];
static void e4m3_table(void) {
  for (int c = 0; c < 127; ++c) {
    int e = c >> 3, m = c & 7;
    e4m3[c] = e == 0 ? ldexp(m / 8.0, -6) : ldexp(1.0 + m / 8.0, e - 7);
  }
}
/* Code of a value with |v| <= 448: nearest table entry, ties to the even code; sign bit 7. */
static int e4m3_code(float v) {
  int sign = (bits(v) >> 31) << 7;
  double a = fabs((double)v);
  int lo = 0, hi = 126;
  while (hi - lo > 1) { int mid = (lo + hi) / 2; if (e4m3[mid] <= a) lo = mid; else hi = mid; }
  int c;
  if (a <= e4m3[lo]) c = lo;
  else if (a >= e4m3[hi]) c = hi;
  else {
    double dl = a - e4m3[lo], dh = e4m3[hi] - a;
    c = dl < dh ? lo : (dh < dl ? hi : ((lo & 1) == 0 ? lo : hi));
  }
  return sign | c;
}
static int code(float q, float M) {
  float cq = fminf(fmaxf(q, -M), M);
  return M == 448.0f ? e4m3_code(cq) : (int)rintf(cq);
}

int main(int argc, char** argv) {
  const float M = (float)atof(argv[1]);
  const int full = atoi(argv[2]);
  e4m3_table();
  const float c = 1.0f / M;
  long scale_bad = 0, scale_n = 0;
  for (uint32_t ab = 1; ab < 0x7F80; ++ab) {
    const float a = bf(ab), s0 = a * c;
    scale_n++;
    if (fmaf(-fmaf(s0, M, -a), c, s0) != a / M) scale_bad++;
  }
  long quot_bad = 0, quot_n = 0;
  /* binades of a: every one, or a spread that includes both ends of the fast range */
  const int sample_exp[] = {-60, -20, -3, 0, 1, 7, 20, 60};
  const int n_exp = full ? 0 : (int)(sizeof(sample_exp) / sizeof(sample_exp[0]));
  for (uint32_t ab = 1; ab < 0x7F80; ++ab) {
    const float a = bf(ab);
    if (!full) {
      int e; frexpf(a, &e);
      int keep = 0;
      for (int i = 0; i < n_exp; ++i) keep |= (e - 1 == sample_exp[i]);
      if (!keep) continue;
    }
    const float s = a / M;
    if (!(s >= 0x1p-80f && s <= 0x1p80f)) continue;
    const float r0 = 1.0f / s;
    const float rs[3] = {r0, from_bits(bits(r0) - 1), from_bits(bits(r0) + 1)};
    for (uint32_t xb = 0; xb < 0x10000; ++xb) {
      const float x = bf(xb);
      if (isnan(x) || isinf(x) || fabsf(x) > a) continue;
      const int want = code(x / s, M);
      for (int k = 0; k < 3; ++k) {
        const float q = x * rs[k];
        const float q1 = fmaf(-fmaf(q, s, -x), rs[k], q);
        quot_n++;
        if (code(q1, M) != want) quot_bad++;
      }
    }
  }
  printf("%ld %ld %ld %ld\n", scale_n, scale_bad, quot_n, quot_bad);
  return 0;
}
"""


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    d = tmp_path_factory.mktemp("quant_arith")
    src = d / "check.c"
    src.write_text(_SRC)
    exe = d / "check"
    # -ffp-contract=off: every product and fma exactly as written, no fusing by the compiler
    subprocess.run([cc, "-O2", "-ffp-contract=off", "-o", str(exe), str(src), "-lm"], check=True)
    return exe


@pytest.mark.parametrize("M", [448, 127])
def test_shortcuts_give_the_correctly_rounded_codes(checker, M):
    full = os.environ.get("SEG_ATTN_EXHAUSTIVE") == "1"
    out = subprocess.run([str(checker), str(M), "1" if full else "0"], check=True,
                         capture_output=True, text=True, timeout=900).stdout.split()
    scale_n, scale_bad, quot_n, quot_bad = map(int, out)
    assert scale_n == 32639 and scale_bad == 0
    assert quot_n > 10 ** 6 and quot_bad == 0


def test_the_checker_sees_a_plain_product_fail(checker, tmp_path):
    # without the residual step the codes do differ for some pairs: the check has teeth
    src = tmp_path / "plain.c"
    src.write_text(_SRC.replace("const float q1 = fmaf(-fmaf(q, s, -x), rs[k], q);",
                                "const float q1 = q;"))
    exe = tmp_path / "plain"
    cc = shutil.which("gcc") or shutil.which("cc")
    subprocess.run([cc, "-O2", "-ffp-contract=off", "-o", str(exe), str(src), "-lm"], check=True)
    out = subprocess.run([str(exe), "448", "0"], check=True, capture_output=True, text=True,
                         timeout=900).stdout.split()
    assert int(out[3]) > 0
