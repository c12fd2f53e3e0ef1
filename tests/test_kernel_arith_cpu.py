"""CPU checks of arithmetic building blocks the HIP kernels rely on.

These compile the kernels' own helper header for the host and compare it with
IEEE arithmetic exhaustively; no GPU and no oracle is involved.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "error_compensated_bit_echo_amd", "csrc")

DIV7_CHECK = r"""
#include <stdint.h>
#include <stdio.h>
#include <string.h>
#define ECHO_DIV7_QUAL static inline
#include "echo_div7.h"

int main(void) {
  long long bad = 0;
  uint32_t first = 0;
  /* every non-negative finite binary32, subnormals included */
  #pragma omp parallel for reduction(+:bad) schedule(static, 1 << 20)
  for (long long i = 0; i < 0x7F800000LL; ++i) {
    uint32_t u = (uint32_t)i;
    float a;
    memcpy(&a, &u, 4);
    volatile float seven = 7.0f;
    float want = a / seven;
    float got = echo_div7(a);
    uint32_t x, y;
    memcpy(&x, &want, 4);
    memcpy(&y, &got, 4);
    if (x != y) bad++;
  }
  printf("%lld\n", bad);
  return bad != 0;
}
"""


def _has_fma() -> bool:
    try:
        with open("/proc/cpuinfo") as f:
            return " fma " in f.read()
    except OSError:
        return False


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_div7_matches_ieee_division_exhaustively(tmp_path):
    """fl(a/7) by multiply + two FMA corrections equals IEEE a/7 for every
    non-negative finite binary32 a (2^31 - 2^23 values)."""
    src = tmp_path / "div7.c"
    exe = tmp_path / "div7"
    src.write_text(DIV7_CHECK)
    flags = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", f"-I{CSRC}"]
    if _has_fma():
        flags.append("-mfma")  # otherwise __builtin_fmaf calls libm's exact fmaf
    subprocess.run(["gcc", *flags, str(src), "-o", str(exe), "-lm"], check=True)
    env = dict(os.environ)
    env.setdefault("OMP_NUM_THREADS", str(min(8, os.cpu_count() or 1)))
    res = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=600)
    assert res.returncode == 0, f"mismatches: {res.stdout.strip()} {res.stderr.strip()}"
    assert res.stdout.strip() == "0"


QUANT_CHECK = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>
#define ECHO_DIV7_QUAL static inline
#define ECHO_QUANT_QUAL static inline
#include "echo_div7.h"
#include "echo_quant.h"

static float fb(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t ub(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* nearest integer to the exact v/s, ties to even: binary64 decides exactly */
static int nearest(float v, float s) { return (int)rint((double)v / (double)s); }

/* 0 if echo_code_magic gives the nearest code for all three reciprocals
   (correctly rounded 1/s and its two neighbours: the hardware reciprocal is
   within one ulp), and its low nibble is the code in two's complement */
static int bad(float v, float s) {
  const float r = 1.0f / s;
  const float invs[3] = {r, nextafterf(r, 0.0f), nextafterf(r, INFINITY)};
  const int want = nearest(v, s);
  int n = 0;
  for (int i = 0; i < 3; ++i) {
    const float f = echo_code_magic(v, s, invs[i], 0.5f * s);
    const int k = (int)(f - ECHO_ROUND_MAGIC);
    n += (k != want) || ((ub(f) & 15u) != ((uint32_t)want & 15u));
  }
  return n;
}

static uint64_t rng(uint64_t* x) { *x ^= *x << 13; *x ^= *x >> 7; *x ^= *x << 17; return *x; }

int main(void) {
  long long nbad = 0, ntie = 0, n = 0;
  /* A: bfloat16 groups.  Absmax a over every positive bf16 with exponent in
     [-40, 40]; v over every bf16 with |v| <= a. */
  #pragma omp parallel for reduction(+:nbad, n) schedule(dynamic, 16)
  for (int ia = 0; ia < 81 * 128; ++ia) {
    const uint32_t ea = (uint32_t)(ia / 128 - 40 + 127), ma = (uint32_t)(ia % 128);
    const float a = fb((ea << 23) | (ma << 16));
    const float s = echo_div7(a);
    for (uint32_t vb = 0; vb < 65536; ++vb) {
      const float v = fb(vb << 16);
      if (!(fabsf(v) <= a)) continue;
      nbad += bad(v, s);
      n++;
    }
  }
  /* B: random binary32 groups: a with exponent in [-90, 90], v uniform bits in [-a, a] */
  #pragma omp parallel for reduction(+:nbad, n) schedule(static)
  for (int t = 0; t < 64; ++t) {
    uint64_t x = 0x9E3779B97F4A7C15ull * (uint64_t)(t + 1);
    for (int i = 0; i < 1000000; ++i) {
      const uint32_t ea = (uint32_t)(rng(&x) % 181) + 127 - 90;
      const float a = fb((ea << 23) | (uint32_t)(rng(&x) & 0x7FFFFF));
      const float s = echo_div7(a);
      const float v = a * (float)((double)(rng(&x) >> 11) / 9007199254740992.0 * 2.0 - 1.0);
      nbad += bad(v, s);
      n++;
    }
  }
  /* C: exact ties v = (2k+1)/2 * s (s with zero low mantissa bits, so v is
     exact) and their binary32 neighbours */
  #pragma omp parallel for reduction(+:nbad, n, ntie) schedule(static)
  for (int t = 0; t < 16; ++t) {
    uint64_t x = 0xD1B54A32D192ED03ull * (uint64_t)(t + 1);
    for (int i = 0; i < 200000; ++i) {
      const uint32_t es = (uint32_t)(rng(&x) % 161) + 127 - 80;
      const float s = fb((es << 23) | ((uint32_t)rng(&x) & 0x7FFF00u));
      for (int k2 = -13; k2 <= 13; k2 += 2) {
        const float v = (float)k2 * 0.5f * s;
        if ((double)v != (double)k2 * 0.5 * (double)s) continue;
        ntie++;
        nbad += bad(v, s) + bad(nextafterf(v, 0.0f), s) + bad(nextafterf(v, INFINITY), s);
        n += 3;
      }
    }
  }
  printf("%lld %lld %lld\n", nbad, n, ntie);
  return nbad != 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_code_choice_matches_exact_round_half_even(tmp_path):
    """The binary32 code decision of the kernels equals round-half-even of the
    exact quotient v/s on every bf16 (v, absmax) pair over 81 binades, on 64M
    random binary32 pairs and on constructed exact ties and their neighbours,
    for the correctly rounded reciprocal and both one-ulp neighbours."""
    src = tmp_path / "quant.c"
    exe = tmp_path / "quant"
    src.write_text(QUANT_CHECK)
    flags = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", f"-I{CSRC}"]
    if _has_fma():
        flags.append("-mfma")
    subprocess.run(["gcc", *flags, str(src), "-o", str(exe), "-lm"], check=True)
    env = dict(os.environ)
    env.setdefault("OMP_NUM_THREADS", str(min(8, os.cpu_count() or 1)))
    res = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=900)
    nbad, n, ntie = (int(x) for x in res.stdout.split())
    assert ntie > 1_000_000 and n > 500_000_000
    assert res.returncode == 0 and nbad == 0, f"{nbad} wrong codes out of {n}"


DEQUANT_CHECK = r"""
#include <stdint.h>
#include <stdio.h>
#include <string.h>
#define ECHO_QUANT_QUAL static inline
#include "echo_quant.h"

int main(void) {
  long long bad = 0, n = 0;
  /* every 61st non-negative binary32 below 2^124 (all binades, subnormals
     included), every code q in [-8, 7] given as u = q + 8 */
  const uint32_t top = 0x7D800000u; /* 2^124 */
  #pragma omp parallel for reduction(+:bad, n) schedule(static, 1 << 16)
  for (long long i = 0; i < (long long)top; i += 61) {
    uint32_t b = (uint32_t)i;
    float s;
    memcpy(&s, &b, 4);
    if (!(s < ECHO_DEQUANT_FMA_MAX_SCALE)) continue;
    const float m8 = -8.0f * s;
    for (int u = 0; u < 16; ++u) {
      /* a zero scale only ever carries code 0 (all-zero group): -0 vs +0 */
      if (s == 0.0f && u != 8) continue;
      volatile float q = (float)(u - 8);
      const float want = q * s;                /* fl(q * s): one rounding */
      const float got = echo_dequant_fma((float)u, s, m8);
      uint32_t x, y;
      memcpy(&x, &want, 4);
      memcpy(&y, &got, 4);
      bad += (x != y);
      n++;
    }
  }
  printf("%lld %lld\n", bad, n);
  return bad != 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_dequant_fma_equals_rounded_product(tmp_path):
    """fma(q + 8, s, -8 s) is exactly fl(q * s) for every code and the sampled
    scales (a zero scale is checked with code 0 only, the one code it carries)."""
    src = tmp_path / "deq.c"
    exe = tmp_path / "deq"
    src.write_text(DEQUANT_CHECK)
    flags = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", f"-I{CSRC}"]
    if _has_fma():
        flags.append("-mfma")
    subprocess.run(["gcc", *flags, str(src), "-o", str(exe), "-lm"], check=True)
    env = dict(os.environ)
    env.setdefault("OMP_NUM_THREADS", str(min(8, os.cpu_count() or 1)))
    res = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=600)
    bad, n = (int(x) for x in res.stdout.split())
    assert n > 500_000_000
    assert res.returncode == 0 and bad == 0, f"{bad} of {n} differ"
