// Nearest int4 code of one element, decided in binary32 with exact tests.
//
// The group scale is s = fl(absmax / 7) and the code of v is the integer in
// [-7, 7] nearest to the exact quotient v/s, ties to the even integer.  With
// inv an approximation of 1/s (the hardware reciprocal is within one ulp),
// t = v * inv is within far less than 1/2 of v/s, so k = rint(t) is the nearest
// code or one of its neighbours.  e = fma(-k, s, v) is v - k*s rounded once:
// its sign is exact and |e| < s/2 proves k nearest.  Otherwise v/s lies
// beyond, on, or just short of the half-integer m = k + sign(e)/2, and
// d = fma(-m, s, v) tells which, exactly: d is zero only for an exact tie (m*s
// is a multiple of half an ulp of s, which is far above the subnormal spacing
// for s >= 2^-100, so a nonzero difference cannot round to zero), and a tie
// goes to the even code.
//
// bfloat16 inputs hit ties and near-ties often (v = absmax/2 gives v/s = 3.5
// up to the rounding of s), which is why the test is done per element and in
// binary32 rather than by falling back to a division.
//
// The code is returned as f = k + 1.5 * 2^23: that float holds k, in two's
// complement, in its low mantissa bits, and f - 1.5 * 2^23 is k exactly.
// Adding 1.5 * 2^23 to t rounds t to an integer, ties to even (|t| < 2^22).
//
// The header is plain C so that a host-side test can include it: define
// ECHO_QUANT_QUAL before including it to change the function qualifiers.
#ifndef ECHO_QUANT_H
#define ECHO_QUANT_H

#ifndef ECHO_QUANT_QUAL
#define ECHO_QUANT_QUAL __device__ __forceinline__
#endif

#define ECHO_ROUND_MAGIC 12582912.0f /* 1.5 * 2^23 */

// Smallest scale for which the binary32 decision below is used; smaller
// nonzero scales take an exact binary64 path.
#define ECHO_TINY_SCALE 0x1p-100f

// v: element; s: group scale (s >= ECHO_TINY_SCALE); inv: approximately 1/s;
// h: s / 2.  Returns k + 1.5 * 2^23 for the nearest code k, ties to even.
ECHO_QUANT_QUAL float echo_code_magic(float v, float s, float inv, float h) {
  float f = v * inv + ECHO_ROUND_MAGIC;
  const float k = f - ECHO_ROUND_MAGIC;
  const float e = __builtin_fmaf(-k, s, v);
  if (!(__builtin_fabsf(e) < h)) {
    const float dir = __builtin_copysignf(1.0f, e);
    const float d = __builtin_fmaf(-(k + 0.5f * dir), s, v);
    union { float f; unsigned int u; } bits;
    bits.f = f;
    const int step = d != 0.0f ? ((d > 0.0f) == (e > 0.0f)) : (int)(bits.u & 1u);
    if (step) f = (k + dir) + ECHO_ROUND_MAGIC;
  }
  return f;
}

// Dequantization fl(q * s) of a code q in [-8, 7] given as u = q + 8 in
// [0, 15] (which one byte-to-float conversion produces from a nibble stored
// with its sign bit flipped): the exact value (q + 8) * s - 8 * s equals q * s,
// so one fused multiply-add rounds it once, to exactly fl(q * s), provided
// m8 = -8 * s is finite (s < 2^124 is enough).  The one difference is the sign
// of a zero: with s = 0 and q < 0, fl(q * s) is -0 and the fma gives +0; a
// zero scale only comes from an all-zero group, whose codes are all 0.
#define ECHO_DEQUANT_FMA_MAX_SCALE 0x1p124f

ECHO_QUANT_QUAL float echo_dequant_fma(float u, float s, float m8) {
  return __builtin_fmaf(u, s, m8);
}

#endif  // ECHO_QUANT_H
