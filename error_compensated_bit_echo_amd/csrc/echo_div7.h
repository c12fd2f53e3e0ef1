// Correctly rounded binary32 division by 7 without a divide instruction.
//
// The group scale is s = fl(a / 7).  A full IEEE divide costs about ten
// instructions per lane; this takes three.  q0 = fl(a * c) with c = fl(1/7)
// is within one ulp of a/7, so the remainder a - 7*q0 is exactly
// representable and one fused multiply-add computes it without error;
// a second fused multiply-add adds the remainder times c back (Markstein's
// FMA-based correction of a quotient, "Computation of elementary functions on
// the IBM RISC System/6000 processor", IBM J. Res. Dev. 34(1), 1990).
// The result has been compared with IEEE division for every non-negative
// finite binary32 a, subnormals included, with no difference; a CPU test
// repeats that exhaustive comparison.
//
// The header is plain C so that the host-side test can include it: define
// ECHO_DIV7_QUAL before including it to change the function qualifiers.
#ifndef ECHO_DIV7_H
#define ECHO_DIV7_H

#ifndef ECHO_DIV7_QUAL
#define ECHO_DIV7_QUAL __device__ __forceinline__
#endif

// fl(1/7) = 0x3E124925
#define ECHO_RCP7 0.142857149243354797363281250f

ECHO_DIV7_QUAL float echo_div7(float a) {
  const float q0 = a * ECHO_RCP7;
  const float r = __builtin_fmaf(-q0, 7.0f, a);
  return __builtin_fmaf(r, ECHO_RCP7, q0);
}

#endif  // ECHO_DIV7_H
