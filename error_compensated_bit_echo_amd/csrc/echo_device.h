// Device-side building blocks shared by the kernels: cache-policy accessors,
// the group absmax across lanes, the exact int4 code choice, packing and
// unpacking, and bfloat16 conversions.  Every floating-point step is a
// separate IEEE binary32 operation (contraction off), so the kernels that use
// these reproduce the same sequence of roundings.
#pragma once

#pragma clang fp contract(off)

#include "echo_internal.h"
#include "echo_div7.h"
#include "echo_quant.h"

namespace echo {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Cache policy of a global access: plain, or non-temporal (streamed once).
template <bool NT, typename T>
__device__ __forceinline__ T ld(const T* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}
template <bool NT, typename T>
__device__ __forceinline__ void st(T v, T* p) {
  if constexpr (NT) __builtin_nontemporal_store(v, p);
  else *p = v;
}

// Policy bits of the kernels' template parameter POL.
constexpr int kNtIn = 1;         // stage 1: partials; owner: stage-1 codes; decode: codes
constexpr int kNtStateLd = 2;    // owner: compensator loads
constexpr int kNtStateSt = 4;    // owner: compensator stores
constexpr int kNtOut = 8;        // decode: output stores; stage 1 / owner: code stores

__device__ __forceinline__ float quad_max(float x) {
  // quad_perm(1,0,3,2) then quad_perm(2,3,0,1): all four lanes get the max.
  int xi = __float_as_int(x);
  float y = __int_as_float(__builtin_amdgcn_update_dpp(xi, xi, 0xB1, 0xF, 0xF, false));
  x = fmaxf(x, y);
  xi = __float_as_int(x);
  y = __int_as_float(__builtin_amdgcn_update_dpp(xi, xi, 0x4E, 0xF, 0xF, false));
  return fmaxf(x, y);
}

// Max over the LPG lanes of an aligned group (LPG = 4, 8 or 16): the quad
// first, then row_half_mirror (lane i and 7 - i of each 8 lanes) and row_mirror
// (lane i and 15 - i of each 16 lanes) bring in the other quad and the other
// half-row.
template <int LPG>
__device__ __forceinline__ float group_max(float x) {
  static_assert(LPG == 4 || LPG == 8 || LPG == 16, "4, 8 or 16 lanes per group");
  x = quad_max(x);
  if constexpr (LPG >= 8) {
    const int xi = __float_as_int(x);
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(xi, xi, 0x141, 0xF, 0xF, false)));
  }
  if constexpr (LPG >= 16) {
    const int xi = __float_as_int(x);
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(xi, xi, 0x140, 0xF, 0xF, false)));
  }
  return x;
}

constexpr int log2i(int x) { return x <= 1 ? 0 : 1 + log2i(x / 2); }

// Nearest code in [-7, 7] to the exact quotient v / s (s > 0), ties to even,
// in binary64: a quotient of two binary32 values that is not a tie lies at
// least 2^-26 from a half-integer, far beyond binary64's rounding error, and
// a tie is representable.  Used for the (rare) groups whose scale is nonzero
// but below ECHO_TINY_SCALE, where rcp(s) could overflow.
__device__ __forceinline__ int exact_code(float v, float s) {
  double q = __builtin_rint(static_cast<double>(v) / static_cast<double>(s));
  q = q > 7.0 ? 7.0 : q;
  q = q < -7.0 ? -7.0 : q;
  return static_cast<int>(q);
}

// Codes of the 8 values a lane holds, for group scale s = fl(absmax / 7).
// Returns the packed nibbles; kf receives the codes as floats.
__device__ __forceinline__ uint32_t quantize8(const float (&v)[8], float s, float (&kf)[8]) {
  uint32_t w = 0;
  if (s >= ECHO_TINY_SCALE) {
    const float inv = __builtin_amdgcn_rcpf(s);  // within 1 ulp of 1/s
    const float h = 0.5f * s;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float f = echo_code_magic(v[j], s, inv, h);
      kf[j] = f - ECHO_ROUND_MAGIC;  // exact
      // shift the code's nibble in from the top: after 8 steps element j sits
      // in bits 4j..4j+3
      w = __builtin_amdgcn_alignbit(__float_as_uint(f), w, 4);
    }
  } else if (s > 0.0f) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int k = exact_code(v[j], s);
      kf[j] = static_cast<float>(k);
      w |= (static_cast<uint32_t>(k) & 15u) << (4 * j);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) kf[j] = 0.0f;
  }
  return w;
}

// Signed code of element j (0..7) of a packed word.
__device__ __forceinline__ int nibble(uint32_t w, int j) {
  return static_cast<int>(w << (28 - 4 * j)) >> 28;
}

// Each rank's contribution d[r][j] = fl(q_r,j * s_r) for the 8 elements of a
// chunk.  Flipping the sign bit of every nibble turns code q into q + 8 in
// [0, 15], a byte after one mask, which one conversion turns into a float;
// echo_dequant_fma then gives fl(q * s) exactly in one instruction (two fewer
// than extract, convert and multiply).  Scales of 2^124 and above, which only
// inputs near the top of the binary32 range produce, take the direct product.
template <int P>
__device__ __forceinline__ void dequant_ranks(const uint32_t (&w)[P], const float (&s)[P],
                                              float (&d)[P][8]) {
  float smax = s[0];
#pragma unroll
  for (int r = 1; r < P; ++r) smax = fmaxf(smax, s[r]);
  if (__builtin_expect(smax < ECHO_DEQUANT_FMA_MAX_SCALE, 1)) {
#pragma unroll
    for (int r = 0; r < P; ++r) {
      const uint32_t x = w[r] ^ 0x88888888u;
      const uint32_t lo = x & 0x0F0F0F0Fu;         // elements 0, 2, 4, 6
      const uint32_t hi = (x >> 4) & 0x0F0F0F0Fu;  // elements 1, 3, 5, 7
      const float m8 = -8.0f * s[r];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        d[r][2 * j] = echo_dequant_fma(static_cast<float>((lo >> (8 * j)) & 0xFFu), s[r], m8);
        d[r][2 * j + 1] = echo_dequant_fma(static_cast<float>((hi >> (8 * j)) & 0xFFu), s[r], m8);
      }
    }
  } else {
#pragma unroll
    for (int r = 0; r < P; ++r)
#pragma unroll
      for (int j = 0; j < 8; ++j) d[r][j] = static_cast<float>(nibble(w[r], j)) * s[r];
  }
}

__device__ __forceinline__ float absmax8(const float (&v)[8]) {
  float m = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) m = fmaxf(m, __builtin_fabsf(v[j]));
  return m;
}

// A chunk of 8 input elements as loaded: 16 B of bf16 or 32 B of fp32.
template <bool BF16>
struct Raw {
  u32x4 q[BF16 ? 1 : 2];
};

template <bool BF16, bool NT>
__device__ __forceinline__ Raw<BF16> load_raw(const void* base, int64_t c) {
  const u32x4* p = static_cast<const u32x4*>(base) + c * (BF16 ? 1 : 2);
  Raw<BF16> r;
#pragma unroll
  for (int i = 0; i < (BF16 ? 1 : 2); ++i) r.q[i] = ld<NT>(p + i);
  return r;
}

template <bool BF16>
__device__ __forceinline__ void widen(const Raw<BF16>& r, float (&v)[8]) {
  if constexpr (BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(r.q[0][i] << 16);
      v[2 * i + 1] = __uint_as_float(r.q[0][i] & 0xFFFF0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = __uint_as_float(r.q[i >> 2][i & 3]);
  }
}

// Eight fp32 values rounded to bfloat16 (nearest, ties to even: adding
// 0x7FFF plus the lowest kept bit to the binary32 pattern carries into the
// top 16 bits exactly when the dropped part is above half, or half with an
// odd kept part) and packed two per word by one byte permutation.
__device__ __forceinline__ uint32_t bf16_rne_carry(float x) {
  const uint32_t u = __float_as_uint(x);
  return u + 0x7FFFu + ((u >> 16) & 1u);  // the bfloat16 is the top 16 bits (finite x)
}

__device__ __forceinline__ uint16_t bf16_rne(float x) {
  return static_cast<uint16_t>(bf16_rne_carry(x) >> 16);
}

__device__ __forceinline__ u32x4 pack_bf16x8(const float (&m)[8]) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)  // hi's top half : lo's top half
    w[i] = __builtin_amdgcn_perm(bf16_rne_carry(m[2 * i + 1]), bf16_rne_carry(m[2 * i]), 0x07060302u);
  return u32x4{w[0], w[1], w[2], w[3]};
}

}  // namespace
}  // namespace echo
