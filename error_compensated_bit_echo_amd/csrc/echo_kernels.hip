// HIP kernels (gfx950) of the Echo error-compensated int4 all-reduce.
//
// Method: rit.work blog post "echo-4-bit-gpu-communication", section «Как Echo
// возвращает ошибку в следующие вызовы» (segments travel as 4-bit integers,
// the owner sums in high precision, measures the error of its own rounding and
// feeds two smoothed estimates of it into later calls, every element rounded
// at most twice); heraldofai.com «Come Echo permette ai modelli AI…», section
// «Come Echo evita che gli errori si accumulino».
//
// Layout shared by all kernels.  A lane owns 8 consecutive elements (a
// "chunk"); the 4 lanes of an aligned quad own one 32-element group.  The
// group absmax is combined across the quad with two DPP quad permutations, so
// no LDS traffic is needed.  A chunk's 8 int4 codes are one 32-bit word
// (element j of the chunk in bits 4j..4j+3), so a wavefront moves 256
// contiguous bytes of codes per instruction and 1 KiB of bf16 input per
// 128-bit load.
//
// Every floating-point step is a separate IEEE binary32 operation with round
// to nearest even: the file is compiled with contraction off (also pinned by
// the pragma below) and with denormals preserved, so results are bit-identical
// to any other faithful evaluation of the same sequence of operations.
#include "echo_internal.h"

#pragma clang fp contract(off)

namespace echo {
namespace {

// Codes whose quotient t = v * rcp(s) lies this close to a half-integer are
// re-decided exactly.  |t - v/s| < 1.4 * 2^-20 (rcp: 1 ulp, product: 1/2 ulp,
// |v/s| <= 7.0000005), so outside the guard band the rounded t is the correct
// code; inside it the quotient is recomputed in binary64, where it decides
// exactly (a non-tie quotient of two binary32 values is at least 2^-26 from a
// half-integer, and a tie is representable).
constexpr float kTieGuard = 0.5f - 0x1p-17f;
// Below this scale rcp(s) may overflow; such groups take the exact path.
constexpr float kTinyScale = 0x1p-100f;

__device__ __forceinline__ float quad_max(float x) {
  // quad_perm(1,0,3,2) then quad_perm(2,3,0,1): all four lanes get the max.
  int xi = __float_as_int(x);
  float y = __int_as_float(__builtin_amdgcn_update_dpp(xi, xi, 0xB1, 0xF, 0xF, false));
  x = fmaxf(x, y);
  xi = __float_as_int(x);
  y = __int_as_float(__builtin_amdgcn_update_dpp(xi, xi, 0x4E, 0xF, 0xF, false));
  return fmaxf(x, y);
}

// Nearest code in [-7, 7] to the exact quotient v / s (s > 0), ties to even.
__device__ __forceinline__ int exact_code(float v, float s) {
  double q = __builtin_rint(static_cast<double>(v) / static_cast<double>(s));
  q = q > 7.0 ? 7.0 : q;
  q = q < -7.0 ? -7.0 : q;
  return static_cast<int>(q);
}

// Codes of the 8 values a lane holds, for group scale s = fl(absmax / 7).
// k receives the signed codes, the return value the packed nibbles.
__device__ __forceinline__ uint32_t quantize8(const float (&v)[8], float s, int (&k)[8]) {
  if (s >= kTinyScale) {
    const float inv = __builtin_amdgcn_rcpf(s);
    bool near_tie = false;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float t = v[j] * inv;
      const float r = __builtin_rintf(t);
      k[j] = static_cast<int>(r);
      near_tie |= !(__builtin_fabsf(t - r) < kTieGuard);
    }
    if (near_tie) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float t = v[j] * inv;
        const float r = __builtin_rintf(t);
        if (!(__builtin_fabsf(t - r) < kTieGuard)) k[j] = exact_code(v[j], s);
      }
    }
  } else if (s > 0.0f) {
#pragma unroll
    for (int j = 0; j < 8; ++j) k[j] = exact_code(v[j], s);
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) k[j] = 0;
  }
  uint32_t w = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) w |= (static_cast<uint32_t>(k[j]) & 15u) << (4 * j);
  return w;
}

// Signed code of element j (0..7) of a packed chunk word.
__device__ __forceinline__ int nibble(uint32_t w, int j) {
  return static_cast<int>(w << (28 - 4 * j)) >> 28;
}

__device__ __forceinline__ float absmax8(const float (&v)[8]) {
  float m = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) m = fmaxf(m, __builtin_fabsf(v[j]));
  return m;
}

template <bool BF16>
__device__ __forceinline__ void load_chunk(const void* base, int64_t c, float (&v)[8]) {
  if constexpr (BF16) {
    const uint4 x = *reinterpret_cast<const uint4*>(static_cast<const char*>(base) + c * 16);
    const uint32_t u[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(u[i] << 16);
      v[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const char*>(base) + c * 32);
    const float4 a = p[0];
    const float4 b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

// ---------------------------------------------------------------------------
// Stage 1 (every rank): partial -> int4 codes + fp32 group scales.
// grid = (ceil(nchunk / (256*U)), P); one block covers 256*U chunks of one rank.
// ---------------------------------------------------------------------------
template <bool BF16, int U>
__global__ __launch_bounds__(kBlock) void echo_quant_pack_k(const Stage1Args a) {
  const int r = blockIdx.y;
  const void* src = a.src[0];
#pragma unroll
  for (int i = 1; i < kMaxRanks; ++i)
    if (r == i) src = a.src[i];
  uint32_t* codes = a.codes + static_cast<int64_t>(r) * a.codes_stride_words;
  float* scales = a.scales + static_cast<int64_t>(r) * a.scales_stride;
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * (kBlock * U) + threadIdx.x;

  float v[U][8];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t c = c0 + static_cast<int64_t>(u) * kBlock;
    if (c < a.nchunk) {
      load_chunk<BF16>(src, c, v[u]);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[u][j] = 0.0f;
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t c = c0 + static_cast<int64_t>(u) * kBlock;
    const float s = quad_max(absmax8(v[u])) / 7.0f;  // IEEE division
    int k[8];
    const uint32_t w = quantize8(v[u], s, k);
    if (c < a.nchunk) {
      codes[c] = w;
      if ((threadIdx.x & 3) == 0) scales[c >> 2] = s;
    }
  }
}

// ---------------------------------------------------------------------------
// Owner stage, all segments at once: decode P payloads, fp32 sum in rank
// order, correction, stage-2 quantization, error and both estimates.
// grid = ceil(nchunk / 256); one lane per chunk.
// ---------------------------------------------------------------------------
template <int P, bool COMP>
__global__ __launch_bounds__(kBlock) void echo_owner_k(const OwnerArgs a) {
  const int64_t c = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  const bool ok = c < a.nchunk;
  const int64_t g = c >> 2;

  uint32_t w[P];
  float s[P];
  float mf[8], ms[8];
  if (ok) {
#pragma unroll
    for (int r = 0; r < P; ++r) {
      w[r] = a.codes1[r * a.codes_stride_words + c];
      s[r] = a.scales1[r * a.scales_stride + g];
    }
    if constexpr (COMP) {
      const float4* pf = reinterpret_cast<const float4*>(a.m_fast + c * 8);
      const float4* ps = reinterpret_cast<const float4*>(a.m_slow + c * 8);
      const float4 f0 = pf[0], f1 = pf[1], s0 = ps[0], s1 = ps[1];
      mf[0] = f0.x; mf[1] = f0.y; mf[2] = f0.z; mf[3] = f0.w;
      mf[4] = f1.x; mf[5] = f1.y; mf[6] = f1.z; mf[7] = f1.w;
      ms[0] = s0.x; ms[1] = s0.y; ms[2] = s0.z; ms[3] = s0.w;
      ms[4] = s1.x; ms[5] = s1.y; ms[6] = s1.z; ms[7] = s1.w;
    }
  } else {
#pragma unroll
    for (int r = 0; r < P; ++r) { w[r] = 0; s[r] = 0.0f; }
#pragma unroll
    for (int j = 0; j < 8; ++j) { mf[j] = 0.0f; ms[j] = 0.0f; }
  }

  float V[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float S = static_cast<float>(nibble(w[0], j)) * s[0];
#pragma unroll
    for (int r = 1; r < P; ++r) S = S + static_cast<float>(nibble(w[r], j)) * s[r];
    if constexpr (COMP) {
      const float corr = 0.5f * mf[j] + 0.5f * ms[j];
      V[j] = S + corr;
    } else {
      V[j] = S;
    }
  }

  const float s2 = quad_max(absmax8(V)) / 7.0f;  // IEEE division
  int k[8];
  const uint32_t w2 = quantize8(V, s2, k);
  if (ok) {
    a.codes2[c] = w2;
    if ((threadIdx.x & 3) == 0) a.scales2[g] = s2;
    if constexpr (COMP) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float B = static_cast<float>(k[j]) * s2;
        const float e = V[j] - B;
        mf[j] = a.beta_fast * mf[j] + a.omega_fast * e;
        ms[j] = a.beta_slow * ms[j] + a.omega_slow * e;
      }
      float4* pf = reinterpret_cast<float4*>(a.m_fast + c * 8);
      float4* ps = reinterpret_cast<float4*>(a.m_slow + c * 8);
      pf[0] = make_float4(mf[0], mf[1], mf[2], mf[3]);
      pf[1] = make_float4(mf[4], mf[5], mf[6], mf[7]);
      ps[0] = make_float4(ms[0], ms[1], ms[2], ms[3]);
      ps[1] = make_float4(ms[4], ms[5], ms[6], ms[7]);
    }
  }
}

// ---------------------------------------------------------------------------
// Decode of the broadcast payload on every rank: out = fl(q2 * s2), fp32.
// ---------------------------------------------------------------------------
template <int U>
__global__ __launch_bounds__(kBlock) void echo_unpack_k(const uint32_t* __restrict__ codes,
                                                         const float* __restrict__ scales,
                                                         float* __restrict__ out, int64_t nchunk) {
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * (kBlock * U) + threadIdx.x;
  uint32_t w[U];
  float s[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t c = c0 + static_cast<int64_t>(u) * kBlock;
    w[u] = 0;
    s[u] = 0.0f;
    if (c < nchunk) {
      w[u] = codes[c];
      s[u] = scales[c >> 2];
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t c = c0 + static_cast<int64_t>(u) * kBlock;
    if (c < nchunk) {
      float o[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) o[j] = static_cast<float>(nibble(w[u], j)) * s[u];
      float4* p = reinterpret_cast<float4*>(out + c * 8);
      p[0] = make_float4(o[0], o[1], o[2], o[3]);
      p[1] = make_float4(o[4], o[5], o[6], o[7]);
    }
  }
}

__global__ __launch_bounds__(kBlock) void echo_zero_k(float* __restrict__ p, int64_t n) {
  const int64_t i = (static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x) * 4;
  if (i + 4 <= n) {
    *reinterpret_cast<float4*>(p + i) = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  } else {
    for (int64_t t = i; t < n; ++t) p[t] = 0.0f;
  }
}

constexpr int kStage1Unroll = 2;
constexpr int kDecodeUnroll = 2;

template <int P>
hipError_t owner_p(const OwnerArgs& a, bool comp, hipStream_t s) {
  const int64_t blocks = (a.nchunk + kBlock - 1) / kBlock;
  if (comp)
    hipLaunchKernelGGL((echo_owner_k<P, true>), dim3(static_cast<unsigned>(blocks)), dim3(kBlock), 0, s, a);
  else
    hipLaunchKernelGGL((echo_owner_k<P, false>), dim3(static_cast<unsigned>(blocks)), dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_stage1(const Stage1Args& a, int P, bool bf16, hipStream_t s) {
  constexpr int U = kStage1Unroll;
  const int64_t blocks = (a.nchunk + kBlock * U - 1) / (kBlock * U);
  const dim3 grid(static_cast<unsigned>(blocks), static_cast<unsigned>(P));
  if (bf16)
    hipLaunchKernelGGL((echo_quant_pack_k<true, U>), grid, dim3(kBlock), 0, s, a);
  else
    hipLaunchKernelGGL((echo_quant_pack_k<false, U>), grid, dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_owner(const OwnerArgs& a, int P, bool compensate, hipStream_t s) {
  switch (P) {
    case 1: return owner_p<1>(a, compensate, s);
    case 2: return owner_p<2>(a, compensate, s);
    case 3: return owner_p<3>(a, compensate, s);
    case 4: return owner_p<4>(a, compensate, s);
    case 5: return owner_p<5>(a, compensate, s);
    case 6: return owner_p<6>(a, compensate, s);
    case 7: return owner_p<7>(a, compensate, s);
    case 8: return owner_p<8>(a, compensate, s);
    case 9: return owner_p<9>(a, compensate, s);
    case 10: return owner_p<10>(a, compensate, s);
    case 11: return owner_p<11>(a, compensate, s);
    case 12: return owner_p<12>(a, compensate, s);
    case 13: return owner_p<13>(a, compensate, s);
    case 14: return owner_p<14>(a, compensate, s);
    case 15: return owner_p<15>(a, compensate, s);
    case 16: return owner_p<16>(a, compensate, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode(const uint32_t* codes, const float* scales, float* out, int64_t nchunk,
                         hipStream_t s) {
  constexpr int U = kDecodeUnroll;
  const int64_t blocks = (nchunk + kBlock * U - 1) / (kBlock * U);
  hipLaunchKernelGGL((echo_unpack_k<U>), dim3(static_cast<unsigned>(blocks)), dim3(kBlock), 0, s,
                     codes, scales, out, nchunk);
  return hipGetLastError();
}

hipError_t launch_zero(float* p, int64_t n_floats, hipStream_t s) {
  const int64_t blocks = (n_floats + kBlock * 4 - 1) / (kBlock * 4);
  hipLaunchKernelGGL(echo_zero_k, dim3(static_cast<unsigned>(blocks)), dim3(kBlock), 0, s, p,
                     n_floats);
  return hipGetLastError();
}

}  // namespace echo
