// HIP kernels (gfx950) of the Echo error-compensated int4 all-reduce.
//
// Method: rit.work blog post "echo-4-bit-gpu-communication", section «Как Echo
// возвращает ошибку в следующие вызовы» (segments travel as 4-bit integers,
// the owner sums in high precision, measures the error of its own rounding and
// feeds two smoothed estimates of it into later calls, every element rounded
// at most twice); heraldofai.com «Come Echo permette ai modelli AI…», section
// «Come Echo evita che gli errori si accumulino».
//
// Stage-1 and owner layout.  A lane owns 8 consecutive elements (a "chunk");
// the LPG = group/8 aligned lanes of a group (4 for the default group of 32;
// 8 and 16 for the group-size variants 64 and 128) combine its absmax with
// DPP lane permutations (no LDS traffic).
// A chunk's 8 int4 codes are one 32-bit word (element j in bits 4j..4j+3).
// Every kernel has a bounds-check-free path for whole tiles, which issues all
// of a lane's global loads before the first use, and a guarded path that only
// the last block of a launch takes.
//
// Every floating-point step is a separate IEEE binary32 operation with round
// to nearest even: the file is compiled with contraction off (also pinned by
// the pragma below) and with denormals preserved, so results are bit-identical
// to any other faithful evaluation of the same sequence of operations.  The
// only fused multiply-adds are those of the exact division by 7 (echo_div7.h),
// the sign-exact residual tests of the code choice and the dequantization
// fma((q + 8), s, -8s), which rounds once to exactly fl(q * s) (echo_quant.h);
// no other value of the method's arithmetic chain (sums, correction, error,
// estimates) is fused.
#pragma clang fp contract(off)

#include "echo_device.h"

namespace echo {
namespace {

// ---------------------------------------------------------------------------
// Stage 1 (every rank): partial -> int4 codes + fp32 group scales.
// grid = (ceil(nchunk / (256*U)), P); a block covers 256*U chunks of one rank,
// chunk c0 + u*256 for lane c0.
// ---------------------------------------------------------------------------
// Chunks in [skip_lo, skip_hi) are neither read nor written (the rank's own
// segment when the owner adds its partial exactly); the whole-tile path is only
// taken by tiles that do not meet that range.
template <bool BF16, int U, int POL, int LPG, bool SFB, bool FULL>
__device__ __forceinline__ void stage1_tile(const void* src, uint32_t* codes, float* scales,
                                            float* err, int64_t c0, int64_t nchunk,
                                            int64_t skip_lo, int64_t skip_hi) {
  Raw<BF16> raw[U];
  f32x4 ev[SFB ? U : 1][2];  // sender feedback: the rank's stage-1 error of these elements
  auto live = [&](int64_t c) { return FULL || (c < nchunk && (c < skip_lo || c >= skip_hi)); };
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t c = c0 + static_cast<int64_t>(u) * kBlock;
    if (live(c)) {
      raw[u] = load_raw<BF16, (POL & kNtIn) != 0>(src, c);
      if constexpr (SFB) {
        ev[u][0] = reinterpret_cast<const f32x4*>(err)[2 * c];
        ev[u][1] = reinterpret_cast<const f32x4*>(err)[2 * c + 1];
      }
    } else {
#pragma unroll
      for (int i = 0; i < (BF16 ? 1 : 2); ++i) raw[u].q[i] = u32x4{0u, 0u, 0u, 0u};
      if constexpr (SFB) ev[u][0] = ev[u][1] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t c = c0 + static_cast<int64_t>(u) * kBlock;
    float v[8];
    widen<BF16>(raw[u], v);
    if constexpr (SFB) {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = v[j] + ev[u][j >> 2][j & 3];  // x' = fl(x + e)
    }
    const float s = echo_div7(group_max<LPG>(absmax8(v)));
    float kf[8];
    const uint32_t w = quantize8(v, s, kf);
    if (live(c)) {
      st<(POL & kNtOut) != 0>(w, codes + c);
      if ((threadIdx.x & (LPG - 1)) == 0) scales[c >> log2i(LPG)] = s;
      if constexpr (SFB) {
        float e[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) e[j] = v[j] - kf[j] * s;  // e = x' - fl(q*s), exact
        reinterpret_cast<f32x4*>(err)[2 * c] = f32x4{e[0], e[1], e[2], e[3]};
        reinterpret_cast<f32x4*>(err)[2 * c + 1] = f32x4{e[4], e[5], e[6], e[7]};
      }
    }
  }
}

template <bool BF16, int U, int POL, int LPG, bool SFB>
__global__ __launch_bounds__(kBlock) void echo_quant_pack_k(const Stage1Args a) {
  const int r = blockIdx.y;
  const void* src = a.src[0];
#pragma unroll
  for (int i = 1; i < kMaxRanks; ++i)
    if (r == i) src = a.src[i];
  uint32_t* codes = a.codes + static_cast<int64_t>(r) * a.codes_stride_words;
  float* scales = a.scales + static_cast<int64_t>(r) * a.scales_stride;
  float* err = SFB ? a.err + static_cast<int64_t>(r) * a.err_stride : nullptr;
  const int64_t cb = static_cast<int64_t>(blockIdx.x) * (kBlock * U);
  const int64_t ce = cb + kBlock * U;
  const int64_t skip_lo = a.own_chunks * r, skip_hi = skip_lo + a.own_chunks;
  if (cb >= skip_lo && ce <= skip_hi) return;  // the whole tile is the rank's own segment
  const int64_t c0 = cb + threadIdx.x;
  if (ce <= a.nchunk && (ce <= skip_lo || cb >= skip_hi))
    stage1_tile<BF16, U, POL, LPG, SFB, true>(src, codes, scales, err, c0, a.nchunk, 0, 0);
  else
    stage1_tile<BF16, U, POL, LPG, SFB, false>(src, codes, scales, err, c0, a.nchunk, skip_lo,
                                               skip_hi);
}

// ---------------------------------------------------------------------------
// Owner stage, all segments at once: decode P payloads, fp32 sum in rank
// order, correction, stage-2 quantization, error and both estimates.
// grid = ceil(nchunk / 256); one lane per chunk.
// ---------------------------------------------------------------------------
// OWN: the owner of the chunk adds its own partial exactly (the chunk's
// owner is the number of segment starts r * own_chunks, r = 1..P-1, at or
// below c); its payload slot, which stage 1 left unwritten, is not read.
template <int P, bool COMP, int POL, int LPG, bool SB16, bool OWN, bool FULL>
__device__ __forceinline__ void owner_tile(const OwnerArgs& a, int64_t c) {
  const bool ok = FULL || c < a.nchunk;
  const int64_t g = c >> log2i(LPG);

  int owner = -1;
  const void* own = a.own_src[0];
  if constexpr (OWN) {
    owner = 0;
#pragma unroll
    for (int r = 1; r < P; ++r) owner += c >= a.own_chunks * r ? 1 : 0;
#pragma unroll
    for (int r = 1; r < P; ++r) own = owner == r ? a.own_src[r] : own;
  }

  uint32_t w[P];
  float s[P];
  f32x4 mf4[2], ms4[2];
  u32x4 xo[2] = {u32x4{0u, 0u, 0u, 0u}, u32x4{0u, 0u, 0u, 0u}};  // OWN: the owner's raw chunk
  if (ok) {
#pragma unroll
    for (int r = 0; r < P; ++r) {
      if (!OWN || r != owner) {
        w[r] = ld<(POL & kNtIn) != 0>(a.codes1[r] + c);
        s[r] = a.scales1[r][g];
      } else {
        w[r] = 0;
        s[r] = 0.0f;
      }
    }
    if constexpr (OWN) {
      const u32x4* p = static_cast<const u32x4*>(own);
      if (a.own_bf16) {
        xo[0] = p[c];
      } else {
        xo[0] = p[2 * c];
        xo[1] = p[2 * c + 1];
      }
    }
    if constexpr (COMP) {
      constexpr bool nt = (POL & kNtStateLd) != 0;
      if constexpr (SB16) {
        // 8 bfloat16 per vector and lane: one 16-byte load each, widened exactly
        Raw<true> rf, rs;
        rf.q[0] = ld<nt>(reinterpret_cast<const u32x4*>(a.m_fast) + c);
        rs.q[0] = ld<nt>(reinterpret_cast<const u32x4*>(a.m_slow) + c);
        float f[8], g[8];
        widen<true>(rf, f);
        widen<true>(rs, g);
        mf4[0] = f32x4{f[0], f[1], f[2], f[3]};
        mf4[1] = f32x4{f[4], f[5], f[6], f[7]};
        ms4[0] = f32x4{g[0], g[1], g[2], g[3]};
        ms4[1] = f32x4{g[4], g[5], g[6], g[7]};
      } else {
        const f32x4* pf = reinterpret_cast<const f32x4*>(a.m_fast) + 2 * c;
        const f32x4* ps = reinterpret_cast<const f32x4*>(a.m_slow) + 2 * c;
        mf4[0] = ld<nt>(pf);
        mf4[1] = ld<nt>(pf + 1);
        ms4[0] = ld<nt>(ps);
        ms4[1] = ld<nt>(ps + 1);
      }
    }
  } else {
#pragma unroll
    for (int r = 0; r < P; ++r) {
      w[r] = 0;
      s[r] = 0.0f;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) mf4[i] = ms4[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }

  float d[P][8];
  dequant_ranks<P>(w, s, d);
  if constexpr (OWN) {
    float x[8];
    if (a.own_bf16) {
      Raw<true> rb;
      rb.q[0] = xo[0];
      widen<true>(rb, x);
    } else {
      Raw<false> rf;
      rf.q[0] = xo[0];
      rf.q[1] = xo[1];
      widen<false>(rf, x);
    }
#pragma unroll
    for (int r = 0; r < P; ++r)
#pragma unroll
      for (int k = 0; k < 8; ++k) d[r][k] = r == owner ? x[k] : d[r][k];
  }
  float mf[8], ms[8], V[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    mf[j] = mf4[j >> 2][j & 3];
    ms[j] = ms4[j >> 2][j & 3];
    float S = d[0][j];
#pragma unroll
    for (int r = 1; r < P; ++r) S = S + d[r][j];
    if constexpr (COMP) {
      const float corr = 0.5f * mf[j] + 0.5f * ms[j];
      V[j] = S + corr;
    } else {
      V[j] = S;
    }
  }

  const float s2 = echo_div7(group_max<LPG>(absmax8(V)));
  float kf[8];
  const uint32_t w2 = quantize8(V, s2, kf);
  if (ok) {
    st<(POL & kNtOut) != 0>(w2, a.codes2 + c);
    if ((threadIdx.x & (LPG - 1)) == 0) a.scales2[g] = s2;
    if constexpr (COMP) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float B = kf[j] * s2;
        // with a bfloat16 output the error is that of the value delivered
        const float Bo = a.out_bf16 ? __uint_as_float(bf16_rne_carry(B) & 0xFFFF0000u) : B;
        const float e = V[j] - Bo;
        mf[j] = a.beta_fast * mf[j] + a.omega_fast * e;
        ms[j] = a.beta_slow * ms[j] + a.omega_slow * e;
      }
      constexpr bool nt = (POL & kNtStateSt) != 0;
      if constexpr (SB16) {
        st<nt>(pack_bf16x8(mf), reinterpret_cast<u32x4*>(a.m_fast) + c);
        st<nt>(pack_bf16x8(ms), reinterpret_cast<u32x4*>(a.m_slow) + c);
      } else {
        f32x4* pf = reinterpret_cast<f32x4*>(a.m_fast) + 2 * c;
        f32x4* ps = reinterpret_cast<f32x4*>(a.m_slow) + 2 * c;
        st<nt>(f32x4{mf[0], mf[1], mf[2], mf[3]}, pf);
        st<nt>(f32x4{mf[4], mf[5], mf[6], mf[7]}, pf + 1);
        st<nt>(f32x4{ms[0], ms[1], ms[2], ms[3]}, ps);
        st<nt>(f32x4{ms[4], ms[5], ms[6], ms[7]}, ps + 1);
      }
    }
  }
}

template <int P, bool COMP, int POL, int LPG, bool SB16, bool OWN>
__global__ __launch_bounds__(kBlock) void echo_owner_k(const OwnerArgs a) {
  const int64_t cb = static_cast<int64_t>(blockIdx.x) * kBlock;
  if (cb + kBlock <= a.nchunk)
    owner_tile<P, COMP, POL, LPG, SB16, OWN, true>(a, cb + threadIdx.x);
  else
    owner_tile<P, COMP, POL, LPG, SB16, OWN, false>(a, cb + threadIdx.x);
}

// ---------------------------------------------------------------------------
// Decode of the broadcast payload on every rank: out = fl(q2 * s2), fp32.
// A lane owns 4 consecutive elements (unit i = elements 4i..4i+3, the low or
// high half of code word i/2, group i/8), so each wavefront store writes 1 KiB
// of contiguous output.  grid = ceil(n4 / (256*U)), unit i0 + u*256 for lane i0.
// ---------------------------------------------------------------------------
template <int U, int POL, int LPG, bool FULL>
__device__ __forceinline__ void decode_tile(const uint32_t* codes, const float* scales, float* out,
                                            int64_t i0, int64_t n4) {
  constexpr int kUnitsPerGroupLog2 = log2i(2 * LPG);  // 4-element units per group
  uint32_t w[U];
  float s[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t i = i0 + static_cast<int64_t>(u) * kBlock;
    if (FULL || i < n4) {
      w[u] = ld<(POL & kNtIn) != 0>(codes + (i >> 1));
      s[u] = scales[i >> kUnitsPerGroupLog2];
    } else {
      w[u] = 0;
      s[u] = 0.0f;
    }
  }
  const int half = static_cast<int>(i0 & 1) * 16;  // same parity for every u
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t i = i0 + static_cast<int64_t>(u) * kBlock;
    if (FULL || i < n4) {
      const uint32_t h = w[u] >> half;
      f32x4 o;
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] = static_cast<float>(nibble(h, j)) * s[u];
      st<(POL & kNtOut) != 0>(o, reinterpret_cast<f32x4*>(out) + i);
    }
  }
}

// bfloat16 output: a lane owns a whole code word (8 elements, 16 bytes of
// output), so a wavefront store is again 1 KiB of contiguous output.
// grid = ceil(nchunk / (256*U)), chunk c0 + u*256 for lane c0.
template <int U, int POL, int LPG, bool FULL>
__device__ __forceinline__ void decode_bf16_tile(const uint32_t* codes, const float* scales,
                                                 uint16_t* out, int64_t c0, int64_t nchunk) {
  uint32_t w[U];
  float s[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t c = c0 + static_cast<int64_t>(u) * kBlock;
    if (FULL || c < nchunk) {
      w[u] = ld<(POL & kNtIn) != 0>(codes + c);
      s[u] = scales[c >> log2i(LPG)];
    } else {
      w[u] = 0;
      s[u] = 0.0f;
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t c = c0 + static_cast<int64_t>(u) * kBlock;
    if (FULL || c < nchunk) {
      float b[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) b[k] = static_cast<float>(nibble(w[u], k)) * s[u];
      st<(POL & kNtOut) != 0>(pack_bf16x8(b), reinterpret_cast<u32x4*>(out) + c);
    }
  }
}

template <int U, int POL, int LPG>
__global__ __launch_bounds__(kBlock) void echo_unpack_bf16_k(const uint32_t* __restrict__ codes,
                                                              const float* __restrict__ scales,
                                                              uint16_t* __restrict__ out,
                                                              int64_t nchunk) {
  const int64_t cb = static_cast<int64_t>(blockIdx.x) * (kBlock * U);
  if (cb + kBlock * U <= nchunk)
    decode_bf16_tile<U, POL, LPG, true>(codes, scales, out, cb + threadIdx.x, nchunk);
  else
    decode_bf16_tile<U, POL, LPG, false>(codes, scales, out, cb + threadIdx.x, nchunk);
}

template <int U, int POL, int LPG>
__global__ __launch_bounds__(kBlock) void echo_unpack_k(const uint32_t* __restrict__ codes,
                                                         const float* __restrict__ scales,
                                                         float* __restrict__ out, int64_t n4) {
  const int64_t ib = static_cast<int64_t>(blockIdx.x) * (kBlock * U);
  if (ib + kBlock * U <= n4)
    decode_tile<U, POL, LPG, true>(codes, scales, out, ib + threadIdx.x, n4);
  else
    decode_tile<U, POL, LPG, false>(codes, scales, out, ib + threadIdx.x, n4);
}

__global__ __launch_bounds__(kBlock) void echo_zero_k(float* __restrict__ p, int64_t n) {
  const int64_t i = (static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x) * 4;
  if (i + 4 <= n) {
    *reinterpret_cast<f32x4*>(p + i) = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  } else {
    for (int64_t t = i; t < n; ++t) p[t] = 0.0f;
  }
}

// Tuning of the launches (unroll and cache policy), chosen by measurement.
constexpr int kStage1Unroll = 2;
constexpr int kStage1Pol = kNtIn | kNtOut;
constexpr int kOwnerPol = 0;
constexpr int kDecodeUnroll = 2;
constexpr int kDecodePol = kNtOut;

template <int P, int LPG, bool OWN, int POL = kOwnerPol>
hipError_t owner_pgo(const OwnerArgs& a, bool comp, bool sb16, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((a.nchunk + kBlock - 1) / kBlock));
  // without compensation the state is not touched, so its dtype does not matter
  if (!comp)
    hipLaunchKernelGGL((echo_owner_k<P, false, POL, LPG, false, OWN>), grid, dim3(kBlock), 0, s, a);
  else if (sb16)
    hipLaunchKernelGGL((echo_owner_k<P, true, POL, LPG, true, OWN>), grid, dim3(kBlock), 0, s, a);
  else
    hipLaunchKernelGGL((echo_owner_k<P, true, POL, LPG, false, OWN>), grid, dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

template <int P, int LPG>
hipError_t owner_pg(const OwnerArgs& a, bool comp, bool sb16, bool own, hipStream_t s) {
  return own ? owner_pgo<P, LPG, true>(a, comp, sb16, s) : owner_pgo<P, LPG, false>(a, comp, sb16, s);
}

template <int P>
hipError_t owner_p(const OwnerArgs& a, bool comp, int group, bool sb16, bool own, hipStream_t s) {
  switch (group) {
    case 32: return owner_pg<P, 4>(a, comp, sb16, own, s);
    case 64: return owner_pg<P, 8>(a, comp, sb16, own, s);
    case 128: return owner_pg<P, 16>(a, comp, sb16, own, s);
    default: return hipErrorInvalidValue;
  }
}

template <int U, int POL = kStage1Pol, int LPG = 4, bool SFB = false>
hipError_t stage1_u(const Stage1Args& a, int P, bool bf16, hipStream_t s) {
  const int64_t blocks = (a.nchunk + kBlock * U - 1) / (kBlock * U);
  const dim3 grid(static_cast<unsigned>(blocks), static_cast<unsigned>(P));
  if (bf16)
    hipLaunchKernelGGL((echo_quant_pack_k<true, U, POL, LPG, SFB>), grid, dim3(kBlock), 0, s, a);
  else
    hipLaunchKernelGGL((echo_quant_pack_k<false, U, POL, LPG, SFB>), grid, dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

template <int LPG>
hipError_t stage1_g(const Stage1Args& a, int P, bool bf16, hipStream_t s) {
  if (a.err != nullptr) return stage1_u<kStage1Unroll, kStage1Pol, LPG, true>(a, P, bf16, s);
  return stage1_u<kStage1Unroll, kStage1Pol, LPG, false>(a, P, bf16, s);
}

template <int U, int POL = kDecodePol, int LPG = 4>
hipError_t decode_u(const uint32_t* codes, const float* scales, void* out, int64_t numel,
                    bool out_bf16, hipStream_t s) {
  if (out_bf16) {
    const int64_t nchunk = numel / kElemsPerLane;
    const int64_t blocks = (nchunk + kBlock * U - 1) / (kBlock * U);
    hipLaunchKernelGGL((echo_unpack_bf16_k<U, POL, LPG>), dim3(static_cast<unsigned>(blocks)),
                       dim3(kBlock), 0, s, codes, scales, static_cast<uint16_t*>(out), nchunk);
  } else {
    const int64_t n4 = numel / 4;
    const int64_t blocks = (n4 + kBlock * U - 1) / (kBlock * U);
    hipLaunchKernelGGL((echo_unpack_k<U, POL, LPG>), dim3(static_cast<unsigned>(blocks)), dim3(kBlock),
                       0, s, codes, scales, static_cast<float*>(out), n4);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_stage1(const Stage1Args& a, int P, bool bf16, int group, hipStream_t s) {
  switch (group) {
    case 32: return stage1_g<4>(a, P, bf16, s);
    case 64: return stage1_g<8>(a, P, bf16, s);
    case 128: return stage1_g<16>(a, P, bf16, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_owner(const OwnerArgs& a, int P, bool compensate, int group, bool sb16,
                        bool own, hipStream_t s) {
  switch (P) {
    case 1: return owner_p<1>(a, compensate, group, sb16, own, s);
    case 2: return owner_p<2>(a, compensate, group, sb16, own, s);
    case 3: return owner_p<3>(a, compensate, group, sb16, own, s);
    case 4: return owner_p<4>(a, compensate, group, sb16, own, s);
    case 5: return owner_p<5>(a, compensate, group, sb16, own, s);
    case 6: return owner_p<6>(a, compensate, group, sb16, own, s);
    case 7: return owner_p<7>(a, compensate, group, sb16, own, s);
    case 8: return owner_p<8>(a, compensate, group, sb16, own, s);
    case 9: return owner_p<9>(a, compensate, group, sb16, own, s);
    case 10: return owner_p<10>(a, compensate, group, sb16, own, s);
    case 11: return owner_p<11>(a, compensate, group, sb16, own, s);
    case 12: return owner_p<12>(a, compensate, group, sb16, own, s);
    case 13: return owner_p<13>(a, compensate, group, sb16, own, s);
    case 14: return owner_p<14>(a, compensate, group, sb16, own, s);
    case 15: return owner_p<15>(a, compensate, group, sb16, own, s);
    case 16: return owner_p<16>(a, compensate, group, sb16, own, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode(const uint32_t* codes, const float* scales, void* out, int64_t numel,
                         int group, bool out_bf16, hipStream_t s) {
  switch (group) {
    case 32: return decode_u<kDecodeUnroll, kDecodePol, 4>(codes, scales, out, numel, out_bf16, s);
    case 64: return decode_u<kDecodeUnroll, kDecodePol, 8>(codes, scales, out, numel, out_bf16, s);
    case 128: return decode_u<kDecodeUnroll, kDecodePol, 16>(codes, scales, out, numel, out_bf16, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_zero(float* p, int64_t n_floats, hipStream_t s) {
  const int64_t blocks = (n_floats + kBlock * 4 - 1) / (kBlock * 4);
  hipLaunchKernelGGL(echo_zero_k, dim3(static_cast<unsigned>(blocks)), dim3(kBlock), 0, s, p,
                     n_floats);
  return hipGetLastError();
}

}  // namespace echo
