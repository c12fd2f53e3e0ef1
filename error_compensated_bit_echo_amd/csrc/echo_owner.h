// Owner-stage kernel of the Echo all-reduce (gfx950), shared by the units
// that instantiate it for four rank counts each (so that they compile in
// parallel): decode the P stage-1 payloads, add them in fp32 in rank order,
// add the correction, re-quantize and update the two error estimates.
//
// Method: rit.work blog post "echo-4-bit-gpu-communication", section «Как Echo
// возвращает ошибку в следующие вызовы»; heraldofai.com «Come Echo permette ai
// modelli AI…», section «Come Echo evita che gli errori si accumulino».  Every
// floating-point step is its own binary32 operation (contraction off).
#pragma once

#pragma clang fp contract(off)

#include "echo_device.h"

namespace echo {
namespace {

// ---------------------------------------------------------------------------
// Owner stage, all segments at once: decode P payloads, fp32 sum in rank
// order, correction, stage-2 quantization, error and both estimates.
// grid = ceil(nchunk / (256*U)); a lane takes chunks c0 + u*256, u < U, and
// issues the loads of all U before the first use.
// ---------------------------------------------------------------------------
// OWN: the owner of the chunk adds its own partial exactly (the chunk's
// owner is the number of segment starts r * own_chunks, r = 1..P-1, at or
// below c); its payload slot, which stage 1 left unwritten, is not read.
// The loads of U chunks and their arithmetic are two separate loops over
// plain per-chunk register arrays (no array of aggregates, which the
// compiler would keep in scratch memory).
template <int P, bool COMP, int POL, int LPG, bool SB16, bool OWN, int U, bool FULL>
__device__ __forceinline__ void owner_tile(const OwnerArgs& a, int64_t c0) {
  uint32_t w[U][P];    // stage-1 code words of the P ranks
  float s[U][P];       // their scales
  f32x4 mf4[U][2], ms4[U][2];  // the estimates (bfloat16 pairs in [0] with SB16)
  u32x4 xo[U][2];      // OWN: the owner's own raw chunk (16 B bf16 or 32 B fp32)
  int owner[U];        // OWN: the rank that owns the chunk

#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t c = c0 + static_cast<int64_t>(u) * kBlock;
    const int64_t g = c >> log2i(LPG);
    const bool ok = FULL || c < a.nchunk;
    owner[u] = -1;
    const void* own = a.own_src[0];
    if constexpr (OWN) {
      owner[u] = 0;
#pragma unroll
      for (int r = 1; r < P; ++r) owner[u] += c >= a.own_chunks * r ? 1 : 0;
#pragma unroll
      for (int r = 1; r < P; ++r) own = owner[u] == r ? a.own_src[r] : own;
    }
    xo[u][0] = xo[u][1] = u32x4{0u, 0u, 0u, 0u};
    if (ok) {
#pragma unroll
      for (int r = 0; r < P; ++r) {
        if (!OWN || r != owner[u]) {
          w[u][r] = ld<(POL & kNtIn) != 0>(a.codes1[r] + c);
          s[u][r] = a.scales1[r][g];
        } else {
          w[u][r] = 0;
          s[u][r] = 0.0f;
        }
      }
      if constexpr (OWN) {
        const u32x4* p = static_cast<const u32x4*>(own);
        if (a.own_bf16) {
          xo[u][0] = p[c];
        } else {
          xo[u][0] = p[2 * c];
          xo[u][1] = p[2 * c + 1];
        }
      }
      if constexpr (COMP) {
        constexpr bool nt = (POL & kNtStateLd) != 0;
        if constexpr (SB16) {
          // 8 bfloat16 per vector and lane: one 16-byte load each, widened later
          mf4[u][0] = __builtin_bit_cast(f32x4, ld<nt>(reinterpret_cast<const u32x4*>(a.m_fast) + c));
          ms4[u][0] = __builtin_bit_cast(f32x4, ld<nt>(reinterpret_cast<const u32x4*>(a.m_slow) + c));
        } else {
          const f32x4* pf = reinterpret_cast<const f32x4*>(a.m_fast) + 2 * c;
          const f32x4* ps = reinterpret_cast<const f32x4*>(a.m_slow) + 2 * c;
          mf4[u][0] = ld<nt>(pf);
          mf4[u][1] = ld<nt>(pf + 1);
          ms4[u][0] = ld<nt>(ps);
          ms4[u][1] = ld<nt>(ps + 1);
        }
      }
    } else {
#pragma unroll
      for (int r = 0; r < P; ++r) {
        w[u][r] = 0;
        s[u][r] = 0.0f;
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) mf4[u][i] = ms4[u][i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
  }

#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t c = c0 + static_cast<int64_t>(u) * kBlock;
    const int64_t g = c >> log2i(LPG);
    const bool ok = FULL || c < a.nchunk;
    float d[P][8];
    dequant_ranks<P>(w[u], s[u], d);
    if constexpr (OWN) {
      float x[8];
      if (a.own_bf16) {
        Raw<true> rb;
        rb.q[0] = xo[u][0];
        widen<true>(rb, x);
      } else {
        Raw<false> rf;
        rf.q[0] = xo[u][0];
        rf.q[1] = xo[u][1];
        widen<false>(rf, x);
      }
#pragma unroll
      for (int r = 0; r < P; ++r)
#pragma unroll
        for (int k = 0; k < 8; ++k) d[r][k] = r == owner[u] ? x[k] : d[r][k];
    }
    float mf[8], ms[8], V[8];
    if constexpr (COMP && SB16) {
      Raw<true> rf, rs;
      rf.q[0] = __builtin_bit_cast(u32x4, mf4[u][0]);
      rs.q[0] = __builtin_bit_cast(u32x4, ms4[u][0]);
      widen<true>(rf, mf);
      widen<true>(rs, ms);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        mf[j] = mf4[u][j >> 2][j & 3];
        ms[j] = ms4[u][j >> 2][j & 3];
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
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
}

template <int P, bool COMP, int POL, int LPG, bool SB16, bool OWN, int U>
__global__ __launch_bounds__(kBlock) void echo_owner_k(const OwnerArgs a) {
  const int64_t cb = static_cast<int64_t>(blockIdx.x) * (kBlock * U);
  if (cb + kBlock * U <= a.nchunk)
    owner_tile<P, COMP, POL, LPG, SB16, OWN, U, true>(a, cb + threadIdx.x);
  else
    owner_tile<P, COMP, POL, LPG, SB16, OWN, U, false>(a, cb + threadIdx.x);
}

// Cache policy of the owner's accesses in streaming calls (OwnerArgs::streaming),
// chosen by measuring the whole call (stage 1, owner, decode back to back, 1 GiB
// at P = 8): non-temporal loads of the stage-1 codes and non-temporal stores of
// the broadcast codes and of the estimates, plain loads of the estimates
// (non-temporal ones made the kernel 14 % slower).  Against plain accesses the
// owner takes 2.12 instead of 2.19 ms.  Calls whose data mostly stays in the
// last-level cache run every access plain.  The policy is a template parameter:
// a run-time switch between two loads that differ only in their cache hint is
// merged by the compiler into one plain load.
constexpr int kOwnerPolStreaming = kNtIn | kNtOut | kNtStateSt;
constexpr int kOwnerPolCached = 0;

// Chunks per lane, chosen by measurement (1 GiB messages at P = 2, 4 and 8,
// 512 MiB at P = 16): two is within 1 % of the best everywhere and up to 5 %
// faster than one, except for the owner's own share above 8 ranks, where the
// extra registers halve the occupancy and one chunk per lane is 20 % faster.
// Small messages take one chunk per lane whatever the rank count: below 2^18
// chunks (2^21 elements) two per lane would launch fewer than two blocks per
// CU and leave CUs idle (at P = 8, 2^18 elements: 3.7 us against 4.6).
template <int P, bool OWN>
constexpr int owner_unroll() { return OWN && P > 8 ? 1 : 2; }
constexpr int64_t kOwnerSmallChunks = int64_t(1) << 18;

template <int P, int LPG, bool OWN, int U, int POL>
hipError_t owner_pgou(const OwnerArgs& a, bool comp, bool sb16, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((a.nchunk + kBlock * U - 1) / (kBlock * U)));
  // without compensation the state is not touched, so its dtype does not matter
  if (!comp)
    hipLaunchKernelGGL((echo_owner_k<P, false, POL, LPG, false, OWN, U>), grid, dim3(kBlock), 0, s, a);
  else if (sb16)
    hipLaunchKernelGGL((echo_owner_k<P, true, POL, LPG, true, OWN, U>), grid, dim3(kBlock), 0, s, a);
  else
    hipLaunchKernelGGL((echo_owner_k<P, true, POL, LPG, false, OWN, U>), grid, dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

template <int P, int LPG, bool OWN, int POL>
hipError_t owner_pgop(const OwnerArgs& a, bool comp, bool sb16, hipStream_t s) {
  constexpr int U = owner_unroll<P, OWN>();
  if (U == 1 || a.nchunk < kOwnerSmallChunks) return owner_pgou<P, LPG, OWN, 1, POL>(a, comp, sb16, s);
  return owner_pgou<P, LPG, OWN, U, POL>(a, comp, sb16, s);
}

template <int P, int LPG, bool OWN>
hipError_t owner_pgo(const OwnerArgs& a, bool comp, bool sb16, hipStream_t s) {
  if (a.streaming) return owner_pgop<P, LPG, OWN, kOwnerPolStreaming>(a, comp, sb16, s);
  return owner_pgop<P, LPG, OWN, kOwnerPolCached>(a, comp, sb16, s);
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

}  // namespace
}  // namespace echo
