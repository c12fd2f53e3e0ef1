// HIP kernels (gfx950) of the Echo error-compensated int4 all-reduce: stage 1,
// the decode and the state fill (the owner stage is in echo_owner.h).
//
// Method: rit.work blog post "echo-4-bit-gpu-communication", section «Как Echo
// возвращает ошибку в следующие вызовы» (segments travel as 4-bit integers,
// the owner sums in high precision, measures the error of its own rounding and
// feeds two smoothed estimates of it into later calls, every element rounded
// at most twice); heraldofai.com «Come Echo permette ai modelli AI…», section
// «Come Echo evita che gli errori si accumulino».
//
// Stage-1 and owner layout (shared with echo_owner.h).  A lane owns 8
// consecutive elements (a "chunk");
// the LPG = group/8 aligned lanes of a group (4 for the default group of 32;
// 8 and 16 for the group-size variants 64 and 128) combine its absmax with
// DPP lane permutations (no LDS traffic).
// A chunk's 8 int4 codes are one 32-bit word (element j in bits 4j..4j+3).
// Every kernel has a bounds-check-free path for whole tiles, which issues all
// of a lane's global loads before the first use, and a guarded path that only
// the last block of a launch takes (and, in stage 1, tiles that meet the
// rank's own segment when the owner keeps its partial).
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
// SFB (sender feedback): 0 off; 1 the rank's stage-1 errors are fp32 (32 B per
// chunk); 2 they are bfloat16 (16 B per chunk), each new error rounded to
// nearest even before it is kept.
template <bool BF16, int U, int POL, int LPG, int SFB, bool FULL>
__device__ __forceinline__ void stage1_tile(const void* src, uint32_t* codes, float* scales,
                                            float* err, int64_t c0, int64_t nchunk,
                                            int64_t skip_lo, int64_t skip_hi) {
  Raw<BF16> raw[U];
  Raw<SFB == 2> ev[SFB ? U : 1];  // sender feedback: the rank's stage-1 error of these elements
  auto live = [&](int64_t c) { return FULL || (c < nchunk && (c < skip_lo || c >= skip_hi)); };
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t c = c0 + static_cast<int64_t>(u) * kBlock;
    if (live(c)) {
      raw[u] = load_raw<BF16, (POL & kNtIn) != 0>(src, c);
      if constexpr (SFB != 0) ev[u] = load_raw<SFB == 2, false>(err, c);
    } else {
#pragma unroll
      for (int i = 0; i < (BF16 ? 1 : 2); ++i) raw[u].q[i] = u32x4{0u, 0u, 0u, 0u};
      if constexpr (SFB != 0) {
#pragma unroll
        for (int i = 0; i < (SFB == 2 ? 1 : 2); ++i) ev[u].q[i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t c = c0 + static_cast<int64_t>(u) * kBlock;
    float v[8];
    widen<BF16>(raw[u], v);
    if constexpr (SFB != 0) {
      float e[8];
      widen<SFB == 2>(ev[u], e);
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = v[j] + e[j];  // x' = fl(x + e)
    }
    const float s = echo_div7(group_max<LPG>(absmax8(v)));
    float kf[8];
    const uint32_t w = quantize8(v, s, kf);
    if (live(c)) {
      st<(POL & kNtOut) != 0>(w, codes + c);
      if ((threadIdx.x & (LPG - 1)) == 0) scales[c >> log2i(LPG)] = s;
      if constexpr (SFB != 0) {
        float e[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) e[j] = v[j] - kf[j] * s;  // e = x' - fl(q*s), exact
        if constexpr (SFB == 2) {
          reinterpret_cast<u32x4*>(err)[c] = pack_bf16x8(e);
        } else {
          reinterpret_cast<f32x4*>(err)[2 * c] = f32x4{e[0], e[1], e[2], e[3]};
          reinterpret_cast<f32x4*>(err)[2 * c + 1] = f32x4{e[4], e[5], e[6], e[7]};
        }
      }
    }
  }
}

template <bool BF16, int U, int POL, int LPG, int SFB>
__global__ __launch_bounds__(kBlock) void echo_quant_pack_k(const Stage1Args a) {
  const int r = blockIdx.y;
  const void* src = a.src[0];
#pragma unroll
  for (int i = 1; i < kMaxRanks; ++i)
    if (r == i) src = a.src[i];
  uint32_t* codes = a.codes + static_cast<int64_t>(r) * a.codes_stride_words;
  float* scales = a.scales + static_cast<int64_t>(r) * a.scales_stride;
  float* err = SFB != 0 ? a.err + static_cast<int64_t>(r) * a.err_stride : nullptr;
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

// Tuning of the launches (unroll and cache policy), chosen by measurement of
// the whole call (the kernels back to back, as a call runs them).  Two cache
// policies: streaming calls read the partials and write the stage-1 payload
// non-temporally and the decode stores plainly (right after a streaming owner,
// non-temporal decode stores took 0.44 ms against 0.39 at 1 GiB, P = 8); calls
// whose data stays in the last-level cache between the stages run stage 1 and
// the owner plain, so that the owner finds the payload in the cache, and the
// decode stores non-temporally; the largest of them also read the partials
// non-temporally (see call_policy).
constexpr int kStage1Unroll = 2;
constexpr int kStage1Pol = kNtIn | kNtOut;
constexpr int kDecodeUnroll = 2;
constexpr int kDecodePolStreaming = 0;
constexpr int kDecodePolCached = kNtOut;

template <int U, int POL = kStage1Pol, int LPG = 4, int SFB = 0>
hipError_t stage1_u(const Stage1Args& a, int P, bool bf16, hipStream_t s) {
  const int64_t blocks = (a.nchunk + kBlock * U - 1) / (kBlock * U);
  const dim3 grid(static_cast<unsigned>(blocks), static_cast<unsigned>(P));
  if (bf16)
    hipLaunchKernelGGL((echo_quant_pack_k<true, U, POL, LPG, SFB>), grid, dim3(kBlock), 0, s, a);
  else
    hipLaunchKernelGGL((echo_quant_pack_k<false, U, POL, LPG, SFB>), grid, dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

// Small messages take one chunk per lane: when two per lane would launch fewer
// than 1024 blocks over all ranks (four per CU), one per lane is faster (at
// P = 8, 2^18 elements: 2.9 us against 3.5).
template <int LPG, int POL>
hipError_t stage1_gp(const Stage1Args& a, int P, bool bf16, hipStream_t s) {
  const int64_t blocks = (a.nchunk + kBlock * kStage1Unroll - 1) / (kBlock * kStage1Unroll) * P;
  const int sfb = a.err == nullptr ? 0 : (a.err_bf16 ? 2 : 1);
  if (blocks < 1024) {
    if (sfb == 2) return stage1_u<1, POL, LPG, 2>(a, P, bf16, s);
    if (sfb == 1) return stage1_u<1, POL, LPG, 1>(a, P, bf16, s);
    return stage1_u<1, POL, LPG, 0>(a, P, bf16, s);
  }
  if (sfb == 2) return stage1_u<kStage1Unroll, POL, LPG, 2>(a, P, bf16, s);
  if (sfb == 1) return stage1_u<kStage1Unroll, POL, LPG, 1>(a, P, bf16, s);
  return stage1_u<kStage1Unroll, POL, LPG, 0>(a, P, bf16, s);
}

template <int LPG>
hipError_t stage1_g(const Stage1Args& a, int P, bool bf16, CallPolicy policy, hipStream_t s) {
  switch (policy) {
    case kCallStreaming: return stage1_gp<LPG, kStage1Pol>(a, P, bf16, s);
    case kCallCachedStreamIn: return stage1_gp<LPG, kNtIn>(a, P, bf16, s);
    default: return stage1_gp<LPG, 0>(a, P, bf16, s);
  }
}

template <int U, int POL, int LPG>
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

// Cache policy of a call, from the bytes it touches (stage 1 + owner + decode,
// group 32).  Between 96 MB and 1.2 GB stage 1 and the owner access memory
// plainly, so that much of the stage-1 payload is still in the 256 MB
// last-level cache when the owner reads it: 10-14 % faster than streaming at
// 100-550 MB per call (P = 4 and 8), equal below 96 MB.  From 480 MB on, stage 1
// reads the partials non-temporally so that they do not push the payload out
// of the cache: against all-plain accesses 5-6 % faster at 533-575 MB, equal at
// 466 MB and 3-8 % slower below; against streaming 7-14 % faster at 666-932 MB,
// 2-4 % at 1.06-1.11 GB and equal at 1.2-1.33 GB, while streaming is 1-5 %
// faster from 1.4 GB on (and at 1 GB for P = 16).  P = 2, 4, 8 and 16,
// graph-replayed calls, each comparison measured on one machine.
CallPolicy call_policy(int P, int64_t numel, bool bf16_input) {
  const double bytes = static_cast<double>(numel) * (P * ((bf16_input ? 2.0 : 4.0) + 0.625) + 21.25);
  if (bytes < 96e6 || bytes > 1200e6) return kCallStreaming;
  return bytes >= 480e6 ? kCallCachedStreamIn : kCallCached;
}

hipError_t launch_stage1(const Stage1Args& a, int P, bool bf16, int group, CallPolicy policy,
                         hipStream_t s) {
  switch (group) {
    case 32: return stage1_g<4>(a, P, bf16, policy, s);
    case 64: return stage1_g<8>(a, P, bf16, policy, s);
    case 128: return stage1_g<16>(a, P, bf16, policy, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_owner(const OwnerArgs& a, int P, bool compensate, int group, bool sb16,
                        bool own, hipStream_t s) {
  switch ((P + 1) / 2) {
    case 1: return launch_owner_p1_2(a, P, compensate, group, sb16, own, s);
    case 2: return launch_owner_p3_4(a, P, compensate, group, sb16, own, s);
    case 3: return launch_owner_p5_6(a, P, compensate, group, sb16, own, s);
    case 4: return launch_owner_p7_8(a, P, compensate, group, sb16, own, s);
    case 5: return launch_owner_p9_10(a, P, compensate, group, sb16, own, s);
    case 6: return launch_owner_p11_12(a, P, compensate, group, sb16, own, s);
    case 7: return launch_owner_p13_14(a, P, compensate, group, sb16, own, s);
    case 8: return launch_owner_p15_16(a, P, compensate, group, sb16, own, s);
    default: return hipErrorInvalidValue;
  }
}

// Below 2^20 elements the decode takes one unit per lane (more blocks, fewer
// idle CUs); above, two.
template <int U, int POL>
hipError_t decode_g(const uint32_t* codes, const float* scales, void* out, int64_t numel, int group,
                    bool out_bf16, hipStream_t s) {
  switch (group) {
    case 32: return decode_u<U, POL, 4>(codes, scales, out, numel, out_bf16, s);
    case 64: return decode_u<U, POL, 8>(codes, scales, out, numel, out_bf16, s);
    case 128: return decode_u<U, POL, 16>(codes, scales, out, numel, out_bf16, s);
    default: return hipErrorInvalidValue;
  }
}

template <int POL>
hipError_t decode_p(const uint32_t* codes, const float* scales, void* out, int64_t numel, int group,
                    bool out_bf16, hipStream_t s) {
  if (numel < (int64_t(1) << 20)) return decode_g<1, POL>(codes, scales, out, numel, group, out_bf16, s);
  return decode_g<kDecodeUnroll, POL>(codes, scales, out, numel, group, out_bf16, s);
}

hipError_t launch_decode(const uint32_t* codes, const float* scales, void* out, int64_t numel,
                         int group, bool out_bf16, bool streaming, hipStream_t s) {
  if (streaming) return decode_p<kDecodePolStreaming>(codes, scales, out, numel, group, out_bf16, s);
  return decode_p<kDecodePolCached>(codes, scales, out, numel, group, out_bf16, s);
}

hipError_t launch_zero(float* p, int64_t n_floats, hipStream_t s) {
  const int64_t blocks = (n_floats + kBlock * 4 - 1) / (kBlock * 4);
  hipLaunchKernelGGL(echo_zero_k, dim3(static_cast<unsigned>(blocks)), dim3(kBlock), 0, s, p,
                     n_floats);
  return hipGetLastError();
}

}  // namespace echo
