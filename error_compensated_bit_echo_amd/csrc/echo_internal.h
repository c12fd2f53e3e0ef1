// Internal interface between the C-ABI host code and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace echo {

constexpr int kMaxRanks = 16;
constexpr int kGroup = 32;
constexpr int kElemsPerLane = 8;   // stage 1 / owner: one lane owns 8 consecutive elements
constexpr int kBlock = 256;

// Stage 1: quantize P rank partials into their payload buffers.
struct Stage1Args {
  const void* src[kMaxRanks];  // rank partials (bf16 or fp32), 16-byte aligned
  uint32_t* codes;             // rank r at codes + r * codes_stride_words
  float* scales;               // rank r at scales + r * scales_stride
  int64_t codes_stride_words;  // uint32 words between ranks
  int64_t scales_stride;       // floats between ranks
  int64_t nchunk;              // N / 8
  float* err;                  // sender feedback: rank r's stage-1 error at err + r * err_stride
  int64_t err_stride;          // 4-byte words between ranks (err == nullptr: no sender feedback)
  int32_t err_bf16;            // the errors are kept as bfloat16 bits (with the bf16 state), else fp32
  int64_t own_chunks;          // own_exact: chunks per owner segment, rank r skips chunks
                               // [r * own_chunks, (r + 1) * own_chunks); 0: nothing skipped
};

// Owner stage: sum, correct, re-quantize, update the compensator.
struct OwnerArgs {
  const uint32_t* codes1[kMaxRanks];  // stage-1 codes of rank r
  const float* scales1[kMaxRanks];    // stage-1 scales of rank r
  uint32_t* codes2;
  float* scales2;
  float* m_fast;  // fp32, or bfloat16 bits when the kernel's SB16 switch is on
  float* m_slow;
  int64_t nchunk;
  float beta_fast, omega_fast, beta_slow, omega_slow;
  int32_t out_bf16;              // error measured against bf16(B), the delivered value
  int32_t own_bf16;              // own_exact: the partials are bfloat16 (else fp32)
  int64_t own_chunks;            // own_exact: chunks per owner segment (owner of chunk c
                                 // is min(c / own_chunks, P - 1)); 0 when off
  const void* own_src[kMaxRanks];  // own_exact: the rank partials
  int32_t streaming;             // 1: the streaming cache policy (non-temporal codes and
                                 // estimate stores); 0: every access plain
};

// Cache policy of a call, from the bytes it touches: streaming (its data does not
// stay in the last-level cache between the stages), cached (stage 1 and the owner
// access memory plainly), or cached with the partials read non-temporally.
// launch_stage1 takes the policy; the owner (OwnerArgs::streaming) and
// launch_decode only distinguish streaming from the cached two.
enum CallPolicy { kCallCached = 0, kCallCachedStreamIn = 1, kCallStreaming = 2 };
CallPolicy call_policy(int P, int64_t numel, bool bf16_input);
// group: 32, 64 or 128 elements per scale
hipError_t launch_stage1(const Stage1Args& a, int P, bool bf16, int group, CallPolicy policy,
                         hipStream_t s);
// state_bf16: m_fast / m_slow hold bfloat16 (the variant), else fp32;
// own_exact: a.own_src / a.own_chunks are set
hipError_t launch_owner(const OwnerArgs& a, int P, bool compensate, int group, bool state_bf16,
                        bool own_exact, hipStream_t s);
// the owner launches by rank count, two per compilation unit (echo_owner_p*.hip)
hipError_t launch_owner_p1_2(const OwnerArgs& a, int P, bool compensate, int group, bool state_bf16,
                             bool own_exact, hipStream_t s);
hipError_t launch_owner_p3_4(const OwnerArgs& a, int P, bool compensate, int group, bool state_bf16,
                             bool own_exact, hipStream_t s);
hipError_t launch_owner_p5_6(const OwnerArgs& a, int P, bool compensate, int group, bool state_bf16,
                             bool own_exact, hipStream_t s);
hipError_t launch_owner_p7_8(const OwnerArgs& a, int P, bool compensate, int group, bool state_bf16,
                             bool own_exact, hipStream_t s);
hipError_t launch_owner_p9_10(const OwnerArgs& a, int P, bool compensate, int group, bool state_bf16,
                             bool own_exact, hipStream_t s);
hipError_t launch_owner_p11_12(const OwnerArgs& a, int P, bool compensate, int group, bool state_bf16,
                             bool own_exact, hipStream_t s);
hipError_t launch_owner_p13_14(const OwnerArgs& a, int P, bool compensate, int group, bool state_bf16,
                             bool own_exact, hipStream_t s);
hipError_t launch_owner_p15_16(const OwnerArgs& a, int P, bool compensate, int group, bool state_bf16,
                             bool own_exact, hipStream_t s);
// out: N fp32, or N bfloat16 when out_bf16
hipError_t launch_decode(const uint32_t* codes, const float* scales, void* out,
                         int64_t numel, int group, bool out_bf16, bool streaming, hipStream_t s);
hipError_t launch_zero(float* p, int64_t n_floats, hipStream_t s);

// The producing product partial_r = bf16(A_r * W_r^T) of every rank (A_r [M, K],
// W_r [H, K], bf16 row-major; M % 64 == 0, H % 128 == 0, K % 64 == 0), either
// written out (out[r], [M, H] bf16) or quantized in the epilogue into the
// stage-1 payload (codes / scales as in Stage1Args, group 32; with err set, the
// rank's stage-1 error is added first and updated, as stage 1 does).
struct GemmArgs {
  const uint16_t* A[kMaxRanks];
  const uint16_t* W[kMaxRanks];
  uint16_t* out[kMaxRanks];
  uint32_t* codes;
  float* scales;
  int64_t codes_stride_words;
  int64_t scales_stride;
  int64_t M, K, H;
  float* err;           // fused with sender feedback: rank r's stage-1 error at err + r * err_stride
  int64_t err_stride;   // 4-byte words between ranks (err == nullptr: no sender feedback)
  int32_t err_bf16;     // the errors are bfloat16 bits (with the bf16 state), else fp32
};
// kGemmTileM x kGemmTileN: the tile unit the launcher counts; M must be a
// multiple of kGemmRowStep, H of kGemmTileN and K of kGemmTileK.
constexpr int kGemmTileM = 128, kGemmTileN = 128, kGemmTileK = 64, kGemmRowStep = 64;
hipError_t launch_gemm(const GemmArgs& a, int P, bool fused, hipStream_t s);

}  // namespace echo
