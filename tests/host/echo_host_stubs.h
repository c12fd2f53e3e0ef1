// Record of the launches the C-ABI host code makes when it runs against the
// host-only stand-ins of echo_host_stubs.cpp.
#pragma once

#include <vector>

#include "echo_internal.h"

struct HostLaunch {
  enum Kind { kStage1, kOwner, kDecode, kZero, kGemm } kind;
  echo::Stage1Args stage1;
  echo::OwnerArgs owner;
  echo::GemmArgs gemm;
  const uint32_t* codes;  // decode: broadcast codes
  const float* scales;    // decode: broadcast scales
  void* out;              // decode: output; zero: the filled floats
  int64_t n;              // decode: elements; zero: floats
  int P, group;
  bool flag;              // stage 1: bf16 input; owner: compensate; decode: bf16 output; gemm: fused
  bool state_bf16, own_exact;
};

extern std::vector<HostLaunch> g_launches;
extern int g_device;  // what hipGetDevice reports
// Failure injection: the launch attempt whose index (counted from 0 since
// g_attempts was last cleared) equals g_fail_at returns hipErrorLaunchFailure
// and records nothing; -1 = every launch succeeds.
extern int g_fail_at;
// Where the stand-in of the library's static scratch lives.
constexpr unsigned long long kFakeScratch = 1ull << 50;
namespace echo {
hipError_t static_scratch(int device, void** ptr);
}
extern int g_attempts;
