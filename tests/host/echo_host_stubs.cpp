// Host-only stand-ins for the device side of libecho, so that the C-ABI host
// code (validation, workspace carving, launch arguments) can run on a machine
// without a GPU: every launch is recorded instead of enqueued, and the one HIP
// runtime call the host code makes reports device 0.  Used by
// echo_host_check.cpp; never linked into libecho.
#include <vector>

#include "echo_host_stubs.h"

std::vector<HostLaunch> g_launches;
int g_device = 0;
int g_fail_at = -1;
int g_attempts = 0;

namespace {
bool fails_now() { return g_attempts++ == g_fail_at; }
}  // namespace

extern "C" hipError_t hipGetDevice(int* device) {
  if (device == nullptr) return hipErrorInvalidValue;
  *device = g_device;
  return hipSuccess;
}

namespace echo {

CallPolicy call_policy(int, int64_t, bool) { return kCallStreaming; }

hipError_t launch_stage1(const Stage1Args& a, int P, bool bf16, int group, CallPolicy, hipStream_t) {
  if (fails_now()) return hipErrorLaunchFailure;
  HostLaunch l{};
  l.kind = HostLaunch::kStage1;
  l.stage1 = a;
  l.P = P;
  l.flag = bf16;
  l.group = group;
  g_launches.push_back(l);
  return hipSuccess;
}

hipError_t launch_owner(const OwnerArgs& a, int P, bool compensate, int group, bool state_bf16,
                        bool own_exact, hipStream_t) {
  if (fails_now()) return hipErrorLaunchFailure;
  HostLaunch l{};
  l.kind = HostLaunch::kOwner;
  l.owner = a;
  l.P = P;
  l.flag = compensate;
  l.group = group;
  l.state_bf16 = state_bf16;
  l.own_exact = own_exact;
  g_launches.push_back(l);
  return hipSuccess;
}

hipError_t launch_decode(const uint32_t* codes, const float* scales, void* out, int64_t numel,
                         int group, bool out_bf16, bool, hipStream_t) {
  if (fails_now()) return hipErrorLaunchFailure;
  HostLaunch l{};
  l.kind = HostLaunch::kDecode;
  l.codes = codes;
  l.scales = scales;
  l.out = out;
  l.n = numel;
  l.group = group;
  l.flag = out_bf16;
  g_launches.push_back(l);
  return hipSuccess;
}

hipError_t launch_zero(float* p, int64_t n_floats, hipStream_t) {
  if (fails_now()) return hipErrorLaunchFailure;
  HostLaunch l{};
  l.kind = HostLaunch::kZero;
  l.out = p;
  l.n = n_floats;
  g_launches.push_back(l);
  return hipSuccess;
}

// the static scratch: a fake device address far from every other fake buffer
hipError_t static_scratch(int, void** ptr) {
  *ptr = reinterpret_cast<void*>(static_cast<uintptr_t>(kFakeScratch));
  return hipSuccess;
}

hipError_t launch_gemm(const GemmArgs& a, int P, bool fused, hipStream_t) {
  if (fails_now()) return hipErrorLaunchFailure;
  HostLaunch l{};
  l.kind = HostLaunch::kGemm;
  l.gemm = a;
  l.P = P;
  l.flag = fused;
  g_launches.push_back(l);
  return hipSuccess;
}

}  // namespace echo
