// The library's static device scratch: the stage-1 payloads of the P ranks and
// the broadcast payload of echo_reduce_noalloc, the one entry point that
// allocates nothing (for callers that cannot call hipMalloc).
//
// The array is a file-scope device variable: every device the library runs on
// holds its own copy, at its own address, from the moment the code object is
// loaded there until the process ends.  In host code its name is only a
// host-side stand-in, so the device address is looked up once per device with
// hipGetSymbolAddress (that device current) and kept; kernels and copies get
// that address, never the name.
#include <atomic>
#include <mutex>

#include "echo.h"
#include "echo_internal.h"

namespace {

__device__ __align__(256) unsigned char scratch[ECHO_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 256;
std::atomic<void*> g_scratch_at[kMaxDevices];  // the array's address on each device, once looked up
std::mutex g_lookup;                           // serialises the first lookup on a device

}  // namespace

namespace echo {

hipError_t static_scratch(int device, void** ptr) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_at[device].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_lookup);
    p = g_scratch_at[device].load(std::memory_order_relaxed);
    if (p == nullptr) {
      const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (p == nullptr) return hipErrorInvalidSymbol;
      g_scratch_at[device].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

}  // namespace echo
