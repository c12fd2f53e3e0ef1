// Owner-stage launches for 15 and 16 ranks (one of eight units, so that the
// instantiations compile in parallel).
#include "echo_owner.h"

namespace echo {

hipError_t launch_owner_p15_16(const OwnerArgs& a, int P, bool compensate, int group, bool sb16,
                          bool own, hipStream_t s) {
  switch (P) {
    case 15: return owner_p<15>(a, compensate, group, sb16, own, s);
    case 16: return owner_p<16>(a, compensate, group, sb16, own, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace echo
