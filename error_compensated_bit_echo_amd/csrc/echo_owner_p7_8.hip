// Owner-stage launches for 7 and 8 ranks (one of eight units, so that the
// instantiations compile in parallel).
#include "echo_owner.h"

namespace echo {

hipError_t launch_owner_p7_8(const OwnerArgs& a, int P, bool compensate, int group, bool sb16,
                          bool own, hipStream_t s) {
  switch (P) {
    case 7: return owner_p<7>(a, compensate, group, sb16, own, s);
    case 8: return owner_p<8>(a, compensate, group, sb16, own, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace echo
