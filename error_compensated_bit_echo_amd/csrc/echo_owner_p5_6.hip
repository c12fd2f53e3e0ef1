// Owner-stage launches for 5 and 6 ranks (one of eight units, so that the
// instantiations compile in parallel).
#include "echo_owner.h"

namespace echo {

hipError_t launch_owner_p5_6(const OwnerArgs& a, int P, bool compensate, int group, bool sb16,
                          bool own, hipStream_t s) {
  switch (P) {
    case 5: return owner_p<5>(a, compensate, group, sb16, own, s);
    case 6: return owner_p<6>(a, compensate, group, sb16, own, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace echo
