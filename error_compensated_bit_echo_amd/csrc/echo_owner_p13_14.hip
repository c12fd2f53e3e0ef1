// Owner-stage launches for 13 and 14 ranks (one of eight units, so that the
// instantiations compile in parallel).
#include "echo_owner.h"

namespace echo {

hipError_t launch_owner_p13_14(const OwnerArgs& a, int P, bool compensate, int group, bool sb16,
                          bool own, hipStream_t s) {
  switch (P) {
    case 13: return owner_p<13>(a, compensate, group, sb16, own, s);
    case 14: return owner_p<14>(a, compensate, group, sb16, own, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace echo
