// Owner-stage launches for 9 and 10 ranks (one of eight units, so that the
// instantiations compile in parallel).
#include "echo_owner.h"

namespace echo {

hipError_t launch_owner_p9_10(const OwnerArgs& a, int P, bool compensate, int group, bool sb16,
                          bool own, hipStream_t s) {
  switch (P) {
    case 9: return owner_p<9>(a, compensate, group, sb16, own, s);
    case 10: return owner_p<10>(a, compensate, group, sb16, own, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace echo
