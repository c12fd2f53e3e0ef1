// Owner-stage launches for 5 to 8 ranks (one of four units, so that the
// instantiations compile in parallel).
#include "echo_owner.h"

namespace echo {

hipError_t launch_owner_p5_8(const OwnerArgs& a, int P, bool compensate, int group, bool sb16,
                          bool own, hipStream_t s) {
  switch (P) {
    case 5: return owner_p<5>(a, compensate, group, sb16, own, s);
    case 6: return owner_p<6>(a, compensate, group, sb16, own, s);
    case 7: return owner_p<7>(a, compensate, group, sb16, own, s);
    case 8: return owner_p<8>(a, compensate, group, sb16, own, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace echo
