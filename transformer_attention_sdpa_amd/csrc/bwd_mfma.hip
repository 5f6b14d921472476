// bwd_mfma.hip -- matrix-core form of the dK/dV and dQ passes of the attention gradient.
#include "device_common.h"

namespace sdpa {

bool bwd_mfma_supports(const BwdArgs& g) {
  (void)g;
  return false;
}

hipError_t launch_bwd_mfma_dkdv(const BwdArgs& g, hipStream_t s) {
  (void)g; (void)s;
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_mfma_dq(const BwdArgs& g, hipStream_t s) {
  (void)g; (void)s;
  return hipErrorInvalidValue;
}

}  // namespace sdpa
