// fwd_mfma.hip -- bf16 attention forward on the gfx950 matrix cores (in progress).
#include "device_common.h"

namespace sdpa {

bool fwd_mfma_supports(const AttnArgs& a) {
  (void)a;
  return false;
}

hipError_t launch_fwd_mfma(const AttnArgs& a, hipStream_t s) {
  (void)a;
  (void)s;
  return hipErrorNotSupported;
}

}  // namespace sdpa
