// Matrix-core backward, bf16 inputs: head-dim dispatch.
#include "bwd_mfma_launch.h"

namespace sdpa {

hipError_t launch_bwd_mfma_bf16(const BwdArgs& a) {
  switch (a.d) {
    case 32: return launch_bwd_d<true, 32>(a);
    case 64: return launch_bwd_d<true, 64>(a);
    case 128: return launch_bwd_d<true, 128>(a);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bwd_mfma_masked_bf16(const BwdArgs& a) {
  switch (a.d) {
    case 32: return launch_bwd_d<true, 32>(a, true);
    case 64: return launch_bwd_d<true, 64>(a, true);
    case 128: return launch_bwd_d<true, 128>(a, true);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sdpa
