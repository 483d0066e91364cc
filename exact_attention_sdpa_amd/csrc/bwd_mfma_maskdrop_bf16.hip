// Instantiations of the matrix-core backward with an elementwise mask and
// dropout: bf16 inputs, every head dim.
#include "bwd_mfma_launch.h"

namespace sdpa {
template <>
hipError_t launch_bwd_masked_drop_tiles<true, 32>(const BwdArgs& a, const BwdParams& p) {
  return launch_bwd_masked_tiles_impl<true, 32, true>(a, p);
}
template <>
hipError_t launch_bwd_masked_drop_tiles<true, 64>(const BwdArgs& a, const BwdParams& p) {
  return launch_bwd_masked_tiles_impl<true, 64, true>(a, p);
}
template <>
hipError_t launch_bwd_masked_drop_tiles<true, 128>(const BwdArgs& a, const BwdParams& p) {
  return launch_bwd_masked_tiles_impl<true, 128, true>(a, p);
}
}  // namespace sdpa
