// Instantiations of the matrix-core backward with an elementwise mask and
// dropout: f16 inputs, every head dim.
#include "bwd_mfma_launch.h"

namespace sdpa {
template <>
hipError_t launch_bwd_masked_drop_tiles<false, 32>(const BwdArgs& a, const BwdParams& p) {
  return launch_bwd_masked_tiles_impl<false, 32, true>(a, p);
}
template <>
hipError_t launch_bwd_masked_drop_tiles<false, 64>(const BwdArgs& a, const BwdParams& p) {
  return launch_bwd_masked_tiles_impl<false, 64, true>(a, p);
}
template <>
hipError_t launch_bwd_masked_drop_tiles<false, 128>(const BwdArgs& a, const BwdParams& p) {
  return launch_bwd_masked_tiles_impl<false, 128, true>(a, p);
}
}  // namespace sdpa
