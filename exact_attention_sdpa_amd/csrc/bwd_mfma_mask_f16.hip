// Instantiations of the matrix-core backward with an elementwise or a
// block-sparse mask:
// f16 inputs, every head dim.
#include "bwd_mfma_launch.h"

namespace sdpa {
template <>
hipError_t launch_bwd_masked_tiles<false, 32>(const BwdArgs& a, const BwdParams& p) {
  return launch_bwd_masked_tiles_impl<false, 32>(a, p);
}
template <>
hipError_t launch_bwd_masked_tiles<false, 64>(const BwdArgs& a, const BwdParams& p) {
  return launch_bwd_masked_tiles_impl<false, 64>(a, p);
}
template <>
hipError_t launch_bwd_masked_tiles<false, 128>(const BwdArgs& a, const BwdParams& p) {
  return launch_bwd_masked_tiles_impl<false, 128>(a, p);
}
template <>
hipError_t launch_bwd_bsp_tiles<false, 32>(const BwdArgs& a, const BwdParams& p) {
  return launch_bwd_bsp_tiles_impl<false, 32>(a, p);
}
template <>
hipError_t launch_bwd_bsp_tiles<false, 64>(const BwdArgs& a, const BwdParams& p) {
  return launch_bwd_bsp_tiles_impl<false, 64>(a, p);
}
template <>
hipError_t launch_bwd_bsp_tiles<false, 128>(const BwdArgs& a, const BwdParams& p) {
  return launch_bwd_bsp_tiles_impl<false, 128>(a, p);
}
}  // namespace sdpa
