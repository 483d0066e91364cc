// Instantiations of the matrix-core forward with an elementwise mask and
// dropout: f16 inputs, head dim 32.
#include "fwd_mfma_launch.h"

namespace sdpa {
template hipError_t launch_mfma_masked_drop_d<false, 32>(const FwdArgs&);
}  // namespace sdpa
