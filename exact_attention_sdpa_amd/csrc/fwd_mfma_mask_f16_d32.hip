// Instantiations of the matrix-core forward with an elementwise mask:
// f16 inputs, head dim 32.
#include "fwd_mfma_launch.h"

namespace sdpa {
template hipError_t launch_mfma_masked_d<false, 32>(const FwdArgs&);
}  // namespace sdpa
