// Instantiations of the matrix-core forward with an elementwise mask and
// dropout: bf16 inputs, head dim 64.
#include "fwd_mfma_launch.h"

namespace sdpa {
template hipError_t launch_mfma_masked_drop_d<true, 64>(const FwdArgs&);
}  // namespace sdpa
