// Head-dim dispatch of the matrix-core forward.
#include "fwd_mfma_launch.h"

namespace sdpa {

extern template hipError_t launch_mfma_d<false, 32>(const FwdArgs&);
extern template hipError_t launch_mfma_d<false, 64>(const FwdArgs&);
extern template hipError_t launch_mfma_d<false, 128>(const FwdArgs&);
extern template hipError_t launch_mfma_d<true, 32>(const FwdArgs&);
extern template hipError_t launch_mfma_d<true, 64>(const FwdArgs&);
extern template hipError_t launch_mfma_d<true, 128>(const FwdArgs&);
extern template hipError_t launch_mfma_masked_d<false, 32>(const FwdArgs&);
extern template hipError_t launch_mfma_masked_d<false, 64>(const FwdArgs&);
extern template hipError_t launch_mfma_masked_d<false, 128>(const FwdArgs&);
extern template hipError_t launch_mfma_masked_d<true, 32>(const FwdArgs&);
extern template hipError_t launch_mfma_masked_d<true, 64>(const FwdArgs&);
extern template hipError_t launch_mfma_masked_d<true, 128>(const FwdArgs&);
extern template hipError_t launch_mfma_masked_drop_d<false, 32>(const FwdArgs&);
extern template hipError_t launch_mfma_masked_drop_d<false, 64>(const FwdArgs&);
extern template hipError_t launch_mfma_masked_drop_d<false, 128>(const FwdArgs&);
extern template hipError_t launch_mfma_masked_drop_d<true, 32>(const FwdArgs&);
extern template hipError_t launch_mfma_masked_drop_d<true, 64>(const FwdArgs&);
extern template hipError_t launch_mfma_masked_drop_d<true, 128>(const FwdArgs&);

hipError_t launch_fwd_mfma_f16(const FwdArgs& a) {
  switch (a.d) {
    case 32: return launch_mfma_d<false, 32>(a);
    case 64: return launch_mfma_d<false, 64>(a);
    case 128: return launch_mfma_d<false, 128>(a);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_fwd_mfma_bf16(const FwdArgs& a) {
  switch (a.d) {
    case 32: return launch_mfma_d<true, 32>(a);
    case 64: return launch_mfma_d<true, 64>(a);
    case 128: return launch_mfma_d<true, 128>(a);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_fwd_mfma_masked_f16(const FwdArgs& a) {
  switch (a.d) {
    case 32: return a.dropout ? launch_mfma_masked_drop_d<false, 32>(a) : launch_mfma_masked_d<false, 32>(a);
    case 64: return a.dropout ? launch_mfma_masked_drop_d<false, 64>(a) : launch_mfma_masked_d<false, 64>(a);
    case 128:
      return a.dropout ? launch_mfma_masked_drop_d<false, 128>(a) : launch_mfma_masked_d<false, 128>(a);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_fwd_mfma_masked_bf16(const FwdArgs& a) {
  switch (a.d) {
    case 32: return a.dropout ? launch_mfma_masked_drop_d<true, 32>(a) : launch_mfma_masked_d<true, 32>(a);
    case 64: return a.dropout ? launch_mfma_masked_drop_d<true, 64>(a) : launch_mfma_masked_d<true, 64>(a);
    case 128:
      return a.dropout ? launch_mfma_masked_drop_d<true, 128>(a) : launch_mfma_masked_d<true, 128>(a);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sdpa
