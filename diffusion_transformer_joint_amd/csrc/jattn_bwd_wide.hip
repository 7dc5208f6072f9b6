// Backward pass of QK-RMSNorm joint attention on gfx950, head dims 80 to 128 (the kernels are those of
// jattn_bwd_kernels.h). These instantiations run one wave per SIMD: the dK and dV accumulators (128
// floats per lane at D = 128) then leave too few VGPRs for the loop's operands, so this file is
// compiled without -amdgpu-mfma-vgpr-form and the compiler keeps MFMA accumulators in AGPRs, which
// measured 5 % faster for both backward kernels at D = 128 than holding them in VGPRs.
#include "jattn_bwd_kernels.h"

namespace jattn {

template <bool S, bool V, bool W>
static hipError_t launch_wide_s(int D, const BwdArgs& a, bool prenorm, const hipEvent_t* events, int n_events,
                                hipStream_t stream) {
  switch (D) {
#define JATTN_CASE(DD) \
  case DD: return launch_bwd_d<DD, S, V, W>(a, prenorm, events, n_events, stream);
    JATTN_FOR_EACH_WIDE_HEAD_DIM(JATTN_CASE)
#undef JATTN_CASE
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bwd_wide(int D, Variant var, const BwdArgs& a, bool prenorm, const hipEvent_t* events, int n_events,
                           hipStream_t stream) {
  switch (var) {
    case kStreams: return launch_wide_s<true, false, false>(D, a, prenorm, events, n_events, stream);
    case kVarlen: return launch_wide_s<false, true, false>(D, a, prenorm, events, n_events, stream);
    case kWindow: return launch_wide_s<false, false, true>(D, a, prenorm, events, n_events, stream);
    default: return launch_wide_s<false, false, false>(D, a, prenorm, events, n_events, stream);
  }
}

}  // namespace jattn
