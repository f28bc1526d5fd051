// Train-step backward (gpu_moe_h100.json header: value and gradient with
// respect to the parameters and the input).
#include "gemm_core.h"

namespace moe {

size_t bwd_ws_bytes(const moe_problem&) { return 0; }

hipError_t launch_bwd(const moe_problem&, const void*, const moe_weights&, const moe_routing&,
                      const void*, const void*, const void*, void*, const moe_grads&, void*,
                      hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace moe
