// expert_mfma.hip — grouped bf16-MFMA expert passes (prefill-sized groups).
#include "device.hpp"
#include "layer.hpp"

namespace moe {

bool has_mfma_instance(const Dims&) { return false; }

hipError_t launch_experts_mfma(const Dims&, const void*, const moe_expert_bank&,
                               const moe_expert_bank*, const Work&, hipStream_t, hipEvent_t) {
  return hipErrorInvalidValue;
}

}  // namespace moe
