// moe_static.hip — moe_forward for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid allocation): its scratch is a file-scope device array of a fixed
// size instead of a caller-provided workspace.
//
// Each GPU the library runs on holds its own copy of the array from the
// code object's load until the process ends. In host code the array's name
// is only a stand-in, so its device address is looked up once per device
// (hipGetSymbolAddress, with that device current, on the first call there)
// and kept; kernels are given that address, never the name. Every call on
// one device shares the array: calls that overlap on one GPU (other streams,
// other host threads) race on it. The layer reads no scratch byte it has not
// written in the same call (the single-launch decode layer's flags excepted:
// they only pass a wait when they hold that call's epoch), so nothing needs
// clearing between calls.
#include <mutex>

#include "layer.hpp"

namespace moe {

constexpr size_t kStaticScratchBytes = (size_t)MOE_STATIC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device

// The current device's copy of `scratch` (looked up on first use), or null.
static void* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace moe

extern "C" moe_status moe_forward_static(const void* x, const float* router_w,
                                         const float* router_bias,
                                         const moe_expert_bank* experts,
                                         const moe_expert_bank* shared, int32_t top_k, void* out,
                                         const moe_config* cfg, const moe_phase_events* events,
                                         void* stream) {
  if (!cfg) return MOE_ERR_NULL;
  const size_t need = moe_workspace_bytes(cfg);
  if (need > moe::kStaticScratchBytes) return MOE_ERR_TOO_LARGE;
  if (need == 0 || cfg->tokens == 0)  // invalid (0 bytes) or empty: moe_forward decides
    return moe_forward(x, router_w, router_bias, experts, shared, top_k, out, cfg, nullptr, 0,
                       events, stream);
  void* ws = moe::device_scratch();
  if (!ws) return MOE_ERR_HIP;
  return moe_forward(x, router_w, router_bias, experts, shared, top_k, out, cfg, ws,
                     moe::kStaticScratchBytes, events, stream);
}
