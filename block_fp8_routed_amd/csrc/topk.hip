// topk.hip — per token: finish the router logits, then pick the top_k experts
// and their gates (select_token, one wavefront per token).
#include "layer.hpp"
#include "select.hpp"

namespace moe {

// U: partial logits requested together per expert (the slice count when it
// is 1 or 4, so that no request repeats a clamped slice)
template <int NV, int U>
__global__ __launch_bounds__(256) void topk_softmax(const float* __restrict__ plog, int slices,
                                                   const float* __restrict__ bias,
                                                   int32_t* __restrict__ topk,
                                                   float* __restrict__ gates,
                                                   float* __restrict__ logits_out, int64_t T,
                                                   int E, int k, int32_t* __restrict__ zero_word) {
  if (zero_word && blockIdx.x == 0 && threadIdx.x == 0) *zero_word = 0;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  select_token<NV, U>(plog, slices, bias, T, t, E, k, topk, gates, logits_out);
}

hipError_t launch_topk(const Dims& d, const float* plog, const float* bias, int32_t* topk,
                       float* gates, float* logits_out, int32_t* zero_word, hipStream_t s) {
  const dim3 grid((unsigned)((d.T + 3) / 4));
  const int ns = router_slices(d);
  const int nv = (d.E + 63) / 64;
#define MOE_TOPKU(NV, U)                                                                    \
  topk_softmax<NV, U><<<grid, 256, 0, s>>>(plog, ns, bias, topk, gates, logits_out, d.T, d.E, \
                                           d.k, zero_word)
#define MOE_TOPK(NV)     \
  if (ns == 1)           \
    MOE_TOPKU(NV, 1);    \
  else if (ns == 4)      \
    MOE_TOPKU(NV, 4);    \
  else                   \
    MOE_TOPKU(NV, NV <= 2 ? 16 : 8)
  if (nv <= 1)
    MOE_TOPK(1);
  else if (nv <= 2)
    MOE_TOPK(2);
  else if (nv <= 4)
    MOE_TOPK(4);
  else if (nv <= 8)
    MOE_TOPK(8);
  else
    MOE_TOPK(16);
#undef MOE_TOPK
#undef MOE_TOPKU
  return hipGetLastError();
}

}  // namespace moe
