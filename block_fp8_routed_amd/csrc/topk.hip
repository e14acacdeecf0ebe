// topk.hip — per token: the top_k experts by router logit and their gates.
//
// Model table of the colizig page ("What this project is trying to prove"):
// top-8 of 128 experts, top-10 of 512. The pages do not give the selection
// rule; the reading used here: the k largest logits, ties to the lower expert
// index, slots in descending-logit order, and gates equal to the softmax over
// all logits renormalised over the selected experts. The full softmax
// denominator cancels in that ratio, so g_j = exp(l_j - l_0) / sum_i
// exp(l_i - l_0) over the selected logits only (l_0 the largest).
//
// One wavefront per token: lane L holds logits L, L+64, ... in registers and
// each of the k rounds is a local scan plus a 6-step butterfly argmax whose
// comparison (larger value, then lower index) is order-independent, so the
// result is deterministic.
#include <float.h>

#include "device.hpp"
#include "layer.hpp"

namespace moe {

template <int NV>
__global__ __launch_bounds__(256) void topk_softmax(const float* __restrict__ logits,
                                                   int32_t* __restrict__ topk,
                                                   float* __restrict__ gates, int64_t T, int E,
                                                   int k) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* l = logits + t * E;
  float v[NV];
  uint32_t avail = 0;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = lane + 64 * i;
    float val = -INFINITY;
    if (e < E) {
      val = l[e];
      if (val != val) val = -INFINITY;  // NaN never outranks a number
      avail |= 1u << i;
    }
    v[i] = val;
  }
  float my_v = 0.f, top = 0.f;
  int my_i = 0;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = lane + 64 * i;
      if (((avail >> i) & 1u) && (v[i] > bv || (v[i] == bv && e < bi))) {
        bv = v[i];
        bi = e;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if (bi < E && (bi & 63) == lane) avail &= ~(1u << (bi >> 6));
    if (lane == j) {
      my_v = bv;
      my_i = bi;
    }
    if (j == 0) top = bv;
  }
  const float ex = lane < k ? expf(my_v - top) : 0.f;
  const float den = group_sum<64>(ex);
  if (lane < k) {
    topk[t * k + lane] = my_i;
    gates[t * k + lane] = ex / den;
  }
}

hipError_t launch_topk(const Dims& d, const float* logits, int32_t* topk, float* gates,
                       hipStream_t s) {
  const dim3 grid((unsigned)((d.T + 3) / 4));
  const int nv = (d.E + 63) / 64;
  if (nv <= 1)
    topk_softmax<1><<<grid, 256, 0, s>>>(logits, topk, gates, d.T, d.E, d.k);
  else if (nv <= 2)
    topk_softmax<2><<<grid, 256, 0, s>>>(logits, topk, gates, d.T, d.E, d.k);
  else if (nv <= 4)
    topk_softmax<4><<<grid, 256, 0, s>>>(logits, topk, gates, d.T, d.E, d.k);
  else if (nv <= 8)
    topk_softmax<8><<<grid, 256, 0, s>>>(logits, topk, gates, d.T, d.E, d.k);
  else
    topk_softmax<16><<<grid, 256, 0, s>>>(logits, topk, gates, d.T, d.E, d.k);
  return hipGetLastError();
}

}  // namespace moe
