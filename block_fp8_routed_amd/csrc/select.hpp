// select.hpp — top-k selection and gates of one token by one wavefront.
//
// Model table of the colizig page ("What this project is trying to prove"):
// top-8 of 128 experts, top-10 of 512. The pages do not give the selection
// rule; the reading used here: the k largest logits, ties to the lower expert
// index, slots in descending-logit order, and gates equal to the softmax over
// all logits renormalised over the selected experts. The full softmax
// denominator cancels in that ratio, so g_j = exp(l_j - l_0) / sum_i
// exp(l_i - l_0) over the selected logits only (l_0 the largest).
//
// Lane L owns experts L, L+64, ...; it sums the router's partial logits over
// the H slices in slice order and adds the bias. Each of the k rounds is a
// local scan plus a wave argmax (DPP inside 16-lane rows, readlane across
// rows) whose comparison (larger value, then lower index) is order-
// independent, so the result is deterministic. Must be called by all 64 lanes.
#pragma once

#include "device.hpp"

namespace moe {

template <int NV>
__device__ __forceinline__ void select_token(const float* __restrict__ plog, int slices,
                                             const float* __restrict__ bias, int64_t T,
                                             int64_t t, int E, int k, int32_t* topk_out,
                                             float* gates_out, float* logits_out,
                                             int32_t* topk_lds) {
  const int lane = threadIdx.x & 63;
  // Every partial logit (up to kMaxUnrolled slices) and bias term of the
  // lane's experts is requested before any is used: the addresses are
  // clamped into range instead of branched around, so the loads go out
  // together and the token pays one memory latency, not one per expert.
  constexpr int kMaxUnrolled = 8;
  float part[NV][kMaxUnrolled];
  float bv[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = lane + 64 * i < E ? lane + 64 * i : E - 1;
#pragma unroll
    for (int s = 0; s < kMaxUnrolled; ++s) {
      const int sc = s < slices ? s : slices - 1;
      part[i][s] = plog[((size_t)sc * T + t) * E + e];
    }
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = lane + 64 * i < E ? lane + 64 * i : E - 1;
    bv[i] = bias ? bias[e] : 0.f;
  }
  float v[NV];
  uint32_t avail = 0;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = lane + 64 * i;
    float val = part[i][0];  // slices summed in slice order
#pragma unroll
    for (int s = 1; s < kMaxUnrolled; ++s)
      if (s < slices) val += part[i][s];
    if (e < E) {
      for (int s = kMaxUnrolled; s < slices; ++s) val += plog[((size_t)s * T + t) * E + e];
      if (bias) val += bv[i];
      if (logits_out) logits_out[t * E + e] = val;
      if (val != val) val = -INFINITY;  // NaN never outranks a number
      avail |= 1u << i;
    } else {
      val = -INFINITY;
    }
    v[i] = val;
  }
  float my_v = 0.f, top = 0.f;
  int my_i = 0;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < NV; ++i)
      if ((avail >> i) & 1u) take_max(bv, bi, v[i], lane + 64 * i);
    wave_argmax(bv, bi);
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
    topk_out[t * k + lane] = my_i;
    gates_out[t * k + lane] = ex / den;
    if (topk_lds) topk_lds[t * k + lane] = my_i;
  }
}

}  // namespace moe
