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
// lane-local maximum plus a wave maximum (DPP) of 64-bit keys that order by
// logit, then by lower expert index; the order is total, so the result does
// not depend on reduction order. Must be called by all 64 lanes.
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
  // k rounds of a wave-wide maximum over 64-bit order keys: the high word is
  // the logit's bits mapped to an unsigned order (negatives reversed, -0
  // taken as +0 so that equal logits compare equal), the low word the
  // complemented expert index, so the larger logit wins and equal logits go
  // to the lower index. Absent experts have key 0, below every logit. The
  // round's winner is cleared in the lane that holds it.
  uint64_t key[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    uint32_t b = __float_as_uint(v[i]);
    if (b == 0x80000000u) b = 0u;
    b = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    key[i] = ((avail >> i) & 1u) ? (((uint64_t)b << 32) | (uint32_t)~(lane + 64 * i)) : 0ull;
  }
  uint64_t mine = 0;  // lane j < k ends with the j-th winner
  uint64_t first = 0;
  for (int j = 0; j < k; ++j) {
    uint64_t lm = key[0];
#pragma unroll
    for (int i = 1; i < NV; ++i) lm = key[i] > lm ? key[i] : lm;
    const uint64_t m = wave_max_u64(lm);
    if (j == 0) first = m;
    mine = lane == j ? m : mine;
#pragma unroll
    for (int i = 0; i < NV; ++i) key[i] = key[i] == m ? 0ull : key[i];
  }
  // back from keys to (logit, expert)
  const auto key_logit = [](uint64_t kk) {
    const uint32_t hb = (uint32_t)(kk >> 32);
    return __uint_as_float((hb & 0x80000000u) ? (hb & 0x7fffffffu) : ~hb);
  };
  const float top = key_logit(first);
  const float my_v = key_logit(mine);
  const int my_i = (int)~(uint32_t)mine;
  const float ex = lane < k ? expf(my_v - top) : 0.f;
  const float den = group_sum<64>(ex);
  if (lane < k) {
    topk_out[t * k + lane] = my_i;
    gates_out[t * k + lane] = ex / den;
    if (topk_lds) topk_lds[t * k + lane] = my_i;
  }
}

}  // namespace moe
