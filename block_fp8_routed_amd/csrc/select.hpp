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
// the H slices in slice order and adds the bias. Each of the k rounds takes
// the wave-wide maximum (DPP) of 32-bit keys that order the logits exactly,
// then the lowest expert index holding it (one ballot per expert row of the
// lanes, lowest row first); the order is total, so the result does not
// depend on reduction order. Must be called by all 64 lanes; returns, in lane
// j < k, the j-th selected expert (other lanes: -1).
#pragma once

#include "device.hpp"

namespace moe {

// UNROLL: partial logits per expert requested together (more slices are added
// one at a time, in the same slice order).
// COHERENT: the partial logits are read at the point of coherence (written
// by other workgroups of the same kernel).
template <int NV, int UNROLL = (NV <= 2 ? 16 : 8), bool COHERENT = false>
__device__ __forceinline__ int select_token(const float* __restrict__ plog, int slices,
                                            const float* __restrict__ bias, int64_t T, int64_t t,
                                            int E, int k, int32_t* topk_out, float* gates_out,
                                            float* logits_out) {
  const int lane = threadIdx.x & 63;
  // Every partial logit (up to kMaxUnrolled slices: 16 for up to two
  // experts per lane, else 8) and bias term of the lane's experts is
  // requested before any is used: the addresses are clamped into range
  // instead of branched around, so the loads go out together and the token
  // pays one memory latency, not one per expert.
  constexpr int kMaxUnrolled = UNROLL;
  float part[NV][kMaxUnrolled];
  float bv[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = lane + 64 * i < E ? lane + 64 * i : E - 1;
#pragma unroll
    for (int s = 0; s < kMaxUnrolled; ++s) {
      const int sc = s < slices ? s : slices - 1;
      const float* src = plog + ((size_t)sc * T + t) * E + e;
      part[i][s] = COHERENT ? ld_coherent(src) : *src;
    }
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = lane + 64 * i < E ? lane + 64 * i : E - 1;
    bv[i] = bias ? bias[e] : 0.f;
  }
  // order keys: the logit's bits mapped to an unsigned order (negatives
  // reversed, -0 taken as +0 so that equal logits compare equal, NaN taken as
  // -inf so that it never outranks a number). Every logit maps above zero
  // (-inf to 0x007fffff), so 0 marks an absent or already chosen expert.
  uint32_t key[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int e = lane + 64 * i;
    float val = part[i][0];  // slices summed in slice order
#pragma unroll
    for (int s = 1; s < kMaxUnrolled; ++s)
      if (s < slices) val += part[i][s];
    key[i] = 0u;
    if (e < E) {
      for (int s = kMaxUnrolled; s < slices; ++s) {
        const float* src = plog + ((size_t)s * T + t) * E + e;
        val += COHERENT ? ld_coherent(src) : *src;
      }
      if (bias) val += bv[i];
      if (logits_out) logits_out[t * E + e] = val;
      if (val != val) val = -INFINITY;
      uint32_t b = __float_as_uint(val);
      if (b == 0x80000000u) b = 0u;
      key[i] = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    }
  }
  uint32_t mine = 0;  // lane j < k ends with the j-th winner's key and expert
  int mine_e = -1;
  uint32_t first = 0;
  for (int j = 0; j < k; ++j) {
    uint32_t lm = key[0];
#pragma unroll
    for (int i = 1; i < NV; ++i) lm = max(lm, key[i]);
    const uint32_t m = wave_max_u32(lm);
    if (j == 0) first = m;
    // the lowest expert index holding the maximum (the lane's experts are
    // 64 i + lane). Up to two experts per lane: the first row i with a
    // holder (a ballot per row), then its lowest lane. More: each lane
    // offers its lowest holder and a second reduction takes the minimum, as
    // the maximum of the complements (a lane with none offers ~0, which
    // complements to the maximum's neutral 0); a walk over eight or more
    // rows costs more in scalar branches than the reduction. Only valid
    // experts hold m, since every logit's key is above zero.
    int win = -1;
    if constexpr (NV <= 2) {
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const unsigned long long b = __ballot(key[i] == m);
        if (win < 0 && b != 0ull) {
          const int wl = __ffsll((long long)b) - 1;
          win = 64 * i + wl;
          if (lane == wl) key[i] = 0u;
        }
      }
    } else {
      uint32_t loc = 0xffffffffu;
#pragma unroll
      for (int i = NV - 1; i >= 0; --i) loc = key[i] == m ? (uint32_t)(64 * i + lane) : loc;
      win = (int)~wave_max_u32(~loc);
      const bool owner = lane == (win & 63);
#pragma unroll
      for (int i = 0; i < NV; ++i) key[i] = owner && i == (win >> 6) ? 0u : key[i];
    }
    if (lane == j) {
      mine = m;
      mine_e = win;
    }
  }
  // back from keys to logits
  const auto key_logit = [](uint32_t hb) {
    return __uint_as_float((hb & 0x80000000u) ? (hb & 0x7fffffffu) : ~hb);
  };
  const float top = key_logit(first);
  const float my_v = key_logit(mine);
  const float ex = lane < k ? expf(my_v - top) : 0.f;
  const float den = group_sum<64>(ex);
  if (lane < k) {
    topk_out[t * k + lane] = mine_e;
    gates_out[t * k + lane] = ex / den;
  }
  return lane < k ? mine_e : -1;
}

}  // namespace moe
