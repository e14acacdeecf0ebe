// router_decode.hpp — the decode-size router work item (one expert quad, one
// slice of H), shared by router.hip's slice kernel and the single-launch
// decode layer.
#pragma once

#include "device.hpp"
#include "layer.hpp"

namespace moe {

// Decode sizes: workgroup (expert quad q, slice s) has one wavefront per
// group of 4 tokens; each wavefront dots 4 expert rows with its 4 tokens over
// the slice's columns (lane L takes columns 4L + 256j) and reduces the 16
// partial sums across the wave. Token rows are read straight from global
// memory; the expert rows are shared by the workgroup's wavefronts through the
// cache.
// (bx, by) = (expert quad, slice); tb: the workgroup's first token (its
// wavefronts take tokens tb + NT w ..). Wavefronts whose tokens all lie
// past T compute on clamped rows and write nothing.
// COHERENT: the partial logits are stored at the point of coherence (for a
// consumer in the same kernel).
template <int NT, bool XBF16, bool COHERENT = false>
__device__ __forceinline__ void router_slices_item(const void* __restrict__ x,
                                                   const float* __restrict__ wr,
                                                   float* __restrict__ plog, int T, int H, int E,
                                                   int HS, int bx, int by, int tb = 0) {
  const int lane = threadIdx.x & 63;
  const int t0 = tb + (threadIdx.x >> 6) * NT;
  const int h0 = by * HS;
  const int e0 = bx * 4;
  constexpr int J = kRouterSlice / 256;
  // Loads are unconditional, with row and column indices clamped into range
  // (out-of-range terms are zeroed afterwards), so that all of them are in
  // flight together.
  float4 w[4][J];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int c = 4 * lane + 256 * j;
      const int e = e0 + r < E ? e0 + r : E - 1;
      w[r][j] = *reinterpret_cast<const float4*>(wr + (size_t)e * H + h0 + (c < HS ? c : HS - 4));
    }
  float4 xv[NT][J];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int c = 4 * lane + 256 * j;
      const size_t off = (size_t)(t0 + t < T ? t0 + t : T - 1) * H + h0 + (c < HS ? c : HS - 4);
      if (XBF16) {
        const uint2 u = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(x) + off);
        xv[t][j] = make_float4(bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y));
      } else {
        xv[t][j] = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + off);
      }
    }
#pragma unroll
  for (int j = 0; j < J; ++j) {
    if (4 * lane + 256 * j < HS) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r) w[r][j] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int t = 0; t < NT; ++t) xv[t][j] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      float a = 0.f;
#pragma unroll
      for (int j = 0; j < J; ++j) {
        a = fmaf(w[r][j].x, xv[t][j].x, a);
        a = fmaf(w[r][j].y, xv[t][j].y, a);
        a = fmaf(w[r][j].z, xv[t][j].z, a);
        a = fmaf(w[r][j].w, xv[t][j].w, a);
      }
      const float v = group_sum<64>(a);
      const int q = r * NT + t;
      if (t0 + t < T && e0 + r < E && lane == (q & 63))
      {
        float* dst = plog + ((size_t)by * T + t0 + t) * E + e0 + r;
        if (COHERENT)
          st_coherent(dst, v);
        else
          *dst = v;
      }
    }
}

}  // namespace moe
