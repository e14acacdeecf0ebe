// combine.hip — out[t] = sum_j g[t][j] * y[inv[t*k+j]] (+ y[inv[T*k+t]]).
//
// The gate-weighted sum of a token's expert outputs, plus the always-on shared
// expert with weight 1 (colizig page, model table: "top-10 + 1 shared").
// Summed in fp32 in a fixed order (slots j = 0..k-1, then the shared expert),
// so the result does not depend on how the expert passes were scheduled; one
// rounding to the output dtype at the end.
#include "device.hpp"
#include "layer.hpp"

namespace moe {

template <bool OUT_BF16>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y,
                                                     const float* __restrict__ gates,
                                                     const int32_t* __restrict__ inv, int64_t T,
                                                     int H, int k, int S, void* __restrict__ out) {
  const int64_t t = blockIdx.x;
  const int n = (blockIdx.y * 256 + threadIdx.x) * 4;
  if (n >= H) return;
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
  for (int j = 0; j < k; ++j) {
    const float g = gates[t * k + j];
    const float4 v = *reinterpret_cast<const float4*>(y + (size_t)inv[t * k + j] * H + n);
    a0 = fmaf(g, v.x, a0);
    a1 = fmaf(g, v.y, a1);
    a2 = fmaf(g, v.z, a2);
    a3 = fmaf(g, v.w, a3);
  }
  if (S) {
    const float4 v = *reinterpret_cast<const float4*>(y + (size_t)inv[T * k + t] * H + n);
    a0 += v.x;
    a1 += v.y;
    a2 += v.z;
    a3 += v.w;
  }
  if (OUT_BF16) {
    uint2 o;
    o.x = f32_to_bf16_bits(a0) | (f32_to_bf16_bits(a1) << 16);
    o.y = f32_to_bf16_bits(a2) | (f32_to_bf16_bits(a3) << 16);
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + t * H + n) = o;
  } else {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + t * H + n) =
        make_float4(a0, a1, a2, a3);
  }
}

hipError_t launch_combine(const Dims& d, const Work& w, void* out, hipStream_t s) {
  const dim3 grid((unsigned)d.T, (d.H + 1023) / 1024);
  if (d.out_bf16)
    combine_kernel<true><<<grid, 256, 0, s>>>(w.y, w.gates, w.inv, d.T, d.H, d.k, d.S, out);
  else
    combine_kernel<false><<<grid, 256, 0, s>>>(w.y, w.gates, w.inv, d.T, d.H, d.k, d.S, out);
  return hipGetLastError();
}

}  // namespace moe
