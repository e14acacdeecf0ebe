// router.hip — router logits l[t][e] = sum_h x[t][h] * Wr[e][h] (+ b[e]), fp32.
//
// The router is small and always resident (colizig page, "Features" and
// "Architecture & how it works": attention/router/norms stay resident, experts
// are streamed). Its cost is reading Wr at decode sizes and E*T*H FMAs at
// prefill sizes, so there are two kernels:
//  * router_gemv (T <= 16): one wavefront per expert row, coalesced 16-byte
//    loads of Wr, every token's dot product accumulated from the same load;
//  * router_gemm (T > 16): 64x64 LDS-tiled fp32 GEMM.
// Both accumulate in fp32 in two levels (short per-lane or per-128-column
// partial sums added into a running total), which keeps the rounding error of
// a 4096-term logit near 1e-6, well inside the 1e-5 band within which two
// logits count as tied.
#include "device.hpp"
#include "layer.hpp"

namespace moe {

template <int NT, bool XBF16>
__global__ __launch_bounds__(256) void router_gemv(const void* __restrict__ x,
                                                  const float* __restrict__ wr,
                                                  const float* __restrict__ bias,
                                                  float* __restrict__ logits, int T, int H,
                                                  int E) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e >= E) return;
  const float* wrow = wr + (size_t)e * H;
  float acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = 0.f;
  for (int c = 4 * lane; c < H; c += 256) {
    const float4 w = *reinterpret_cast<const float4*>(wrow + c);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (t < T) {
        float xv[4];
        if (XBF16) {
          const uint2 v = *reinterpret_cast<const uint2*>(
              reinterpret_cast<const uint16_t*>(x) + (size_t)t * H + c);
          xv[0] = bf16_lo(v.x);
          xv[1] = bf16_hi(v.x);
          xv[2] = bf16_lo(v.y);
          xv[3] = bf16_hi(v.y);
        } else {
          const float4 v = *reinterpret_cast<const float4*>(
              reinterpret_cast<const float*>(x) + (size_t)t * H + c);
          xv[0] = v.x;
          xv[1] = v.y;
          xv[2] = v.z;
          xv[3] = v.w;
        }
        acc[t] = fmaf(w.x, xv[0], acc[t]);
        acc[t] = fmaf(w.y, xv[1], acc[t]);
        acc[t] = fmaf(w.z, xv[2], acc[t]);
        acc[t] = fmaf(w.w, xv[3], acc[t]);
      }
    }
  }
  const float b = bias ? bias[e] : 0.f;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const float s = group_sum<64>(acc[t]);
    if (t < T && lane == t) logits[(size_t)t * E + e] = s + b;
  }
}

template <bool XBF16>
__global__ __launch_bounds__(256) void router_gemm(const void* __restrict__ x,
                                                  const float* __restrict__ wr,
                                                  const float* __restrict__ bias,
                                                  float* __restrict__ logits, int64_t T, int H,
                                                  int E) {
  __shared__ float As[16][68];
  __shared__ float Bs[16][68];
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int64_t m0 = (int64_t)blockIdx.x * 64;
  const int n0 = blockIdx.y * 64;
  const int lrow = tid >> 2, lk = (tid & 3) * 4;
  const int64_t xm = m0 + lrow;
  const int wn = n0 + lrow;
  float outer[4][4], inner[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) outer[i][j] = inner[i][j] = 0.f;

  for (int k0 = 0; k0 < H; k0 += 16) {
    float xa[4] = {0.f, 0.f, 0.f, 0.f}, wb[4] = {0.f, 0.f, 0.f, 0.f};
    if (xm < T) {
      if (XBF16) {
        const uint2 v = *reinterpret_cast<const uint2*>(
            reinterpret_cast<const uint16_t*>(x) + xm * H + k0 + lk);
        xa[0] = bf16_lo(v.x);
        xa[1] = bf16_hi(v.x);
        xa[2] = bf16_lo(v.y);
        xa[3] = bf16_hi(v.y);
      } else {
        const float4 v =
            *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + xm * H + k0 + lk);
        xa[0] = v.x;
        xa[1] = v.y;
        xa[2] = v.z;
        xa[3] = v.w;
      }
    }
    if (wn < E) {
      const float4 v = *reinterpret_cast<const float4*>(wr + (size_t)wn * H + k0 + lk);
      wb[0] = v.x;
      wb[1] = v.y;
      wb[2] = v.z;
      wb[3] = v.w;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      As[lk + i][lrow] = xa[i];
      Bs[lk + i][lrow] = wb[i];
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      const float4 a = *reinterpret_cast<const float4*>(&As[kk][4 * ty]);
      const float4 b = *reinterpret_cast<const float4*>(&Bs[kk][4 * tx]);
      const float av[4] = {a.x, a.y, a.z, a.w};
      const float bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) inner[i][j] = fmaf(av[i], bv[j], inner[i][j]);
    }
    if (((k0 + 16) & 127) == 0 || k0 + 16 >= H) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          outer[i][j] += inner[i][j];
          inner[i][j] = 0.f;
        }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t m = m0 + 4 * ty + i;
    if (m >= T) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + 4 * tx + j;
      if (n < E) logits[m * E + n] = outer[i][j] + (bias ? bias[n] : 0.f);
    }
  }
}

template <int NT>
static void gemv_launch(const Dims& d, const void* x, const float* wr, const float* bias,
                        float* logits, hipStream_t s) {
  const dim3 grid((d.E + 3) / 4);
  if (d.x_bf16)
    router_gemv<NT, true><<<grid, 256, 0, s>>>(x, wr, bias, logits, (int)d.T, d.H, d.E);
  else
    router_gemv<NT, false><<<grid, 256, 0, s>>>(x, wr, bias, logits, (int)d.T, d.H, d.E);
}

hipError_t launch_router(const Dims& d, const void* x, const float* wr, const float* bias,
                         float* logits, hipStream_t s) {
  if (d.T <= 16) {
    if (d.T <= 1)
      gemv_launch<1>(d, x, wr, bias, logits, s);
    else if (d.T <= 2)
      gemv_launch<2>(d, x, wr, bias, logits, s);
    else if (d.T <= 4)
      gemv_launch<4>(d, x, wr, bias, logits, s);
    else if (d.T <= 8)
      gemv_launch<8>(d, x, wr, bias, logits, s);
    else
      gemv_launch<16>(d, x, wr, bias, logits, s);
  } else {
    const dim3 grid((unsigned)((d.T + 63) / 64), (d.E + 63) / 64);
    if (d.x_bf16)
      router_gemm<true><<<grid, 256, 0, s>>>(x, wr, bias, logits, d.T, d.H, d.E);
    else
      router_gemm<false><<<grid, 256, 0, s>>>(x, wr, bias, logits, d.T, d.H, d.E);
  }
  return hipGetLastError();
}

}  // namespace moe
