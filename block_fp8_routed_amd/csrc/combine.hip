// combine.hip — out[t] = sum_j g[t][j] * y[t*k+j] (+ y[T*k+t]).
//
// The gate-weighted sum of a token's expert outputs, plus the always-on shared
// expert with weight 1 (colizig page, model table: "top-10 + 1 shared").
// Summed in fp32 in a fixed order (slots j = 0..k-1, then the shared expert),
// so the result does not depend on how the expert passes were scheduled; one
// rounding to the output dtype at the end. y rows are stored by slot (the
// down passes write row r's output to y row pair[r]), so a token's outputs
// are rows t*k .. t*k + k - 1 (and T*k + t for the shared expert). The
// decode (GEMV) passes leave y in fp32; the grouped passes leave it as fp16
// with one power-of-two exponent byte per row and 128 columns (value =
// fp16 * 2^(byte - 127)).
#include "device.hpp"
#include "layer.hpp"

namespace moe {

constexpr int kYBlock = 128;  // columns per exponent byte of a scaled fp16 y row

// Thread i of a workgroup sums 8 consecutive outputs of one token (16-byte
// fp16 loads, or two 16-byte fp32 loads, of y; fp32 accumulation). y is read
// once and out written once, so both go through non-temporal accesses. The
// slots are loaded KB at a time, all of a batch's loads issued before the
// first is added, so that a token's k loads cost ceil(k / KB) load
// latencies rather than k (at decode sizes the kernel is that latency); the
// additions keep the slot order.
template <bool OUT_BF16, bool Y_F32>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ yv,
                                                     const uint8_t* __restrict__ yexp,
                                                     const float* __restrict__ gates, int64_t T,
                                                     int H, int k, int S, void* __restrict__ out) {
  const int64_t t = blockIdx.x;
  const int n = (blockIdx.y * 256 + threadIdx.x) * 8;
  if (n >= H) return;
  float a[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = 0.f;
  // the raw words of y row `row`, columns n .. n + 7 (and its exponent byte)
  struct Raw {
    uint4 p, q;
    uint32_t eb;
  };
  auto load = [&](int64_t row) {
    Raw r;
    if (Y_F32) {
      const float* yr = static_cast<const float*>(yv) + row * H + n;
      r.p = ld16_nt(yr);
      r.q = ld16_nt(yr + 4);
      r.eb = 0;
    } else {
      r.p = ld16_nt(static_cast<const uint16_t*>(yv) + row * H + n);
      r.q = make_uint4(0, 0, 0, 0);
      r.eb = yexp[row * (H / kYBlock) + n / kYBlock];
    }
    return r;
  };
  // its values times g added to a (g = 1: plain add)
  auto add = [&](const Raw& r, float g, bool gated) {
    float v[8];
    if (Y_F32) {
      const uint32_t w[8] = {r.p.x, r.p.y, r.p.z, r.p.w, r.q.x, r.q.y, r.q.z, r.q.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = __uint_as_float(w[i]);
    } else {
      const uint32_t w[4] = {r.p.x, r.p.y, r.p.z, r.p.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f16x2_t h2 = __builtin_bit_cast(f16x2_t, w[i]);
        v[2 * i] = f16_scaled_value(h2[0], r.eb);
        v[2 * i + 1] = f16_scaled_value(h2[1], r.eb);
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = gated ? fmaf(g, v[i], a[i]) : a[i] + v[i];
  };
  constexpr int KB = Y_F32 ? 4 : 8;  // slots per batch of loads
  for (int j0 = 0; j0 < k; j0 += KB) {
    Raw r[KB];
    float g[KB];
#pragma unroll
    for (int i = 0; i < KB; ++i) {
      if (j0 + i < k) {
        r[i] = load(t * k + j0 + i);
        g[i] = gates[t * k + j0 + i];
      }
    }
#pragma unroll
    for (int i = 0; i < KB; ++i)
      if (j0 + i < k) add(r[i], g[i], true);
  }
  if (S) add(load(T * k + t), 1.f, false);
  if (OUT_BF16) {
    uint4 o;
    o.x = f32_to_bf16_bits(a[0]) | (f32_to_bf16_bits(a[1]) << 16);
    o.y = f32_to_bf16_bits(a[2]) | (f32_to_bf16_bits(a[3]) << 16);
    o.z = f32_to_bf16_bits(a[4]) | (f32_to_bf16_bits(a[5]) << 16);
    o.w = f32_to_bf16_bits(a[6]) | (f32_to_bf16_bits(a[7]) << 16);
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    __builtin_nontemporal_store(u32x4{o.x, o.y, o.z, o.w},
                                reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(out) + t * H + n));
  } else {
    typedef float f32x4v __attribute__((ext_vector_type(4)));
    f32x4v* o = reinterpret_cast<f32x4v*>(reinterpret_cast<float*>(out) + t * H + n);
    __builtin_nontemporal_store(f32x4v{a[0], a[1], a[2], a[3]}, o);
    __builtin_nontemporal_store(f32x4v{a[4], a[5], a[6], a[7]}, o + 1);
  }
}

hipError_t launch_combine(const Dims& d, const Work& w, void* out, hipStream_t s) {
  const dim3 grid((unsigned)d.T, (d.H + 2047) / 2048);
#define MOE_COMBINE(OB, YF)                                                               \
  combine_kernel<OB, YF><<<grid, 256, 0, s>>>(w.y, w.yexps, w.gates, d.T, d.H, d.k, d.S, \
                                              out)
  if (d.mfma) {
    if (d.out_bf16) MOE_COMBINE(true, false);
    else MOE_COMBINE(false, false);
  } else {
    if (d.out_bf16) MOE_COMBINE(true, true);
    else MOE_COMBINE(false, true);
  }
#undef MOE_COMBINE
  return hipGetLastError();
}

}  // namespace moe
