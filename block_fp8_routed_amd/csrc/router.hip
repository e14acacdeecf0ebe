// router.hip — router logits l[t][e] = sum_h x[t][h] * Wr[e][h], fp32.
//
// The router is small and always resident (colizig page, "Features" and
// "Architecture & how it works": attention/router/norms stay resident, experts
// are streamed). Its cost is reading Wr at decode sizes and E*T*H MACs at
// prefill sizes, so there are three kernels:
//  * router_slices (T <= 16): H is cut into slices of 512 columns; a
//    wavefront dots four expert rows of a slice with four tokens using
//    coalesced 16-byte loads.
//  * router_mfma (T > 16, bf16 activations): bf16 MFMA tiles over an exact
//    three-plane bf16 split of Wr, per slice of 512 columns.
//  * router_gemm (otherwise): 64x64 LDS-tiled fp32 GEMM, one slice.
// Partial sums per slice are written out and the top-k kernel adds them in
// slice order. Every path accumulates in fp32 in two levels (short partial
// sums added into a running total), which keeps the rounding error of a
// 4096-term logit near 1e-6, well inside the 1e-5 band within which two
// logits count as tied. The bias is added by the top-k kernel.
#include "device.hpp"
#include "layer.hpp"
#include "router_decode.hpp"

namespace moe {

template <int NT, bool XBF16>
__global__ __launch_bounds__(256) void router_slices_kernel(const void* __restrict__ x,
                                                           const float* __restrict__ wr,
                                                           float* __restrict__ plog, int T,
                                                           int H, int E, int HS) {
  router_slices_item<NT, XBF16>(x, wr, plog, T, H, E, HS, blockIdx.x, blockIdx.y,
                                (int)blockIdx.z * 4 * NT);
}

template <bool XBF16>
__global__ __launch_bounds__(256) void router_gemm(const void* __restrict__ x,
                                                  const float* __restrict__ wr,
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
      if (n < E) logits[m * E + n] = outer[i][j];
    }
  }
}

template <int NT>
static void slices_launch(const Dims& d, const void* x, const float* wr, float* plog,
                          hipStream_t s) {
  const int ns = router_slices(d);
  const int HS = d.H < kRouterSlice ? d.H : kRouterSlice;
  // up to four wavefronts (4 NT tokens) per workgroup; more tokens take
  // more workgroups along z
  const int64_t per = 4 * NT;
  const dim3 grid((d.E + 3) / 4, ns, (unsigned)((d.T + per - 1) / per));
  const int threads = 64 * (int)((std::min<int64_t>(d.T, per) + NT - 1) / NT);
  if (d.x_bf16)
    router_slices_kernel<NT, true><<<grid, threads, 0, s>>>(x, wr, plog, (int)d.T, d.H, d.E, HS);
  else
    router_slices_kernel<NT, false><<<grid, threads, 0, s>>>(x, wr, plog, (int)d.T, d.H, d.E, HS);
}

// ------------------------------------------------------------ MFMA router --
// Prefill sizes with bf16 activations. Each fp32 router weight is split into
// three bf16 planes, w = hi + mid + lo (hi = bf16(w), mid = bf16(w - hi),
// lo = bf16(w - hi - mid), each difference exact in fp32), which leaves a
// remainder below 2^-24 |w|. A logit is then the sum of three bf16 MFMA
// contractions of the (exact) bf16 activations, each product exact in fp32.
// The split is done in registers as the fp32 weights are staged into LDS.
__device__ __forceinline__ void split3(float w, uint32_t& hb, uint32_t& mb, uint32_t& lb) {
  hb = f32_to_bf16_bits(w);
  const float r1 = w - __uint_as_float(hb << 16);
  mb = f32_to_bf16_bits(r1);
  const float r2 = r1 - __uint_as_float(mb << 16);
  lb = f32_to_bf16_bits(r2);
}

// Tile of 128 tokens x 128 experts over one slice of H (blockIdx.z), 256
// threads as 2 x 2 wavefronts of 64 x 64 (2 x 2 MFMA tiles of 32 x 32). K runs
// in stages of 32: the stage's activation tile (bf16) and weight tile (fp32)
// are fetched global -> registers two stages ahead (a ring of two register
// sets) and stored into the other of two LDS buffers after the stage's MFMAs,
// the weights as their three bf16 planes.
// 16-byte chunks are XOR-swizzled by row (chunk c of row r at slot c ^ ((r >>
// 2) & 3)) against bank conflicts. Rows past T and experts past E repeat the
// last one, and a stage index past the slice's end repeats its last stage
// (loads stay unconditional); none of those is stored.
typedef __bf16 rbf16x8_t __attribute__((ext_vector_type(8)));
typedef float rf32x16_t __attribute__((ext_vector_type(16)));
constexpr int kRtBM = kRouterTile, kRtBN = kRouterTile, kRtKS = 32;
constexpr int kRtRow = kRtKS * 2;                // bytes per tile row per stage
constexpr int kRtA = kRtBM * kRtRow;             // 8 KiB
constexpr int kRtStage = kRtA + 3 * kRtBN * kRtRow;  // 32 KiB

__global__ __launch_bounds__(256) void router_mfma(const uint16_t* __restrict__ x,
                                                  const float* __restrict__ wr,
                                                  float* __restrict__ plog, int T, int H, int E,
                                                  int HS) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kRtStage];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.x * kRtBM, e0 = blockIdx.y * kRtBN, h0 = blockIdx.z * HS;
  // fetch map: A chunk q = tid + 256 i (i < 2): row q / 4, chunk q % 4 (8 bf16);
  // B chunk q = tid + 256 i (i < 4): weight row q / 8, chunk q % 8 (4 fp32),
  // stored as 4 bf16 (8 bytes) at the same place of each of the three planes
  const uint16_t* asrc[2];
  int adst[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = tid + 256 * i, r = q >> 2, c = q & 3;
    const int row = m0 + r < T ? m0 + r : T - 1;
    asrc[i] = x + (size_t)row * H + h0 + 8 * c;
    adst[i] = r * kRtRow + 16 * (c ^ ((r >> 2) & 3));
  }
  const float* bsrc[4];
  int bdst[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = tid + 256 * i, r = q >> 3, c8 = q & 7;
    const int e = e0 + r < E ? e0 + r : E - 1;
    bsrc[i] = wr + (size_t)e * H + h0 + 4 * c8;
    bdst[i] = kRtA + r * kRtRow + 16 * ((c8 >> 1) ^ ((r >> 2) & 3)) + 8 * (c8 & 1);
  }
  const int NS = HS / kRtKS;
  struct StageRegs {
    uint4 a[2], b[4];
  };
  auto fetch = [&](StageRegs& v, int st) {
    st = st < NS ? st : NS - 1;  // past the end: a harmless repeat, never stored
#pragma unroll
    for (int i = 0; i < 2; ++i) v.a[i] = ld16(asrc[i] + st * kRtKS);
#pragma unroll
    for (int i = 0; i < 4; ++i) v.b[i] = ld16(bsrc[i] + st * kRtKS);
  };
  auto put = [&](const StageRegs& v, int buf) {
    uint8_t* L = lds + buf * kRtStage;
#pragma unroll
    for (int i = 0; i < 2; ++i) *reinterpret_cast<uint4*>(L + adst[i]) = v.a[i];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t f[4] = {v.b[i].x, v.b[i].y, v.b[i].z, v.b[i].w};
      uint32_t hb[4], mb[4], lb[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) split3(__uint_as_float(f[j]), hb[j], mb[j], lb[j]);
      *reinterpret_cast<uint2*>(L + bdst[i]) = make_uint2(hb[0] | hb[1] << 16, hb[2] | hb[3] << 16);
      *reinterpret_cast<uint2*>(L + bdst[i] + kRtBN * kRtRow) =
          make_uint2(mb[0] | mb[1] << 16, mb[2] | mb[3] << 16);
      *reinterpret_cast<uint2*>(L + bdst[i] + 2 * kRtBN * kRtRow) =
          make_uint2(lb[0] | lb[1] << 16, lb[2] | lb[3] << 16);
    }
  };
  const int q = lane >> 5, l32 = lane & 31;
  rf32x16_t acc[2][2];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[m][n][j] = 0.f;
  auto compute = [&](int buf) {
    const uint8_t* L = lds + buf * kRtStage;
    __builtin_amdgcn_s_setprio(1);  // a wavefront ready to compute issues first
#pragma unroll
    for (int t = 0; t < 2; ++t) {  // k16 steps; lane group q takes chunk 2t + q
      const int c = 2 * t + q;
      rbf16x8_t a[2];
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int r = 64 * wm + 32 * m + l32;
        a[m] = __builtin_bit_cast(rbf16x8_t,
                                  *reinterpret_cast<const uint4*>(L + r * kRtRow + 16 * (c ^ ((r >> 2) & 3))));
      }
#pragma unroll
      for (int p = 2; p >= 0; --p) {  // lo, mid, hi: the small terms first
#pragma unroll
        for (int n = 0; n < 2; ++n) {
          const int r = 64 * wn + 32 * n + l32;
          const rbf16x8_t b = __builtin_bit_cast(
              rbf16x8_t, *reinterpret_cast<const uint4*>(L + kRtA + p * (kRtBN * kRtRow) + r * kRtRow +
                                                         16 * (c ^ ((r >> 2) & 3))));
#pragma unroll
          for (int m = 0; m < 2; ++m)
            acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[m], b, acc[m][n], 0, 0, 0);
        }
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };
  // stage s lives in register set s % 2 until it is stored to LDS buffer s % 2
  StageRegs v[2];
  fetch(v[0], 0);
  fetch(v[1], 1);
  put(v[0], 0);
  __syncthreads();
  for (int st0 = 0; st0 < NS; st0 += 2) {  // NS is even: slices are multiples of 128 columns
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      fetch(v[j], st0 + j + 2);  // set j held stage st0 + j, stored before this stage
      __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of the stage's MFMAs
      compute(j);
      put(v[j ^ 1], j ^ 1);  // stage st0 + j + 1 (a repeat past the end)
      __syncthreads();
    }
  }
  // D layout (32x32): lane L holds column L % 32, value j row 8 (j / 4) + 4 (L / 32) + j % 4
  float* out = plog + (size_t)blockIdx.z * T * E;
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int t = m0 + 64 * wm + 32 * m + 8 * (j >> 2) + 4 * q + (j & 3);
      if (t >= T) continue;
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        const int e = e0 + 64 * wn + 32 * n + l32;
        if (e < E) out[(size_t)t * E + e] = acc[m][n][j];
      }
    }
}

hipError_t launch_router(const Dims& d, const void* x, const float* wr, const Work& w,
                         hipStream_t s) {
  float* plog = w.logits;
  switch (router_kind(d)) {
    case kRouterDecode:
      // tokens per wavefront (T <= 16 here: at most 4 wavefronts per workgroup)
      if (d.T <= 1)
        slices_launch<1>(d, x, wr, plog, s);
      else if (d.T <= 2)
        slices_launch<2>(d, x, wr, plog, s);
      else
        slices_launch<4>(d, x, wr, plog, s);
      break;
    case kRouterMfma: {
      const int ns = router_slices(d);
      // stages come in pairs (router_kind takes this kernel only for H a
      // multiple of 64, and slices of more than one are multiples of 128)
      if ((d.H / ns) % (2 * kRtKS) != 0) return hipErrorInvalidValue;
      const dim3 grid((unsigned)((d.T + kRtBM - 1) / kRtBM), (d.E + kRtBN - 1) / kRtBN, ns);
      router_mfma<<<grid, 256, 0, s>>>(reinterpret_cast<const uint16_t*>(x), wr, plog, (int)d.T,
                                       d.H, d.E, d.H / ns);
      break;
    }
    default: {
      const dim3 grid((unsigned)((d.T + 63) / 64), (d.E + 63) / 64);
      if (d.x_bf16)
        router_gemm<true><<<grid, 256, 0, s>>>(x, wr, plog, d.T, d.H, d.E);
      else
        router_gemm<false><<<grid, 256, 0, s>>>(x, wr, plog, d.T, d.H, d.E);
    }
  }
  return hipGetLastError();
}

}  // namespace moe
