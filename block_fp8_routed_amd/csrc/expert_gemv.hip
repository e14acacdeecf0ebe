// expert_gemv.hip — the expert passes for decode-sized groups, as wavefront
// GEMV over block-FP8 weights.
//
// At decode sizes a group holds one or a few tokens, so the pass is bound by
// streaming the selected experts' E4M3 bytes from HBM once (colizig page,
// "Benchmarks": decode is memory-bandwidth-bound, not FLOP-bound). Following
// the "Features" description of fused dequant + dot product, weights are
// decoded in registers right after their 16-byte coalesced load (gfx950
// v_cvt_pk_f32_fp8) and multiplied into fp32 partial sums; a block's scale is
// applied once to the partial sum of its columns, never to single weights.
//
// Launch shape (both kernels): blockIdx.y indexes the non-empty groups listed
// by the permutation (extra blocks exit at once); blockIdx.x picks a slab of
// output rows; each of the 4 wavefronts of a workgroup owns a few rows and
// reads them whole. Tokens of a group are taken NT at a time; a larger group
// re-reads its rows (from cache) for each further NT tokens.
//
//   gate/up: rows i (gate) and I + i (up) in the same wavefront, so SwiGLU
//            h = silu(a) * u is applied before anything leaves registers;
//            h is written in fp32, row-major [P][I] in permuted row order.
//   down:    y[row][n] = sum_i h[row][i] * Wd[n][i], fp32 [P][H].
#include "device.hpp"
#include "layer.hpp"

namespace moe {

struct BankPtrs {
  const uint8_t* wgu;  // routed [E][2I][H]
  const uint8_t* wd;   // routed [E][H][I]
  const float* sgu;    // routed [E][2I/B][H/B]
  const float* sd;     // routed [E][H/B][I/B]
  const uint8_t* sh_wgu;
  const uint8_t* sh_wd;
  const float* sh_sgu;
  const float* sh_sd;
};

// Token id of permuted row `row`: routed slots are t*k + j, shared slots T*k + t.
__device__ __forceinline__ int row_token(const int32_t* pair, int row, int k, int64_t TK) {
  const int s = pair[row];
  return s < TK ? s / k : (int)(s - TK);
}

// 16 activations of token `tok` at column `col`, as fp32.
template <bool XBF16>
__device__ __forceinline__ void load_x16(const void* x, int H, int tok, int col, float* o) {
  if (XBF16) {
    const uint16_t* p = reinterpret_cast<const uint16_t*>(x) + (size_t)tok * H + col;
    const uint4 a = ld16(p), b = ld16(p + 8);
    const uint32_t u[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      o[2 * i] = bf16_lo(u[i]);
      o[2 * i + 1] = bf16_hi(u[i]);
    }
  } else {
    const float* p = reinterpret_cast<const float*>(x) + (size_t)tok * H + col;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 v = *reinterpret_cast<const float4*>(p + 4 * i);
      o[4 * i] = v.x;
      o[4 * i + 1] = v.y;
      o[4 * i + 2] = v.z;
      o[4 * i + 3] = v.w;
    }
  }
}

// sum_i dec(w[i]) * xv[i] over 16 E4M3 bytes.
__device__ __forceinline__ float dot16(const uint4 w, const float* xv) {
  float d[16];
  e4m3x4_to_f32(w.x, d);
  e4m3x4_to_f32(w.y, d + 4);
  e4m3x4_to_f32(w.z, d + 8);
  e4m3x4_to_f32(w.w, d + 12);
  float p = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) p = fmaf(d[i], xv[i], p);
  return p;
}

template <int H, int I, int B, int NT, int RP, bool XBF16>
__global__ __launch_bounds__(256) void gemv_gate_up(const void* __restrict__ x, BankPtrs bk,
                                                   const int32_t* __restrict__ offsets,
                                                   const int32_t* __restrict__ meta,
                                                   const int32_t* __restrict__ active,
                                                   const int32_t* __restrict__ pair, int k,
                                                   int64_t TK, int E, float* __restrict__ h) {
  using M = RowMap<H>;
  static_assert(I % (RP * M::RPL) == 0, "gate rows must split evenly over wavefronts");
  if ((int)blockIdx.y >= meta[0]) return;
  const int g = active[blockIdx.y];
  const bool sh = g == E;
  const uint8_t* W = sh ? bk.sh_wgu : bk.wgu + (size_t)g * 2 * I * H;
  const float* Sc = sh ? bk.sh_sgu : bk.sgu + (size_t)g * (2 * I / B) * (H / B);
  const int r0 = offsets[g], n = offsets[g + 1] - r0;
  const int lane = threadIdx.x & 63;
  const int i0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * RP * M::RPL;
  if (i0 >= I) return;
  const bool act = M::active(lane);
  const int roff = M::row(lane);

  float sg[RP][M::CH], su[RP][M::CH];
#pragma unroll
  for (int r = 0; r < RP; ++r) {
    const int i = i0 + r * M::RPL + roff;
#pragma unroll
    for (int c = 0; c < M::CH; ++c) {
      const int col = M::col(lane, c);
      sg[r][c] = act ? Sc[(i / B) * (H / B) + col / B] : 0.f;
      su[r][c] = act ? Sc[((I + i) / B) * (H / B) + col / B] : 0.f;
    }
  }

  for (int t0 = 0; t0 < n; t0 += NT) {
    int tok[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) tok[t] = (t0 + t < n) ? row_token(pair, r0 + t0 + t, k, TK) : -1;
    float ag[RP][NT], au[RP][NT];
#pragma unroll
    for (int r = 0; r < RP; ++r)
#pragma unroll
      for (int t = 0; t < NT; ++t) ag[r][t] = au[r][t] = 0.f;

#pragma unroll
    for (int c = 0; c < M::CH; ++c) {
      const int col = M::col(lane, c);
      uint4 wg[RP], wu[RP];
#pragma unroll
      for (int r = 0; r < RP; ++r) {
        const int i = i0 + r * M::RPL + roff;
        if (act) {
          wg[r] = ld16(W + (size_t)i * H + col);
          wu[r] = ld16(W + (size_t)(I + i) * H + col);
        } else {
          wg[r] = wu[r] = make_uint4(0, 0, 0, 0);
        }
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (tok[t] < 0) continue;
        float xv[16];
        if (act) {
          load_x16<XBF16>(x, H, tok[t], col, xv);
        } else {
#pragma unroll
          for (int q = 0; q < 16; ++q) xv[q] = 0.f;
        }
#pragma unroll
        for (int r = 0; r < RP; ++r) {
          ag[r][t] = fmaf(sg[r][c], dot16(wg[r], xv), ag[r][t]);
          au[r][t] = fmaf(su[r][c], dot16(wu[r], xv), au[r][t]);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < RP; ++r) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const float a = group_sum<M::RED>(ag[r][t]);
        const float u = group_sum<M::RED>(au[r][t]);
        const int q = r * NT + t;
        const bool writer = M::RED == 64 ? lane == (q & 63) : (lane % M::RED) == (q % M::RED);
        if (tok[t] >= 0 && writer)
          h[(size_t)(r0 + t0 + t) * I + i0 + r * M::RPL + roff] = silu(a) * u;
      }
    }
  }
}

template <int H, int I, int B, int NT, int RD>
__global__ __launch_bounds__(256) void gemv_down(BankPtrs bk, const int32_t* __restrict__ offsets,
                                                const int32_t* __restrict__ meta,
                                                const int32_t* __restrict__ active, int E,
                                                const float* __restrict__ h,
                                                float* __restrict__ y) {
  using M = RowMap<I>;
  static_assert(H % (RD * M::RPL) == 0, "down rows must split evenly over wavefronts");
  if ((int)blockIdx.y >= meta[0]) return;
  const int g = active[blockIdx.y];
  const bool sh = g == E;
  const uint8_t* W = sh ? bk.sh_wd : bk.wd + (size_t)g * H * I;
  const float* Sc = sh ? bk.sh_sd : bk.sd + (size_t)g * (H / B) * (I / B);
  const int r0 = offsets[g], n = offsets[g + 1] - r0;
  const int lane = threadIdx.x & 63;
  const int n0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * RD * M::RPL;
  if (n0 >= H) return;
  const bool act = M::active(lane);
  const int roff = M::row(lane);

  float sd[RD][M::CH];
#pragma unroll
  for (int r = 0; r < RD; ++r) {
    const int row = n0 + r * M::RPL + roff;
#pragma unroll
    for (int c = 0; c < M::CH; ++c)
      sd[r][c] = act ? Sc[(row / B) * (I / B) + M::col(lane, c) / B] : 0.f;
  }

  for (int t0 = 0; t0 < n; t0 += NT) {
    float acc[RD][NT];
#pragma unroll
    for (int r = 0; r < RD; ++r)
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[r][t] = 0.f;
#pragma unroll
    for (int c = 0; c < M::CH; ++c) {
      const int col = M::col(lane, c);
      uint4 wv[RD];
#pragma unroll
      for (int r = 0; r < RD; ++r)
        wv[r] = act ? ld16(W + (size_t)(n0 + r * M::RPL + roff) * I + col)
                    : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (t0 + t >= n) continue;
        float hv[16];
        if (act) {
          const float* p = h + (size_t)(r0 + t0 + t) * I + col;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float4 v = *reinterpret_cast<const float4*>(p + 4 * q);
            hv[4 * q] = v.x;
            hv[4 * q + 1] = v.y;
            hv[4 * q + 2] = v.z;
            hv[4 * q + 3] = v.w;
          }
        } else {
#pragma unroll
          for (int q = 0; q < 16; ++q) hv[q] = 0.f;
        }
#pragma unroll
        for (int r = 0; r < RD; ++r) acc[r][t] = fmaf(sd[r][c], dot16(wv[r], hv), acc[r][t]);
      }
    }
#pragma unroll
    for (int r = 0; r < RD; ++r) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const float v = group_sum<M::RED>(acc[r][t]);
        const int q = r * NT + t;
        const bool writer = M::RED == 64 ? lane == (q & 63) : (lane % M::RED) == (q % M::RED);
        if (t0 + t < n && writer)
          y[(size_t)(r0 + t0 + t) * H + n0 + r * M::RPL + roff] = v;
      }
    }
  }
}

// ---------------------------------------------------------------------------
template <int H, int I, int B, int NT, bool XBF16>
static void run_gemv(const Dims& d, const void* x, const BankPtrs& bk, const Work& w,
                     hipStream_t s, hipEvent_t after_gate_up) {
  using MG = RowMap<H>;
  using MD = RowMap<I>;
  // gate rows (and as many up rows) per wavefront-load, and down rows
  constexpr int RP = I / MG::RPL < 2 ? I / MG::RPL : 2;
  constexpr int RD = H / MD::RPL < 4 ? H / MD::RPL : 4;
  const int groups = (int)std::min<int64_t>(d.E, d.T * d.k) + d.S;
  const dim3 g1((I / (RP * MG::RPL) + 3) / 4, groups);
  gemv_gate_up<H, I, B, NT, RP, XBF16><<<g1, 256, 0, s>>>(
      x, bk, w.offsets, w.meta, w.active, w.pair, d.k, d.T * d.k, d.E,
      reinterpret_cast<float*>(w.h));
  if (after_gate_up) (void)hipEventRecord(after_gate_up, s);
  const dim3 g2((H / (RD * MD::RPL) + 3) / 4, groups);
  gemv_down<H, I, B, NT, RD><<<g2, 256, 0, s>>>(bk, w.offsets, w.meta, w.active, d.E,
                                                reinterpret_cast<const float*>(w.h), w.y);
}

template <int H, int I, int B>
static void run_gemv_nt(const Dims& d, const void* x, const BankPtrs& bk, const Work& w,
                        hipStream_t s, hipEvent_t ev) {
  // tokens per pass: enough for the largest possible group up to 8
  const int64_t most = d.T;
  if (d.x_bf16) {
    if (most <= 1) run_gemv<H, I, B, 1, true>(d, x, bk, w, s, ev);
    else if (most <= 2) run_gemv<H, I, B, 2, true>(d, x, bk, w, s, ev);
    else if (most <= 4) run_gemv<H, I, B, 4, true>(d, x, bk, w, s, ev);
    else run_gemv<H, I, B, 8, true>(d, x, bk, w, s, ev);
  } else {
    if (most <= 1) run_gemv<H, I, B, 1, false>(d, x, bk, w, s, ev);
    else if (most <= 2) run_gemv<H, I, B, 2, false>(d, x, bk, w, s, ev);
    else if (most <= 4) run_gemv<H, I, B, 4, false>(d, x, bk, w, s, ev);
    else run_gemv<H, I, B, 8, false>(d, x, bk, w, s, ev);
  }
}

#define MOE_GEMV_SHAPES(X) \
  X(64, 32, 32)            \
  X(2048, 768, 128)        \
  X(4096, 1024, 128)

bool has_gemv_instance(const Dims& d) {
#define X(h, i, b) \
  if (d.H == h && d.I == i && d.B == b) return true;
  MOE_GEMV_SHAPES(X)
#undef X
  return false;
}

hipError_t launch_experts_gemv(const Dims& d, const void* x, const moe_expert_bank& routed,
                               const moe_expert_bank* shared, const Work& w, hipStream_t s,
                               hipEvent_t after_gate_up) {
  BankPtrs bk{routed.w_gate_up, routed.w_down, routed.s_gate_up, routed.s_down,
              shared ? shared->w_gate_up : nullptr, shared ? shared->w_down : nullptr,
              shared ? shared->s_gate_up : nullptr, shared ? shared->s_down : nullptr};
#define X(h, i, b)                                              \
  if (d.H == h && d.I == i && d.B == b) {                       \
    run_gemv_nt<h, i, b>(d, x, bk, w, s, after_gate_up);        \
    return hipGetLastError();                                   \
  }
  MOE_GEMV_SHAPES(X)
#undef X
  return hipErrorInvalidValue;
}

}  // namespace moe
