// expert_gemv.hip — the expert passes for decode-sized groups, as wavefront
// GEMV over block-FP8 weights.
//
// At decode sizes a group holds one or a few tokens, so the pass is bound by
// streaming the selected experts' E4M3 bytes from HBM once (colizig page,
// "Benchmarks": decode is memory-bandwidth-bound, not FLOP-bound). Following
// the "Features" description of fused dequant + dot product, weights are
// decoded in registers after their 16-byte coalesced load and multiplied into
// fp32 partial sums; a block's scale is applied once to the partial sum of its
// columns, never to single weights.
//
// The work of a pass is cut into slabs: a few whole weight rows of one group
// (~8 KiB for gate/up, ~6 KiB for down), one slab per wavefront. Measured on
// MI355X, HBM reads come closest to peak with many short-lived wavefronts that
// each issue a few KiB of independent 16-byte loads (non-temporal, since the
// weights are read once) at high occupancy, so the kernels keep register use
// low (two tokens per pass) and issue every weight load of the slab before
// anything else.
//
//   gate/up: rows i (gate) and I + i (up) in the same slab, so SwiGLU
//            h = silu(a) * u is applied before anything leaves registers. With
//            bf16 activations, weights become exact bf16 pairs
//            (v_cvt_scalef32_pk_bf16_fp8, unit scale) and meet the packed
//            activations in v_dot2c_f32_bf16; fp32 activations use fp32 FMA.
//            h is written as fp16 (saturated at +-65504), row-major [P][I] in
//            permuted row order, the same form the MFMA family uses.
//   down:    y[row][n] = sum_i h[row][i] * Wd[n][i]: weights become exact fp16
//            pairs and meet h in v_dot2c_f32_f16; y is fp32 [P][H].
// Tokens of a group are taken NT at a time; a larger group takes several
// passes over the weights already held in registers.
#include <algorithm>

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

__device__ __forceinline__ void dec16(const uint4 w, float* d) {
  e4m3x4_to_f32(w.x, d);
  e4m3x4_to_f32(w.y, d + 4);
  e4m3x4_to_f32(w.z, d + 8);
  e4m3x4_to_f32(w.w, d + 12);
}

__device__ __forceinline__ float dot16(const float* d, const float* xv) {
  float p = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) p = fmaf(d[i], xv[i], p);
  return p;
}

// ------------------------------------------------------------- gate/up ---
template <int H, int I, int RP>
struct GateUpSlab {
  using M = RowMap<H>;
  uint4 wg[RP][M::CH], wu[RP][M::CH];
  float sg[RP][M::CH], su[RP][M::CH];
  int r0, n, i0;
};

template <int H, int I, int B, int RP>
__device__ __forceinline__ void gate_up_load(GateUpSlab<H, I, RP>& sl, int s, const BankPtrs& bk,
                                             const int4* __restrict__ gdesc, int E, int lane) {
  using M = RowMap<H>;
  constexpr int SPG = I / (RP * M::RPL);  // slabs per group
  const int y = s / SPG;
  const int4 gd = gdesc[y];
  const int g = gd.x;
  const bool sh = g == E;
  const uint8_t* W = sh ? bk.sh_wgu : bk.wgu + (size_t)g * 2 * I * H;
  const float* Sc = sh ? bk.sh_sgu : bk.sgu + (size_t)g * (2 * I / B) * (H / B);
  sl.r0 = gd.y;
  sl.n = gd.z;
  sl.i0 = (s - y * SPG) * RP * M::RPL;
  const bool act = M::active(lane);
  const int roff = M::row(lane);
#pragma unroll
  for (int r = 0; r < RP; ++r) {
    const int i = sl.i0 + r * M::RPL + roff;
#pragma unroll
    for (int c = 0; c < M::CH; ++c) {
      const int col = M::col(lane, c);
      sl.wg[r][c] = act ? ld16_nt(W + (size_t)i * H + col) : make_uint4(0, 0, 0, 0);
      sl.wu[r][c] = act ? ld16_nt(W + (size_t)(I + i) * H + col) : make_uint4(0, 0, 0, 0);
      sl.sg[r][c] = act ? Sc[(i / B) * (H / B) + col / B] : 0.f;
      sl.su[r][c] = act ? Sc[((I + i) / B) * (H / B) + col / B] : 0.f;
    }
  }
}

template <int H, int I, int NT, int RP, bool XBF16>
__device__ __forceinline__ void gate_up_compute(const GateUpSlab<H, I, RP>& sl,
                                                const void* __restrict__ x,
                                                const int32_t* __restrict__ rtok,
                                                uint16_t* __restrict__ h, int lane) {
  using M = RowMap<H>;
  const bool act = M::active(lane);
  const int roff = M::row(lane);
  for (int t0 = 0; t0 < sl.n; t0 += NT) {
    const int nv = sl.n - t0 < NT ? sl.n - t0 : NT;  // tokens in this pass (uniform)
    int tok[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) tok[t] = t < nv ? rtok[sl.r0 + t0 + t] : 0;
    float ag[RP][NT], au[RP][NT];
#pragma unroll
    for (int r = 0; r < RP; ++r)
#pragma unroll
      for (int t = 0; t < NT; ++t) ag[r][t] = au[r][t] = 0.f;

#pragma unroll
    for (int c = 0; c < M::CH; ++c) {
      const int col = M::col(lane, c);
      if (XBF16) {
        uint32_t xr[NT][8];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          if (t < nv && act) {
            const uint16_t* p = reinterpret_cast<const uint16_t*>(x) + (size_t)tok[t] * H + col;
            const uint4 a = ld16(p), b = ld16(p + 8);
            xr[t][0] = a.x;
            xr[t][1] = a.y;
            xr[t][2] = a.z;
            xr[t][3] = a.w;
            xr[t][4] = b.x;
            xr[t][5] = b.y;
            xr[t][6] = b.z;
            xr[t][7] = b.w;
          } else {
#pragma unroll
            for (int q = 0; q < 8; ++q) xr[t][q] = 0u;
          }
        }
#pragma unroll
        for (int r = 0; r < RP; ++r) {
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const uint4 wq = half ? sl.wu[r][c] : sl.wg[r][c];
            const uint32_t wd[4] = {wq.x, wq.y, wq.z, wq.w};
            bf16x2_t wb[8];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              wb[2 * q] = e4m3x2_to_bf16x2<false>(wd[q]);
              wb[2 * q + 1] = e4m3x2_to_bf16x2<true>(wd[q]);
            }
            const float sc = half ? sl.su[r][c] : sl.sg[r][c];
#pragma unroll
            for (int t = 0; t < NT; ++t) {
              if (t < nv) {
                float p = 0.f;
#pragma unroll
                for (int j = 0; j < 8; ++j) p = dot2_bf16(wb[j], xr[t][j], p);
                if (half)
                  au[r][t] = fmaf(sc, p, au[r][t]);
                else
                  ag[r][t] = fmaf(sc, p, ag[r][t]);
              }
            }
          }
        }
      } else {
        float xv[NT][16];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          if (t < nv && act) {
            const float* p = reinterpret_cast<const float*>(x) + (size_t)tok[t] * H + col;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float4 v = *reinterpret_cast<const float4*>(p + 4 * q);
              xv[t][4 * q] = v.x;
              xv[t][4 * q + 1] = v.y;
              xv[t][4 * q + 2] = v.z;
              xv[t][4 * q + 3] = v.w;
            }
          } else {
#pragma unroll
            for (int q = 0; q < 16; ++q) xv[t][q] = 0.f;
          }
        }
#pragma unroll
        for (int r = 0; r < RP; ++r) {
          float d[16];
          dec16(sl.wg[r][c], d);
#pragma unroll
          for (int t = 0; t < NT; ++t)
            if (t < nv) ag[r][t] = fmaf(sl.sg[r][c], dot16(d, xv[t]), ag[r][t]);
          dec16(sl.wu[r][c], d);
#pragma unroll
          for (int t = 0; t < NT; ++t)
            if (t < nv) au[r][t] = fmaf(sl.su[r][c], dot16(d, xv[t]), au[r][t]);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < RP; ++r) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (t >= nv) continue;
        const float a = group_sum<M::RED>(ag[r][t]);
        const float u = group_sum<M::RED>(au[r][t]);
        const int q = r * NT + t;
        const bool writer = M::RED == 64 ? lane == (q & 63) : (lane % M::RED) == (q % M::RED);
        if (writer)
          h[(size_t)(sl.r0 + t0 + t) * I + sl.i0 + r * M::RPL + roff] = f32_to_f16_sat(silu(a) * u);
      }
    }
  }
}

// grid: (slab blocks of 4 slabs, group slots); slots past the last group exit.
template <int H, int I, int B, int NT, int RP, bool XBF16>
__global__ __launch_bounds__(256) void gemv_gate_up(const void* __restrict__ x, BankPtrs bk,
                                                   const int4* __restrict__ gdesc,
                                                   const int32_t* __restrict__ rtok, int E,
                                                   uint16_t* __restrict__ h) {
  using M = RowMap<H>;
  static_assert(I % (RP * M::RPL) == 0, "gate rows must split evenly into slabs");
  constexpr int SPG = I / (RP * M::RPL);
  const int lane = threadIdx.x & 63;
  const int blk = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (blk >= SPG || gdesc[blockIdx.y].x < 0) return;
  GateUpSlab<H, I, RP> a;
  gate_up_load<H, I, B, RP>(a, (int)blockIdx.y * SPG + blk, bk, gdesc, E, lane);
  gate_up_compute<H, I, NT, RP, XBF16>(a, x, rtok, h, lane);
}

// ---------------------------------------------------------------- down ---
template <int H, int I, int RD>
struct DownSlab {
  using M = RowMap<I>;
  uint4 w[RD][M::CH];
  float sd[RD][M::CH];
  int r0, n, n0;
};

template <int H, int I, int B, int RD>
__device__ __forceinline__ void down_load(DownSlab<H, I, RD>& sl, int s, const BankPtrs& bk,
                                          const int4* __restrict__ gdesc, int E, int lane) {
  using M = RowMap<I>;
  constexpr int SPG = H / (RD * M::RPL);
  const int y = s / SPG;
  const int4 gd = gdesc[y];
  const int g = gd.x;
  const bool sh = g == E;
  const uint8_t* W = sh ? bk.sh_wd : bk.wd + (size_t)g * H * I;
  const float* Sc = sh ? bk.sh_sd : bk.sd + (size_t)g * (H / B) * (I / B);
  sl.r0 = gd.y;
  sl.n = gd.z;
  sl.n0 = (s - y * SPG) * RD * M::RPL;
  const bool act = M::active(lane);
  const int roff = M::row(lane);
#pragma unroll
  for (int r = 0; r < RD; ++r) {
    const int row = sl.n0 + r * M::RPL + roff;
#pragma unroll
    for (int c = 0; c < M::CH; ++c) {
      const int col = M::col(lane, c);
      sl.w[r][c] = act ? ld16_nt(W + (size_t)row * I + col) : make_uint4(0, 0, 0, 0);
      sl.sd[r][c] = act ? Sc[(row / B) * (I / B) + col / B] : 0.f;
    }
  }
}

template <int H, int I, int NT, int RD>
__device__ __forceinline__ void down_compute(const DownSlab<H, I, RD>& sl,
                                             const uint16_t* __restrict__ h,
                                             float* __restrict__ y, int lane) {
  using M = RowMap<I>;
  const bool act = M::active(lane);
  const int roff = M::row(lane);
  for (int t0 = 0; t0 < sl.n; t0 += NT) {
    const int nv = sl.n - t0 < NT ? sl.n - t0 : NT;  // tokens in this pass (uniform)
    float acc[RD][NT];
#pragma unroll
    for (int r = 0; r < RD; ++r)
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[r][t] = 0.f;
#pragma unroll
    for (int c = 0; c < M::CH; ++c) {
      const int col = M::col(lane, c);
      uint32_t hr[NT][8];  // 16 fp16 values of h per token
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (t < nv && act) {
          const uint16_t* p = h + (size_t)(sl.r0 + t0 + t) * I + col;
          const uint4 a = ld16(p), b = ld16(p + 8);
          hr[t][0] = a.x;
          hr[t][1] = a.y;
          hr[t][2] = a.z;
          hr[t][3] = a.w;
          hr[t][4] = b.x;
          hr[t][5] = b.y;
          hr[t][6] = b.z;
          hr[t][7] = b.w;
        } else {
#pragma unroll
          for (int q = 0; q < 8; ++q) hr[t][q] = 0u;
        }
      }
#pragma unroll
      for (int r = 0; r < RD; ++r) {
        const uint32_t wd[4] = {sl.w[r][c].x, sl.w[r][c].y, sl.w[r][c].z, sl.w[r][c].w};
        f16x2_t wf[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          wf[2 * q] = e4m3x2_to_f16x2<false>(wd[q]);
          wf[2 * q + 1] = e4m3x2_to_f16x2<true>(wd[q]);
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          if (t < nv) {
            float p = 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) p = dot2_f16(wf[j], hr[t][j], p);
            acc[r][t] = fmaf(sl.sd[r][c], p, acc[r][t]);
          }
        }
      }
    }
#pragma unroll
    for (int r = 0; r < RD; ++r) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (t >= nv) continue;
        const float v = group_sum<M::RED>(acc[r][t]);
        const int q = r * NT + t;
        const bool writer = M::RED == 64 ? lane == (q & 63) : (lane % M::RED) == (q % M::RED);
        if (writer) y[(size_t)(sl.r0 + t0 + t) * H + sl.n0 + r * M::RPL + roff] = v;
      }
    }
  }
}

template <int H, int I, int B, int NT, int RD>
__global__ __launch_bounds__(256) void gemv_down(BankPtrs bk, const int4* __restrict__ gdesc,
                                                int E, const uint16_t* __restrict__ h,
                                                float* __restrict__ y) {
  using M = RowMap<I>;
  static_assert(H % (RD * M::RPL) == 0, "down rows must split evenly into slabs");
  constexpr int SPG = H / (RD * M::RPL);
  const int lane = threadIdx.x & 63;
  const int blk = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (blk >= SPG || gdesc[blockIdx.y].x < 0) return;
  DownSlab<H, I, RD> a;
  down_load<H, I, B, RD>(a, (int)blockIdx.y * SPG + blk, bk, gdesc, E, lane);
  down_compute<H, I, NT, RD>(a, h, y, lane);
}

// ---------------------------------------------------------------------------
// Rows per slab: about `bytes` of weights, never fewer than one wavefront-load.
template <int K>
constexpr int rows_for(int bytes) {
  return RowMap<K>::RPL * RowMap<K>::CH * 1024 >= bytes ? 1 : bytes / (RowMap<K>::CH * 1024);
}

template <int H, int I, int B, int NT, bool XBF16>
static void run_gemv(const Dims& d, const void* x, const BankPtrs& bk, const Work& w,
                     hipStream_t s, hipEvent_t after_gate_up) {
  using MG = RowMap<H>;
  using MD = RowMap<I>;
  // slab sizes: gate/up RP gate rows plus RP up rows (~8 KiB), down RD rows
  // (~6-8 KiB)
  constexpr int RP0 = rows_for<H>(4096);
  constexpr int RP = I / MG::RPL < RP0 ? I / MG::RPL : RP0;
  constexpr int RD0 = rows_for<I>(8192) > 8 ? 8 : rows_for<I>(8192);
  constexpr int RD = H / MD::RPL < RD0 ? H / MD::RPL : RD0;
  constexpr int SPG1 = I / (RP * MG::RPL), SPG2 = H / (RD * MD::RPL);
  constexpr int NTD = NT;  // tokens per down pass (h fragments are packed fp16)
  const int4* gdesc = reinterpret_cast<const int4*>(w.gdesc);
  const int groups = (int)std::min<int64_t>(d.E, d.T * d.k) + d.S;
  gemv_gate_up<H, I, B, NT, RP, XBF16><<<dim3((SPG1 + 3) / 4, groups), 256, 0, s>>>(
      x, bk, gdesc, w.rtok, d.E, reinterpret_cast<uint16_t*>(w.h));
  if (after_gate_up) (void)hipEventRecord(after_gate_up, s);
  gemv_down<H, I, B, NTD, RD><<<dim3((SPG2 + 3) / 4, groups), 256, 0, s>>>(
      bk, gdesc, d.E, reinterpret_cast<const uint16_t*>(w.h), w.y);
}

template <int H, int I, int B>
static void run_gemv_nt(const Dims& d, const void* x, const BankPtrs& bk, const Work& w,
                        hipStream_t s, hipEvent_t ev) {
  // tokens per gate/up pass: up to 2 with bf16 activations, 1 with fp32 ones
  // (the down pass takes one); larger groups take several passes over the
  // weights held in registers
  if (d.x_bf16) {
    if (d.T <= 1) run_gemv<H, I, B, 1, true>(d, x, bk, w, s, ev);
    else run_gemv<H, I, B, 2, true>(d, x, bk, w, s, ev);
  } else {
    run_gemv<H, I, B, 1, false>(d, x, bk, w, s, ev);
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
#define X(h, i, b)                                       \
  if (d.H == h && d.I == i && d.B == b) {                \
    run_gemv_nt<h, i, b>(d, x, bk, w, s, after_gate_up); \
    return hipGetLastError();                            \
  }
  MOE_GEMV_SHAPES(X)
#undef X
  return hipErrorInvalidValue;
}

}  // namespace moe
