// expert_gemv.hip — the expert passes for decode-sized groups, as wavefront
// GEMV over block-FP8 weights.
//
// At decode sizes a group holds one or a few tokens, so the pass is bound by
// streaming the selected experts' E4M3 bytes from HBM once (colizig page,
// "Benchmarks": decode is memory-bandwidth-bound, not FLOP-bound). Following
// the "Features" description of fused dequant + dot product, weights are
// decoded in registers after their 16-byte coalesced load and multiplied into
// fp32 partial sums; a block's scale is applied once to the partial sum of a
// 16-byte chunk (which lies in one block), never to single weights.
//
// Lane layout. A wavefront owns several whole weight rows and gives each row
// (gate/up: each gate row together with its up row) a segment of W lanes.
// Lane s of a segment takes the row's 16-byte chunks s, s + W, s + 2W, ...,
// so the W lanes of a segment read W*16 contiguous bytes per load, and one
// sequence of DPP steps (seg_sum<W>) reduces every row of the wavefront at
// once. All weight loads of a wavefront (non-temporal, 16 bytes each) are
// issued before anything else. The group's activations (gate/up) or h rows
// (down) are staged in LDS once per workgroup and read back per chunk.
//
//   gate/up: a segment owns gate row i and up row I + i, so SwiGLU
//            h = silu(a) * u is applied in the segment's last lane. bf16
//            activations meet exact bf16 weight pairs (v_cvt_scalef32_pk_
//            bf16_fp8 with unit scale) in v_dot2c_f32_bf16; fp32 activations
//            use fp32 FMA. h is written as fp32, row-major [P][I] in permuted
//            row order (decode groups are small, so h is too).
//   down:    y[row][n] = sum_i h[row][i] * Wd[n][i]. Each workgroup stages
//            its group's h rows in LDS as fp16 scaled by one power of two
//            per row (its largest value lands in [2^14, 2^15): no overflow
//            at any fp32 magnitude, full fp16 precision down to 2^-28 of the
//            row's largest value), so exact fp16 weight pairs meet h in
//            v_dot2c_f32_f16 and the row's power of two is applied to the
//            fp32 sum; y is written as fp32 [P][H] by slot (row r's output to
//            y row pair[r]), the form the combine reads.
// Tokens of a group are taken NT at a time; a larger group takes several
// passes over the weights already held in registers.
#include <hip/hip_ext.h>

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
  // streamed banks: the slot holding each routed expert (-1: not in this
  // round), entry E = 0 when the shared group runs in this round; null: the
  // routed bank holds every expert at its own index
  const int32_t* slot;
};

// gate/up lane map: C chunks of 16 bytes per row, M per lane, LPP lanes per
// row pair, PPW pairs per wavefront.
template <int H, int M>
struct GateUpMap {
  static constexpr int C = H / 16;
  static constexpr int LPP = C / M;
  static constexpr int PPW = 64 / LPP;
  static_assert(H % 16 == 0 && C % M == 0 && LPP * M == C, "chunking");
  static_assert(LPP == 1 || LPP == 2 || LPP == 4 || LPP == 8 || LPP == 16 || LPP == 32 ||
                    LPP == 64, "lanes per pair");
};

// down lane map: C chunks per row, LPR lanes per row (8 for rows of 512+
// bytes), MD chunks per lane, RW rows per wavefront.
template <int I>
struct DownMap {
  static constexpr int C = I / 16;
  static constexpr int LPR = C >= 32 ? 8 : (C >= 4 ? 4 : C);
  static constexpr int MD = C / LPR;
  static constexpr int RW = 64 / LPR;
  static_assert(I % 16 == 0 && LPR * MD == C, "chunking");
  static_assert(LPR == 1 || LPR == 2 || LPR == 4 || LPR == 8 || LPR == 16, "lanes per row");
};

__device__ __forceinline__ void dec16(const uint4 w, float* d) {
  e4m3x4_to_f32(w.x, d);
  e4m3x4_to_f32(w.y, d + 4);
  e4m3x4_to_f32(w.z, d + 8);
  e4m3x4_to_f32(w.w, d + 12);
}

// One pass's activation rows (gate/up: x rows of the pass's tokens; down: the
// group's h rows), moved global -> registers -> LDS in two steps so that the
// kernels can place their loads against the weight stream. Thread i takes the
// 16-byte chunks i, i + 256, ... of the pass's NT rows of L elements of ELEM
// bytes; row_of(t) gives the source row of pass token t. A pass with fewer
// than NT tokens repeats its last row in the unused entries, and chunks past
// the NT rows (when 256 does not divide their count) repeat the last chunk
// into a pad of the LDS buffer, so no load or store is conditional (a
// conditional one would make the compiler wait for every load in flight).
// When a row spans whole multiples of 256 chunks, t is the same for every
// thread of a step (UNIFORM) and known at compile time after unrolling.
// LDS row t starts at byte t * L * ELEM; the buffer takes BYTES.
template <int L, int ELEM, int NT>
struct RowStage {
  static constexpr int CPR = L * ELEM / 16;  // chunks per row
  static constexpr int N = (NT * CPR + 255) / 256;
  static constexpr int BYTES = N * 256 * 16;
  static constexpr bool UNIFORM = CPR % 256 == 0;
  static_assert((L * ELEM) % 16 == 0, "rows must be whole 16-byte chunks");
  uint4 v[N];
  // row t and chunk c of register j (entries past the NT rows repeat the last chunk)
  static __device__ __forceinline__ void at(int j, int& t, int& c) {
    int i = threadIdx.x + 256 * j;
    if (i >= NT * CPR) i = NT * CPR - 1;
    t = UNIFORM ? (256 * j) / CPR : i / CPR;
    c = i - t * CPR;
  }
  template <class RowOf>
  __device__ __forceinline__ void load(const void* src, RowOf row_of) {
#pragma unroll
    for (int j = 0; j < N; ++j) {
      int t, c;
      at(j, t, c);
      v[j] = ld16(reinterpret_cast<const uint8_t*>(src) + ((size_t)row_of(t) * CPR + c) * 16);
    }
  }
  __device__ __forceinline__ void store(void* lds) const {
#pragma unroll
    for (int j = 0; j < N; ++j)
      *reinterpret_cast<uint4*>(reinterpret_cast<uint8_t*>(lds) +
                                (size_t)(threadIdx.x + 256 * j) * 16) = v[j];
  }
};

// A pass's fp32 h rows (held in registers by a RowStage<I, 4, NT>) into LDS
// as fp16, row t scaled by 2^-hexp[t] (f16_block_exponent of the row's
// largest magnitude, found with LDS atomic maxima on the magnitudes' bits:
// non-negative floats order as their bit patterns, and a maximum does not
// depend on the order of the atomics). When a row spans whole multiples of
// 64 chunks every wavefront's chunks lie in one row, so the wavefront takes
// its maximum by DPP and one lane does the atomic: 64 atomics on one LDS
// word serialise (measured: the 4096-hidden down pass at 138 us instead of
// 54). hs row t starts at element t * I.
// Ends with a barrier; the caller's previous reads of hs and hexp must have
// ended (a barrier) before the call.
template <int I, int NT>
__device__ __forceinline__ void put_scaled_rows(const RowStage<I, 4, NT>& st, uint16_t* hs,
                                                uint32_t* hmax, int* hexp) {
  using RS = RowStage<I, 4, NT>;
  if (threadIdx.x < NT) hmax[threadIdx.x] = 0u;
  lds_barrier();
#pragma unroll
  for (int j = 0; j < RS::N; ++j) {
    int t, c;
    RS::at(j, t, c);
    const uint4 w = st.v[j];
    const uint32_t m = max(max(w.x & 0x7fffffffu, w.y & 0x7fffffffu),
                           max(w.z & 0x7fffffffu, w.w & 0x7fffffffu));
    if (RS::CPR % 64 == 0) {
      const uint32_t wm = wave_max_u32(m);
      if ((threadIdx.x & 63) == 0) atomicMax(&hmax[t], wm);
    } else {
      atomicMax(&hmax[t], m);
    }
  }
  lds_barrier();
#pragma unroll
  for (int j = 0; j < RS::N; ++j) {
    int t, c;
    RS::at(j, t, c);
    const int e = f16_block_exponent(__uint_as_float(hmax[t]));
    const uint4 w = st.v[j];
    const uint32_t lo = f32_to_f16(__builtin_ldexpf(__uint_as_float(w.x), -e)) |
                        ((uint32_t)f32_to_f16(__builtin_ldexpf(__uint_as_float(w.y), -e)) << 16);
    const uint32_t hi = f32_to_f16(__builtin_ldexpf(__uint_as_float(w.z), -e)) |
                        ((uint32_t)f32_to_f16(__builtin_ldexpf(__uint_as_float(w.w), -e)) << 16);
    *reinterpret_cast<uint2*>(hs + (size_t)t * I + 4 * c) = make_uint2(lo, hi);
  }
  if (threadIdx.x < NT) hexp[threadIdx.x] = f16_block_exponent(__uint_as_float(hmax[threadIdx.x]));
  lds_barrier();
}

// ------------------------------------------------------------- gate/up ---
// grid: (slabs of PPW row pairs, 4 per workgroup; group slots). Slots past
// the last group exit at once.
template <int H, int I, int B, int NT, int M, bool XBF16>
__global__ __launch_bounds__(256) void gemv_gate_up(const void* __restrict__ x, BankPtrs bk,
                                                   const int4* __restrict__ gdesc,
                                                   const int32_t* __restrict__ rtok, int E,
                                                   float* __restrict__ h) {
  using G = GateUpMap<H, M>;
  constexpr int LPP = G::LPP, PPW = G::PPW, SPG = I / PPW;
  static_assert(I % PPW == 0, "row pairs must split evenly into slabs");
  constexpr int XB = XBF16 ? 2 : 4;  // bytes per activation
  __shared__ __attribute__((aligned(16))) uint8_t xs[RowStage<H, XBF16 ? 2 : 4, NT>::BYTES];
  const int4 gd = gdesc[blockIdx.y];
  const int g = gd.x;
  if (g < 0) return;  // uniform over the workgroup
  const int r0 = gd.y, n = gd.z;
  const int lane = threadIdx.x & 63;
  const int slab = blockIdx.x * 4 + (threadIdx.x >> 6);
  const bool live = slab < SPG;
  const int sub = lane % LPP;
  const int i = (live ? slab : 0) * PPW + lane / LPP;  // gate row; up row is I + i
  const bool sh = g == E;
  if (bk.slot && bk.slot[g] < 0) return;  // a streamed expert outside this round
  const int gs = bk.slot && !sh ? bk.slot[g] : g;
  const uint8_t* W = sh ? bk.sh_wgu : bk.wgu + (size_t)gs * 2 * I * H;
  const float* Sc = sh ? bk.sh_sgu : bk.sgu + (size_t)gs * (2 * I / B) * (H / B);

  // Issue order: the first pass's token ids (a vector load: lane u < NT
  // fetches id u), then the weights and scales, then the token rows, which
  // wait for the ids only (vector loads complete in issue order), so the
  // weights are in flight meanwhile. (A wavefront past the last slab loads
  // slab 0 again and computes nothing: no load is conditional.)
  RowStage<H, XB, NT> st;
  int nv = n < NT ? n : NT;  // tokens in this pass (uniform)
  int mytok = rtok[r0 + (lane < nv ? lane : nv - 1)];
  __builtin_amdgcn_sched_barrier(0);
  uint4 wg[M], wu[M];
  float sg[M], su[M];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int c = m * LPP + sub;
    wg[m] = ld16_nt(W + (size_t)i * H + 16 * c);
    wu[m] = ld16_nt(W + (size_t)(I + i) * H + 16 * c);
  }
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int c = m * LPP + sub;
    sg[m] = Sc[(i / B) * (H / B) + (16 * c) / B];
    su[m] = Sc[((I + i) / B) * (H / B) + (16 * c) / B];
  }
  __builtin_amdgcn_sched_barrier(0);
  // lane t of mytok holds the row of token t of the pass
  const auto token_row = [&](int t) {
    return decltype(st)::UNIFORM ? __builtin_amdgcn_readlane(mytok, t) : __shfl(mytok, t, 64);
  };
  st.load(x, token_row);
  __builtin_amdgcn_sched_barrier(0);
  st.store(xs);
  lds_barrier();
  for (int t0 = 0;;) {
    if (live) {
      float ag[NT], au[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) ag[t] = au[t] = 0.f;
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const int c = m * LPP + sub;
        if (XBF16) {
          const uint32_t gq[4] = {wg[m].x, wg[m].y, wg[m].z, wg[m].w};
          const uint32_t uq[4] = {wu[m].x, wu[m].y, wu[m].z, wu[m].w};
          bf16x2_t gb[8], ub[8];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            gb[2 * q] = e4m3x2_to_bf16x2<false>(gq[q]);
            gb[2 * q + 1] = e4m3x2_to_bf16x2<true>(gq[q]);
            ub[2 * q] = e4m3x2_to_bf16x2<false>(uq[q]);
            ub[2 * q + 1] = e4m3x2_to_bf16x2<true>(uq[q]);
          }
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            if (t < nv) {
              const uint16_t* xr = reinterpret_cast<const uint16_t*>(xs) + t * H + 16 * c;
              const uint4 a = *reinterpret_cast<const uint4*>(xr);
              const uint4 b = *reinterpret_cast<const uint4*>(xr + 8);
              const uint32_t xv[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
              float pg = 0.f, pu = 0.f;
#pragma unroll
              for (int j = 0; j < 8; ++j) {
                pg = dot2_bf16(gb[j], xv[j], pg);
                pu = dot2_bf16(ub[j], xv[j], pu);
              }
              ag[t] = fmaf(sg[m], pg, ag[t]);
              au[t] = fmaf(su[m], pu, au[t]);
            }
          }
        } else {
          float gd16[16], ud16[16];
          dec16(wg[m], gd16);
          dec16(wu[m], ud16);
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            if (t < nv) {
              const float* xr = reinterpret_cast<const float*>(xs) + t * H + 16 * c;
              float pg = 0.f, pu = 0.f;
#pragma unroll
              for (int j = 0; j < 16; ++j) {
                pg = fmaf(gd16[j], xr[j], pg);
                pu = fmaf(ud16[j], xr[j], pu);
              }
              ag[t] = fmaf(sg[m], pg, ag[t]);
              au[t] = fmaf(su[m], pu, au[t]);
            }
          }
        }
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (t >= nv) continue;
        const float a = seg_sum<LPP>(ag[t]);
        const float u = seg_sum<LPP>(au[t]);
        if (sub == LPP - 1) h[(size_t)(r0 + t0 + t) * I + i] = silu(a) * u;
      }
    }
    t0 += NT;
    if (t0 >= n) break;
    nv = n - t0 < NT ? n - t0 : NT;
    mytok = rtok[r0 + t0 + (lane < nv ? lane : nv - 1)];
    st.load(x, token_row);
    lds_barrier();  // every wavefront is done with the previous pass
    st.store(xs);
    lds_barrier();
  }
}

// ---------------------------------------------------------------- down ---
template <int H, int I, int B, int NT>
__global__ __launch_bounds__(256) void gemv_down(BankPtrs bk, const int4* __restrict__ gdesc,
                                                int E, const float* __restrict__ h,
                                                const int32_t* __restrict__ pair,
                                                float* __restrict__ y) {
  using D = DownMap<I>;
  constexpr int LPR = D::LPR, MD = D::MD, RW = D::RW, SPG = H / RW;
  static_assert(H % RW == 0, "rows must split evenly into slabs");
  __shared__ __attribute__((aligned(16))) uint16_t hs[NT * I];  // scaled fp16 h rows
  __shared__ uint32_t hmax[NT];
  __shared__ int hexp[NT];
  const int4 gd = gdesc[blockIdx.y];
  const int g = gd.x;
  if (g < 0) return;  // uniform over the workgroup
  const int r0 = gd.y, n = gd.z;
  const int lane = threadIdx.x & 63;
  const int slab = blockIdx.x * 4 + (threadIdx.x >> 6);
  const bool live = slab < SPG;
  const int sub = lane % LPR;
  const int row = (live ? slab : 0) * RW + lane / LPR;
  const bool sh = g == E;
  if (bk.slot && bk.slot[g] < 0) return;  // a streamed expert outside this round
  const int gs = bk.slot && !sh ? bk.slot[g] : g;
  const uint8_t* W = sh ? bk.sh_wd : bk.wd + (size_t)gs * H * I;
  const float* Sc = sh ? bk.sh_sd : bk.sd + (size_t)gs * (H / B) * (I / B);

  // the group's h rows are contiguous (rows r0 .. r0 + n - 1); the first
  // pass's rows are requested before the weights and scales, so staging them
  // in LDS does not wait for the weights. No load is conditional, as in
  // gemv_gate_up.
  RowStage<I, 4, NT> st;
  int nv = n < NT ? n : NT;  // tokens in this pass (uniform)
  const auto seq_row = [&](int t) { return t < nv ? t : nv - 1; };
  st.load(h + (size_t)r0 * I, seq_row);
  __builtin_amdgcn_sched_barrier(0);
  uint4 w[MD];
  float sd[MD];
#pragma unroll
  for (int m = 0; m < MD; ++m) w[m] = ld16_nt(W + (size_t)row * I + 16 * (m * LPR + sub));
#pragma unroll
  for (int m = 0; m < MD; ++m) sd[m] = Sc[(row / B) * (I / B) + (16 * (m * LPR + sub)) / B];
  __builtin_amdgcn_sched_barrier(0);
  put_scaled_rows(st, hs, hmax, hexp);
  for (int t0 = 0;;) {
    // y is stored by slot (row r's output goes to y row pair[r]), so the
    // combine reads a token's outputs without the inverse permutation
    int oslot[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) oslot[t] = pair[r0 + t0 + (t < nv ? t : nv - 1)];
    if (live) {
      float acc[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[t] = 0.f;
#pragma unroll
      for (int m = 0; m < MD; ++m) {
        const int c = m * LPR + sub;
        const uint32_t wq[4] = {w[m].x, w[m].y, w[m].z, w[m].w};
        f16x2_t wf[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          wf[2 * q] = e4m3x2_to_f16x2<false>(wq[q]);
          wf[2 * q + 1] = e4m3x2_to_f16x2<true>(wq[q]);
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          if (t < nv) {
            const uint4 a = *reinterpret_cast<const uint4*>(hs + t * I + 16 * c);
            const uint4 b = *reinterpret_cast<const uint4*>(hs + t * I + 16 * c + 8);
            const uint32_t hv[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
            float p = 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) p = dot2_f16(wf[j], hv[j], p);
            acc[t] = fmaf(sd[m], p, acc[t]);
          }
        }
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (t >= nv) continue;
        const float v = seg_sum<LPR>(acc[t]);
        if (sub == LPR - 1) y[(size_t)oslot[t] * H + row] = __builtin_ldexpf(v, hexp[t]);
      }
    }
    t0 += NT;
    if (t0 >= n) break;
    nv = n - t0 < NT ? n - t0 : NT;
    st.load(h + (size_t)(r0 + t0) * I, seq_row);
    lds_barrier();  // every wavefront is done with the previous pass
    put_scaled_rows(st, hs, hmax, hexp);
  }
}

// ---------------------------------------------------------------------------
// Chunks per lane per row of gate/up: 4 for rows of 2048+ bytes (8 KiB of
// weights per wavefront, ~108 VGPRs: four wavefronts per SIMD keep enough
// loads in flight to stream at the read ceiling), else one chunk per lane.
template <int H>
constexpr int gate_up_chunks() {
  return H >= 2048 ? 4 : 1;
}

template <int H, int I, int B, int NT, bool XBF16>
static void run_gemv(const Dims& d, const void* x, const BankPtrs& bk, const Work& w,
                     hipStream_t s, KernelEvents ev) {
  constexpr int M = gate_up_chunks<H>();
  constexpr int SPG1 = I / GateUpMap<H, M>::PPW, SPG2 = H / DownMap<I>::RW;
  const int4* gdesc = reinterpret_cast<const int4*>(w.gdesc);
  const int groups = (int)std::min<int64_t>(d.E, d.T * d.k) + d.S;
  const dim3 grid((SPG1 + 3) / 4, groups);
  float* h = static_cast<float*>(w.h);
  if (ev.any())  // the events take the kernel's own start and end times
    hipExtLaunchKernelGGL(gemv_gate_up<H, I, B, NT, M, XBF16>, grid, dim3(256), 0, s, ev.begin,
                          ev.end, 0, x, bk, gdesc, static_cast<const int32_t*>(w.rtok), d.E, h);
  else
    gemv_gate_up<H, I, B, NT, M, XBF16><<<grid, 256, 0, s>>>(x, bk, gdesc, w.rtok, d.E, h);
  gemv_down<H, I, B, NT><<<dim3((SPG2 + 3) / 4, groups), 256, 0, s>>>(
      bk, gdesc, d.E, h, w.pair, static_cast<float*>(w.y));
}

template <int H, int I, int B>
static void run_gemv_nt(const Dims& d, const void* x, const BankPtrs& bk, const Work& w,
                        hipStream_t s, KernelEvents ev) {
  // tokens per pass: up to 4 (fp32 activations of wide rows: 1, which keeps
  // their LDS stage at 16 KiB); larger groups take several passes over the
  // weights held in registers
  constexpr int NTF = H <= 1024 ? 4 : 1;
  if (d.x_bf16) {
    if (d.T <= 1) run_gemv<H, I, B, 1, true>(d, x, bk, w, s, ev);
    else if (d.T <= 2) run_gemv<H, I, B, 2, true>(d, x, bk, w, s, ev);
    else run_gemv<H, I, B, 4, true>(d, x, bk, w, s, ev);
  } else {
    if (d.T <= 1) run_gemv<H, I, B, 1, false>(d, x, bk, w, s, ev);
    else run_gemv<H, I, B, NTF, false>(d, x, bk, w, s, ev);
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
                               KernelEvents gate_up_events, const int32_t* slot) {
  BankPtrs bk{routed.w_gate_up, routed.w_down, routed.s_gate_up, routed.s_down,
              shared ? shared->w_gate_up : nullptr, shared ? shared->w_down : nullptr,
              shared ? shared->s_gate_up : nullptr, shared ? shared->s_down : nullptr, slot};
#define X(h, i, b)                                       \
  if (d.H == h && d.I == i && d.B == b) {                \
    run_gemv_nt<h, i, b>(d, x, bk, w, s, gate_up_events); \
    return hipGetLastError();                            \
  }
  MOE_GEMV_SHAPES(X)
#undef X
  return hipErrorInvalidValue;
}

}  // namespace moe
