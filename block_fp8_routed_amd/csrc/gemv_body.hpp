// gemv_body.hpp — the wavefront GEMV expert passes as work items (one
// group, one slab group, one 256-thread workgroup), shared by the per-pass
// kernels of expert_gemv.hip and the single-launch decode layer of
// decode_fused.hip. The lane layout and numerics are described in
// expert_gemv.hip.
#pragma once

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
  // COHERENT: rows written by other workgroups of the same kernel
  template <bool COHERENT = false, class RowOf>
  __device__ __forceinline__ void load(const void* src, RowOf row_of) {
#pragma unroll
    for (int j = 0; j < N; ++j) {
      int t, c;
      at(j, t, c);
      const uint8_t* p = reinterpret_cast<const uint8_t*>(src) + ((size_t)row_of(t) * CPR + c) * 16;
      v[j] = COHERENT ? ld16_coherent(p) : ld16(p);
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

// Chunks per lane per row of gate/up: 4 for rows of 2048+ bytes (8 KiB of
// weights per wavefront, ~108 VGPRs: four wavefronts per SIMD keep enough
// loads in flight to stream at the read ceiling), else one chunk per lane.
template <int H>
constexpr int gate_up_chunks() {
  return H >= 2048 ? 4 : 1;
}

// ------------------------------------------------------------- gate/up ---
// One work item of the gate/up pass: group descriptor gd (group, first row,
// rows) and slab group bx (slabs 4 bx .. 4 bx + 3 of PPW row pairs, one per
// wavefront), on a 256-thread workgroup; xs: LDS of gate_up_lds_bytes().
// A descriptor with group < 0 (past the last group) does nothing.
// COHERENT: h is stored at the point of coherence (read by other workgroups
// of the same kernel).
template <int H, int I, int B, int NT, int M, bool XBF16>
struct GateUpShape {
  static constexpr int SPG = I / GateUpMap<H, M>::PPW;  // slabs per group
  static constexpr int ITEMS = (SPG + 3) / 4;            // slab groups (work items) per group
  static constexpr int LDS = RowStage<H, XBF16 ? 2 : 4, NT>::BYTES;
};

template <int H, int I, int B, int NT, int M, bool XBF16, bool COHERENT = false>
__device__ __forceinline__ void gate_up_item(const void* __restrict__ x, const BankPtrs& bk,
                                             const int4 gd, const int bx,
                                             const int32_t* __restrict__ rtok, int E,
                                             float* __restrict__ h, uint8_t* xs) {
  using G = GateUpMap<H, M>;
  constexpr int LPP = G::LPP, PPW = G::PPW, SPG = I / PPW;
  static_assert(I % PPW == 0, "row pairs must split evenly into slabs");
  constexpr int XB = XBF16 ? 2 : 4;  // bytes per activation
  const int g = gd.x;
  if (g < 0) return;  // uniform over the workgroup
  const int r0 = gd.y, n = gd.z;
  const int lane = threadIdx.x & 63;
  const int slab = bx * 4 + (threadIdx.x >> 6);
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
        if (sub == LPP - 1) {
          float* dst = h + (size_t)(r0 + t0 + t) * I + i;
          if (COHERENT)
            st_coherent(dst, silu(a) * u);
          else
            *dst = silu(a) * u;
        }
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
// One work item of the down pass: group descriptor gd and slab group bx
// (output rows RW (4 bx) .. RW (4 bx + 4) - 1), on a 256-thread workgroup;
// hs, hmax, hexp: LDS of NT * I fp16, NT words and NT ints.
// HANDOFF (h produced by other workgroups of the same kernel): the weights
// and scales are requested first and wait_h() is called before the group's
// h rows are read (the caller waits there for h, with the weights in
// flight); h is read at the point of coherence. Otherwise the first pass's
// h rows are requested first and wait_h is not called. Y_COHERENT: y is
// stored at the point of coherence (read by other workgroups of the same
// kernel: the combine of complete_rows).
template <int H, int I>
struct DownShape {
  static constexpr int SPG = H / DownMap<I>::RW;  // slabs per group
  static constexpr int ITEMS = (SPG + 3) / 4;      // slab groups (work items) per group
  static constexpr int ROWS = 4 * DownMap<I>::RW;  // output rows per work item
};

struct NoWait {
  __device__ void operator()() const {}
};

template <int H, int I, int B, int NT, bool HANDOFF = false, bool Y_COHERENT = HANDOFF,
          class WaitH = NoWait>
__device__ __forceinline__ void down_item(const BankPtrs& bk, const int4 gd, const int bx, int E,
                                          const float* __restrict__ h,
                                          const int32_t* __restrict__ pair,
                                          float* __restrict__ y, uint16_t* hs, uint32_t* hmax,
                                          int* hexp, WaitH wait_h = WaitH()) {
  using D = DownMap<I>;
  constexpr int LPR = D::LPR, MD = D::MD, RW = D::RW, SPG = H / RW;
  static_assert(H % RW == 0, "rows must split evenly into slabs");
  const int g = gd.x;
  if (g < 0) return;  // uniform over the workgroup
  const int r0 = gd.y, n = gd.z;
  const int lane = threadIdx.x & 63;
  const int slab = bx * 4 + (threadIdx.x >> 6);
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
  if (!HANDOFF) st.load(h + (size_t)r0 * I, seq_row);
  __builtin_amdgcn_sched_barrier(0);
  uint4 w[MD];
  float sd[MD];
#pragma unroll
  for (int m = 0; m < MD; ++m) w[m] = ld16_nt(W + (size_t)row * I + 16 * (m * LPR + sub));
#pragma unroll
  for (int m = 0; m < MD; ++m) sd[m] = Sc[(row / B) * (I / B) + (16 * (m * LPR + sub)) / B];
  __builtin_amdgcn_sched_barrier(0);
  if (HANDOFF) {
    wait_h();
    st.template load<true>(h + (size_t)r0 * I, seq_row);
  }
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
        if (sub == LPR - 1) {
          float* dst = y + (size_t)oslot[t] * H + row;
          if (Y_COHERENT)
            st_coherent(dst, __builtin_ldexpf(v, hexp[t]));
          else
            *dst = __builtin_ldexpf(v, hexp[t]);
        }
      }
    }
    t0 += NT;
    if (t0 >= n) break;
    nv = n - t0 < NT ? n - t0 : NT;
    st.template load<HANDOFF>(h + (size_t)(r0 + t0) * I, seq_row);
    lds_barrier();  // every wavefront is done with the previous pass
    put_scaled_rows(st, hs, hmax, hexp);
  }
}

// ---------------------------------------------------------- combine ---
// The combine done by the down items themselves. After a down item (group
// descriptor gd, slab group bx) has stored its y rows coherently, it adds
// one to the count of (token, row block bx) for each of its tokens; the item
// whose addition completes a count (k routed experts plus the shared one)
// sums that token's rows of the block, in the combine kernel's order (slots
// 0 .. k-1 by gate, then the shared expert with weight 1), and writes them
// to out. No float atomics: every output is summed by one thread in a fixed
// order, so results are the combine kernel's, bit for bit. The counts
// (cmb, stride kCmbStride) must be zero before the first item adds to them.
// Called by the whole workgroup; marked / nmarked: LDS of kGemvMaxTokens + 1
// ints (free again when it returns).
constexpr int kCmbStride = 16;  // int32 words between counters: 64 bytes

template <int H, int ROWS, int ITEMS, bool OUT_BF16>
__device__ __forceinline__ void complete_rows(const int4 gd, const int bx,
                                              const int32_t* __restrict__ rtok,
                                              int32_t* __restrict__ cmb,
                                              const float* __restrict__ gates,
                                              const float* __restrict__ y, int T, int k, int S,
                                              void* __restrict__ out, int* marked,
                                              int* nmarked) {
  const int tid = threadIdx.x;
  if (tid == 0) *nmarked = 0;
  __builtin_amdgcn_s_waitcnt(0);  // this item's y stores are complete
  __syncthreads();
  const int need = k + S;
  for (int r = tid; r < gd.z; r += blockDim.x) {
    const int t = rtok[gd.y + r];
    const int old = __hip_atomic_fetch_add(cmb + (size_t)(t * ITEMS + bx) * kCmbStride, 1,
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old == need - 1) marked[atomicAdd(nmarked, 1)] = t;
  }
  __syncthreads();
  const int nm = *nmarked;
  if (nm > 0) {
    const int row0 = bx * ROWS;
    const int nrows = H - row0 < ROWS ? H - row0 : ROWS;
    for (int q = tid; q < nm * nrows; q += blockDim.x) {
      const int t = marked[q / nrows], row = row0 + q % nrows;
      // every slot's value is requested before the first is added (one load
      // latency, not k), then the sum in slot order
      float yv[kMaxTopK], gv[kMaxTopK];
#pragma unroll
      for (int j = 0; j < kMaxTopK; ++j) {
        if (j < k) {
          yv[j] = ld_coherent(y + (size_t)(t * k + j) * H + row);
          gv[j] = gates[t * k + j];
        }
      }
      const float ysh = S ? ld_coherent(y + (size_t)(T * k + t) * H + row) : 0.f;
      float acc = 0.f;
#pragma unroll
      for (int j = 0; j < kMaxTopK; ++j)
        if (j < k) acc = fmaf(gv[j], yv[j], acc);
      if (S) acc = acc + ysh;
      if (OUT_BF16)
        reinterpret_cast<uint16_t*>(out)[(size_t)t * H + row] = (uint16_t)f32_to_bf16_bits(acc);
      else
        reinterpret_cast<float*>(out)[(size_t)t * H + row] = acc;
    }
  }
  __syncthreads();
}

}  // namespace moe
