// expert_mfma.hip — the expert passes for prefill-sized groups, as grouped
// bf16 MFMA GEMMs over block-FP8 weights.
//
// With tens to thousands of tokens per expert the passes are dense
// contractions, so they run on the matrix cores (v_mfma_f32_32x32x16_bf16 and
// _f16).
// Following the colizig page ("Features": dequantisation fused into the dot
// products), E4M3 weight tiles are staged in LDS as bytes and converted in
// registers as each MFMA operand is read; every E4M3 value is a bf16 (and an
// fp16) value, so the conversion (v_cvt_scalef32_pk_bf16_fp8 with a unit
// scale) is exact and the products are exact in fp32. A block's fp32 scale multiplies the partial sum of its
// 128 columns (one accumulator per scale block, folded into the running
// total), never single weights.
//
// Work list: the permutation emits one (group, first row) entry per tile of
// kMfmaBM = 128 rows of a group; each workgroup takes one (tile, block of
// output columns) pair (entries past the count exit at once).
//
// gate/up runs bf16 MFMA: activations are bf16 and the weights exact in bf16,
// so nothing is rounded on the way in; SwiGLU is applied to the accumulator
// registers and h is written as fp16 [P][I] (11-bit significand, saturated at
// +-65504). down runs fp16 MFMA on h (the weights are exact in fp16 as well)
// and writes y as fp32 [P][H]. h is the one intermediate rounded below fp32:
// fp16 keeps its relative error at 2^-11, which leaves the layer's output well
// inside its tolerance (max error <= 1e-2 x RMS); bf16 would use up most of it.
//
// MFMA operand layout (32x32x16): lane L supplies row L%32 of A and column
// L%32 of B, each as 8 k of the 16 (k = 8*(L/32) .. +7); lane L of the result
// holds column L%32, value v being row 8*(v/4) + 4*(L/32) + v%4.
#include "device.hpp"
#include "layer.hpp"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

struct MfmaBank {
  const uint8_t* wgu;
  const uint8_t* wd;
  const float* sgu;
  const float* sd;
  const uint8_t* sh_wgu;
  const uint8_t* sh_wd;
  const float* sh_sgu;
  const float* sh_sd;
};

constexpr int kBK = 128;            // K per scale block (the block edge)

// 8 E4M3 bytes (two dwords) to 8 bf16 (exact).
__device__ __forceinline__ bf16x8_t e4m3x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  const bf16x2_t a = e4m3x2_to_bf16x2<false>(lo), b = e4m3x2_to_bf16x2<true>(lo);
  const bf16x2_t c = e4m3x2_to_bf16x2<false>(hi), d = e4m3x2_to_bf16x2<true>(hi);
  bf16x8_t r;
  r[0] = a[0];
  r[1] = a[1];
  r[2] = b[0];
  r[3] = b[1];
  r[4] = c[0];
  r[5] = c[1];
  r[6] = d[0];
  r[7] = d[1];
  return r;
}

// 8 E4M3 bytes (two dwords) to 8 fp16 (exact: E4M3 values are fp16 values).
__device__ __forceinline__ f16x8_t e4m3x8_to_f16x8(uint32_t lo, uint32_t hi) {
  const f16x2_t a = e4m3x2_to_f16x2<false>(lo), b = e4m3x2_to_f16x2<true>(lo);
  const f16x2_t c = e4m3x2_to_f16x2<false>(hi), d = e4m3x2_to_f16x2<true>(hi);
  f16x8_t r;
  r[0] = a[0];
  r[1] = a[1];
  r[2] = b[0];
  r[3] = b[1];
  r[4] = c[0];
  r[5] = c[1];
  r[6] = d[0];
  r[7] = d[1];
  return r;
}

// Grouped pass, one template for both projections.
//
// A workgroup (512 threads, 8 wavefronts) computes one tile: up to kMfmaBM =
// 128 rows of one group against 512 weight rows, on 32x32x16 MFMAs
// (v_mfma_f32_32x32x16_*, which keeps the matrix pipe busy with four
// accumulators per wavefront).
//   gate/up (GU): the 512 weight rows are gate rows n0 .. n0 + 255 then the
//     matching up rows; every wavefront holds gate and up tiles of the same
//     columns, so SwiGLU pairs accumulator tiles of one wavefront. A = bf16
//     activation rows gathered by token; bf16 MFMA.
//   down: weight rows n0 .. n0 + 511 are output columns. A = fp16 h rows (a
//     group's rows are contiguous); fp16 MFMA.
// Two tile shapes, chosen per tile:
//   full (more than 64 rows): 2 x 4 wavefronts, each 64 rows x 128 weight
//     rows (2 x 4 MFMA tiles); stages fetched one ahead.
//   thin (at most 64 rows, where the pass streams weights): 1 x 8
//     wavefronts, each 64 rows x 64 weight rows (2 x 2 MFMA tiles); the A
//     tile has 64 rows, and stages are fetched two ahead, so twice the bytes
//     are in flight while the weights stream.
// K runs in stages of 64 (half a scale block). A stage's A tile and B (512 x
// 64 bytes) tile are fetched global -> registers ahead of use and written into
// the other of two LDS buffers after the current stage's MFMAs; one barrier
// per stage. Loads are never conditional (a stage index past the end is
// clamped, rows past the group's end repeat its last row), so the compiler
// can wait for exactly the loads a write needs. In LDS the 16-byte chunks of a
// row are XOR-swizzled with the row index (A: chunk c of row r at slot c ^
// ((r >> 1) & 7); B: c ^ ((r >> 2) & 3)), which makes the 32-row fragment
// reads and the tile writes free of bank conflicts.
//
// K order inside a stage: the contraction does not depend on the order of k,
// as long as A and B use the same one. Lane group q = lane / 32 reads 16 B
// bytes (16 k) of chunk 2p + q for step pair p and uses its halves in steps
// 2p and 2p + 1; the A fragment of step 2p + h for group q is then 8 k at
// chunk 4p + 2q + h (8 bf16 per A chunk).
//
// Block scales: one accumulator per output, kept in units of the current
// block's scale. Entering scale block kb, the accumulators of a 32-column
// tile are multiplied by s(kb-1) / s(kb) before its products are added, and
// by the last scale at the end; the result equals sum_kb s(kb) * P(kb) up to
// fp32 rounding (one extra rounding per block). A block with scale 0 adds
// nothing and is skipped.
// 32-row MFMA tiles wholly past the group's end are skipped, and rows past
// the end are never stored.
constexpr int kTN = 512;            // weight rows per tile
constexpr int kXcds = 8;            // accelerator complex dies (one L2 each)
constexpr int kPassThreads = 512;
constexpr int kKS = 64;             // k per pipeline stage
constexpr int kAStage = kMfmaBM * kKS * 2;  // bytes: 128 rows x 64 bf16/fp16
constexpr int kBStage = kTN * kKS;          // bytes: 512 rows x 64 E4M3
static_assert(kMfmaBM == 128, "tile geometry assumes 128-row tiles");

template <bool GU, int H, int I>
struct PassShape {
  static constexpr int K = GU ? H : I;         // contraction length
  static constexpr int COLS = GU ? 256 : 512;  // output columns per tile
  static constexpr int NOUT = GU ? I : H;      // output row length
};

typedef float f32x16_t __attribute__((ext_vector_type(16)));

// 8 E4M3 bytes to the MFMA operand type (bf16 for GU, fp16 for down) and the
// 32x32x16 MFMA of that type
template <bool GU>
struct Op;
template <>
struct Op<true> {
  typedef bf16x8_t T;
  static __device__ __forceinline__ T cvt(uint32_t lo, uint32_t hi) { return e4m3x8_to_bf16x8(lo, hi); }
  static __device__ __forceinline__ f32x16_t mma(uint4 a, T b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), b, c, 0, 0, 0);
  }
};
template <>
struct Op<false> {
  typedef f16x8_t T;
  static __device__ __forceinline__ T cvt(uint32_t lo, uint32_t hi) { return e4m3x8_to_f16x8(lo, hi); }
  static __device__ __forceinline__ f32x16_t mma(uint4 a, T b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a), b, c, 0, 0, 0);
  }
};

// Tile geometry of one shape (THIN: at most 64 rows).
template <bool GU, bool THIN>
struct TileShape {
  static constexpr int RA = THIN ? 64 : 128;  // A rows fetched per stage
  static constexpr int AC = RA * 8 / kPassThreads;  // A chunks per thread per stage
  static constexpr int NBW = THIN ? 2 : 4;    // 32-column MFMA tiles per wavefront
  static constexpr int DEPTH = THIN ? 2 : 1;  // stages fetched ahead
  // tile-relative weight row of this wavefront's MFMA tile nb (lane 0)
  static __device__ __forceinline__ int brow(int wn, int nb) {
    if (GU) {
      if (THIN) return nb == 0 ? 32 * wn : 256 + 32 * wn;
      return nb < 2 ? 64 * wn + 32 * nb : 256 + 64 * wn + 32 * (nb - 2);
    }
    return (THIN ? 64 : 128) * wn + 32 * nb;
  }
};

template <bool GU, int H, int I, bool THIN>
__device__ __forceinline__ void pass_tile(const uint16_t* __restrict__ act, const uint8_t* W,
                                          const float* Sc, const int* arow, int valid, int r0,
                                          int n0, uint8_t* lds, void* __restrict__ out) {
  using P = PassShape<GU, H, I>;
  using O = Op<GU>;
  using S = TileShape<GU, THIN>;
  constexpr int K = P::K, NS = K / kKS, AC = S::AC, NBW = S::NBW;
  static_assert(NS % 2 == 0, "stages come in pairs (one scale block)");
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = THIN ? 0 : wave >> 2, wn = THIN ? wave : wave & 3;

  // fetch map: A chunk qq = tid + 512 i is row qq / 8, chunk qq % 8; B chunk
  // qq = tid + 512 i (i < 4) is weight row qq / 4, chunk qq % 4
  // (byte offsets from the wave-uniform bases fit in 32 bits: checked on the
  // host for the activation rows, and a weight matrix is below 2 GiB)
  const uint8_t* abase = reinterpret_cast<const uint8_t*>(act);
  uint32_t asrc[AC], bsrc[4];
  int adst[AC], bdst[4];
#pragma unroll
  for (int i = 0; i < AC; ++i) {
    const int qq = tid + kPassThreads * i, r = qq >> 3, c = qq & 7;
    asrc[i] = (uint32_t)arow[r] * (K * 2) + 16 * c;
    adst[i] = r * (kKS * 2) + 16 * (c ^ ((r >> 1) & 7));
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int qq = tid + kPassThreads * i, r = qq >> 2, c = qq & 3;
    const int wrow = GU ? (r < 256 ? n0 + r : I + n0 + r - 256) : n0 + r;
    bsrc[i] = (uint32_t)wrow * K + 16 * c;
    bdst[i] = r * kKS + 16 * (c ^ ((r >> 2) & 3));
  }
  struct Regs {
    uint4 a[AC], b[4];
  };
  auto fetch = [&](Regs& R, int st) {
    st = st < NS ? st : NS - 1;  // past the end: a harmless repeat, never stored
#pragma unroll
    for (int i = 0; i < AC; ++i) R.a[i] = ld16(abase + (asrc[i] + (uint32_t)(st * kKS * 2)));
#pragma unroll
    for (int i = 0; i < 4; ++i) R.b[i] = ld16(W + (bsrc[i] + (uint32_t)(st * kKS)));
  };
  auto put = [&](const Regs& R, int buf) {
    uint8_t* A = lds + buf * (kAStage + kBStage);
    uint8_t* B = A + kAStage;
#pragma unroll
    for (int i = 0; i < AC; ++i) *reinterpret_cast<uint4*>(A + adst[i]) = R.a[i];
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(B + bdst[i]) = R.b[i];
  };

  // this wavefront's fragments: A rows 64 wm + 32 m + lane % 32; B rows
  // brow(nb) + lane % 32
  const int q = lane >> 5, l32 = lane & 31;
  int arw[2], brw[NBW];
#pragma unroll
  for (int m = 0; m < 2; ++m) arw[m] = 64 * wm + 32 * m + l32;
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) brw[nb] = S::brow(wn, nb) + l32;
  // scale row of each MFMA tile
  const float* srow[NBW];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) {
    const int br = S::brow(wn, nb);
    const int wrow = GU ? (br < 256 ? n0 + br : I + n0 + br - 256) : n0 + br;
    srow[nb] = Sc + (size_t)(wrow / kBK) * (K / kBK);
  }
  int mlive = (valid - 64 * wm + 31) / 32;  // 32-row tiles of this wavefront with rows
  mlive = mlive < 0 ? 0 : (mlive > 2 ? 2 : mlive);

  f32x16_t acc[2][NBW];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[m][nb][v] = 0.f;
  float unit[NBW];  // scale the accumulators are expressed in
  bool on[NBW];
  float snext[NBW];  // scales of the next block, read one block ahead
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) {
    unit[nb] = 0.f;
    on[nb] = false;
    snext[nb] = srow[nb][0];
  }

  auto compute = [&](int st) {
    if ((st & 1) == 0) {  // entering scale block st / 2
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) {
        const float sn = snext[nb];
        if (st + 2 < NS) snext[nb] = srow[nb][(st >> 1) + 1];
        on[nb] = sn != 0.f;
        if (on[nb]) {
          const float r = unit[nb] / sn;  // unit 0 (nothing added yet): the accumulators are 0
#pragma unroll
          for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[m][nb][v] *= r;
          unit[nb] = sn;
        }
      }
    }
    const uint8_t* A = lds + (st & 1) * (kAStage + kBStage);
    const uint8_t* B = A + kAStage;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      uint4 braw[NBW];
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) {
        const int r = brw[nb], c = 2 * p + q;
        braw[nb] = *reinterpret_cast<const uint4*>(B + r * kKS + 16 * (c ^ ((r >> 2) & 3)));
      }
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        typename O::T bf[NBW];
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb)
          bf[nb] = hh ? O::cvt(braw[nb].z, braw[nb].w) : O::cvt(braw[nb].x, braw[nb].y);
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          if (m < mlive) {
            const int r = arw[m], c = 4 * p + 2 * q + hh;
            const uint4 af = *reinterpret_cast<const uint4*>(A + r * (kKS * 2) + 16 * (c ^ ((r >> 1) & 7)));
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb)
              if (on[nb]) acc[m][nb] = O::mma(af, bf[nb], acc[m][nb]);
          }
        }
      }
    }
  };

  if (S::DEPTH == 1) {
    Regs R;
    fetch(R, 0);
    put(R, 0);
    __syncthreads();
    for (int st = 0; st < NS; ++st) {
      fetch(R, st + 1);
      compute(st);
      if (st + 1 < NS) put(R, (st + 1) & 1);
      __syncthreads();
    }
  } else {
    // stage st + 1 is in flight while stage st is computed and stage st + 2
    // is requested; the register sets alternate, so the loop runs in pairs
    Regs R0, R1;
    fetch(R0, 0);
    fetch(R1, 1);
    put(R0, 0);
    __syncthreads();
    for (int st = 0; st < NS; st += 2) {
      fetch(R0, st + 2);
      compute(st);
      put(R1, 1);
      __syncthreads();
      fetch(R1, st + 3);
      compute(st + 1);
      if (st + 2 < NS) put(R0, 0);
      __syncthreads();
    }
  }

  // D layout (32x32): lane L holds column L % 32; value v is row
  // 8 (v / 4) + 4 (L / 32) + v % 4
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int row = 64 * wm + 32 * m + 8 * (v >> 2) + 4 * q + (v & 3);
      if (row >= valid) continue;
      if (GU) {
        uint16_t* h = reinterpret_cast<uint16_t*>(out) + (size_t)(r0 + row) * I;
#pragma unroll
        for (int jj = 0; jj < NBW / 2; ++jj)
          h[n0 + S::brow(wn, jj) + l32] = f32_to_f16_sat(silu(acc[m][jj][v] * unit[jj]) *
                                                         (acc[m][jj + NBW / 2][v] * unit[jj + NBW / 2]));
      } else {
        float* y = reinterpret_cast<float*>(out) + (size_t)(r0 + row) * H;
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) y[n0 + S::brow(wn, nb) + l32] = acc[m][nb][v] * unit[nb];
      }
    }
}

template <bool GU, int H, int I>
__global__ __launch_bounds__(kPassThreads) void mfma_pass(const uint16_t* __restrict__ act,
                                                        MfmaBank bk,
                                                        const int32_t* __restrict__ meta,
                                                        const int32_t* __restrict__ tiles,
                                                        const int32_t* __restrict__ offsets,
                                                        const int32_t* __restrict__ rtok, int E,
                                                        void* __restrict__ out) {
  using P = PassShape<GU, H, I>;
  static_assert(P::K % kBK == 0 && P::NOUT % P::COLS == 0, "MFMA tiling");
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * (kAStage + kBStage)];
  __shared__ int arow[kMfmaBM];
  // XCD-aware order: workgroups are dispatched round-robin over the 8 XCDs
  // (each with its own L2), so workgroup L runs on XCD L % 8. XCD x takes row
  // tiles x, x + 8, ... and, for each, all NCB column blocks in a row, so a
  // tile's activation rows are fetched into one L2 and reused from it.
  constexpr int NCB = P::NOUT / P::COLS;
  const int xcd = blockIdx.x % kXcds, j = blockIdx.x / kXcds;
  const int tile = (j / NCB) * kXcds + xcd;
  if (tile >= meta[1]) return;
  const int g = tiles[2 * tile], r0 = tiles[2 * tile + 1];
  const int valid = min(kMfmaBM, offsets[g + 1] - r0);
  const int tid = threadIdx.x;
  const int n0 = (j % NCB) * P::COLS;
  const bool sh = g == E;
  const uint8_t* W;
  const float* Sc;
  if (GU) {
    W = sh ? bk.sh_wgu : bk.wgu + (size_t)g * 2 * I * H;
    Sc = sh ? bk.sh_sgu : bk.sgu + (size_t)g * (2 * I / kBK) * (H / kBK);
  } else {
    W = sh ? bk.sh_wd : bk.wd + (size_t)g * H * I;
    Sc = sh ? bk.sh_sd : bk.sd + (size_t)g * (H / kBK) * (I / kBK);
  }
  // source row of each tile row (GU: the token; down: the h row)
  if (tid < kMfmaBM) {
    const int rr = tid < valid ? tid : valid - 1;
    arow[tid] = GU ? rtok[r0 + rr] : r0 + rr;
  }
  __syncthreads();
  if (valid <= 64)
    pass_tile<GU, H, I, true>(act, W, Sc, arow, valid, r0, n0, lds, out);
  else
    pass_tile<GU, H, I, false>(act, W, Sc, arow, valid, r0, n0, lds, out);
}

// ---------------------------------------------------------------------------
template <int H, int I, int B>
static void run_mfma(const Dims& d, const void* x, const MfmaBank& bk, const Work& w,
                     hipStream_t s, hipEvent_t after_gate_up) {
  static_assert(B == kBK, "MFMA passes take 128 x 128 scale blocks");
  // tile slots rounded up to whole rounds of the XCDs (extra slots exit)
  const unsigned nt8 = (unsigned)((max_mfma_tiles(d) + kXcds - 1) / kXcds * kXcds);
  mfma_pass<true, H, I><<<nt8 * (I / PassShape<true, H, I>::COLS), kPassThreads, 0, s>>>(
      reinterpret_cast<const uint16_t*>(x), bk, w.meta, w.tiles, w.offsets, w.rtok, d.E, w.h);
  if (after_gate_up) (void)hipEventRecord(after_gate_up, s);
  mfma_pass<false, H, I><<<nt8 * (H / PassShape<false, H, I>::COLS), kPassThreads, 0, s>>>(
      reinterpret_cast<const uint16_t*>(w.h), bk, w.meta, w.tiles, w.offsets, w.rtok, d.E, w.y);
}

#define MOE_MFMA_SHAPES(X) \
  X(2048, 768, 128)        \
  X(4096, 1024, 128)

bool has_mfma_instance(const Dims& d) {
#define X(hh, ii, bb) \
  if (d.H == hh && d.I == ii && d.B == bb) return true;
  MOE_MFMA_SHAPES(X)
#undef X
  return false;
}

hipError_t launch_experts_mfma(const Dims& d, const void* x, const moe_expert_bank& routed,
                               const moe_expert_bank* shared, const Work& w, hipStream_t s,
                               hipEvent_t after_gate_up) {
  MfmaBank bk{routed.w_gate_up, routed.w_down, routed.s_gate_up, routed.s_down,
              shared ? shared->w_gate_up : nullptr, shared ? shared->w_down : nullptr,
              shared ? shared->s_gate_up : nullptr, shared ? shared->s_down : nullptr};
#define X(hh, ii, bb)                                    \
  if (d.H == hh && d.I == ii && d.B == bb) {             \
    run_mfma<hh, ii, bb>(d, x, bk, w, s, after_gate_up); \
    return hipGetLastError();                            \
  }
  MOE_MFMA_SHAPES(X)
#undef X
  return hipErrorInvalidValue;
}

}  // namespace moe
