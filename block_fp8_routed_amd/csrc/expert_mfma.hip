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
// registers and h is written as scaled fp16 [P][I]: each row's 128 columns
// (one tile's output) share one power of two, chosen so that the block's
// largest value lands in [2^14, 2^15) (f16_block_exponent), with the
// exponent byte in hexps [P][I/128]. down runs fp16 MFMA on h (the weights
// are exact in fp16 as well): a tile first brings each of its h rows to one
// common power of two (the largest of the row's block exponents; the other
// blocks are multiplied by 2^-d in fp16, exact unless a block is more than
// 2^14 below the row's largest), and applies it to the fp32 result; y is
// written as scaled fp16 [P][H] by slot (row r's output to y row pair[r]),
// one exponent byte per row and 128 columns in yexps. h and y are the two
// intermediates rounded below fp32: fp16 keeps their relative error at
// 2^-11, which leaves the layer's output well inside its tolerance (max
// error <= 1e-2 x RMS; bf16 would use up most of it), and the exponents keep
// any fp32 magnitude representable.
//
// MFMA operand layout (32x32x16): lane L supplies row L%32 of A and column
// L%32 of B, each as 8 k of the 16 (k = 8*(L/32) .. +7); lane L of the result
// holds column L%32, value v being row 8*(v/4) + 4*(L/32) + v%4.
//
// The FP8 variant's two passes, mfma_pass_f8 (both operands of both
// contractions E4M3: the activations quantised beforehand with one
// power-of-two scale per token and 128 columns, h quantised the same way in
// the gate/up epilogue), are described where they are defined, below the
// bf16 passes.
#include <hip/hip_ext.h>

#include "device.hpp"
#include "e4m3_round.hpp"
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
  const int32_t* slot;  // streamed banks: the slot of each routed expert (-1: skip), entry E
                        // for the shared group (null: every expert at its own index)
};

typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kBK = 128;            // K per scale block (the block edge)
constexpr int kPassThreadsDecl = 512;  // threads of a grouped pass workgroup

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

// unit / s for the ratio form of the block scales: the accumulators, held in
// units of the last block's scale, move to the units of the next block's
// scale s (nonzero). Mantissas and exponents are taken apart (frexp reads
// subnormal scales exactly, where the reciprocal of a subnormal overflows),
// so the ratio is finite whenever unit / s is within fp32 range; for normal
// scales it equals unit * rcp(s), the power-of-two factors being exact.
// unit 0 (nothing accumulated yet): 1.
__device__ __forceinline__ float scale_ratio(float unit, float s) {
  if (unit == 0.f) return 1.f;
  const float mu = __builtin_amdgcn_frexp_mantf(unit), ms = __builtin_amdgcn_frexp_mantf(s);
  const int e = __builtin_amdgcn_frexp_expf(unit) - __builtin_amdgcn_frexp_expf(s);
  return __builtin_ldexpf(mu * __builtin_amdgcn_rcpf(ms), e);
}

// A tile's scale rows, before its stages: a block whose scale lies more
// than 2^48 below its row's running scale (the last kept nonzero scale
// before it along K) is dropped (its scale read as 0). Entering it, the
// ratio form would multiply accumulators held in units of the running scale
// by up to 2^127 and overflow; the block adds less than 2^-48 of what a
// block at the running scale can. Magnitudes are compared (a scale may be
// negative).
constexpr float kScaleDropRatio = 0x1p-48f;
__device__ __forceinline__ void drop_far_blocks(float* row, int nkb) {
  float unit = 0.f;
  for (int kb = 0; kb < nkb; ++kb) {
    const float s = row[kb];
    if (s == 0.f) continue;
    if (unit != 0.f && fabsf(s) < fabsf(unit) * kScaleDropRatio)
      row[kb] = 0.f;
    else
      unit = s;
  }
}

// ---- epilogue helpers: an fp32 output tile of 128 columns through LDS ----
// Tile row r at byte r * 512, 16-byte chunk c at slot c ^ f32_swz(r), so the
// two row groups of one accumulator write land on different banks.
__device__ __forceinline__ int f32_swz(int r) { return ((r >> 2) & 1) << 3; }
// (rp: the 512 bytes of tile row `row`)
__device__ __forceinline__ void put_f32_row(uint8_t* rp, int row, int col, float v) {
  *reinterpret_cast<float*>(rp + 16 * ((col >> 2) ^ f32_swz(row)) + 4 * (col & 3)) = v;
}
__device__ __forceinline__ void put_f32(uint8_t* lds, int row, int col, float v) {
  put_f32_row(lds + row * 512, row, col, v);
}
// Rows [0, valid) of an RA-row fp32 tile in LDS (as put_f32 leaves it; row r
// at rows(r)) stored as scaled fp16: 16 lanes (one DPP row) per tile row take 8 values each, a
// DPP maximum gives the row's largest magnitude and f16_block_exponent its
// power of two; dst(r) is the row's first fp16 element in global memory,
// ebyte(r) where its exponent byte goes. `wave` is the (uniform) wavefront
// index: the thread index is rebuilt from it and the lane id, which keeps
// the loop before the epilogue from holding the thread index in a register.
template <int RA, class Rows, class Dst, class Eb>
__device__ __forceinline__ void store_f16_rows(Rows rows, int valid, int wave, Dst dst, Eb ebyte) {
  static_assert((RA * 16) % kPassThreadsDecl == 0, "tile rows per thread");
  const int tid = 64 * wave + (int)__lane_id();
#pragma unroll
  for (int i = 0; i < RA * 16 / kPassThreadsDecl; ++i) {
    const int idx = tid + kPassThreadsDecl * i, r = idx >> 4, k = idx & 15;
    const uint8_t* rp = rows(r);
    const uint4 a = *reinterpret_cast<const uint4*>(rp + 16 * ((2 * k) ^ f32_swz(r)));
    const uint4 b = *reinterpret_cast<const uint4*>(rp + 16 * ((2 * k + 1) ^ f32_swz(r)));
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    uint32_t mx = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) mx = max(mx, w[j] & 0x7fffffffu);
    const int e = f16_block_exponent(__uint_as_float(row16_max_u32(mx)));
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      o[j] = f32_to_f16(__builtin_ldexpf(__uint_as_float(w[2 * j]), -e)) |
             ((uint32_t)f32_to_f16(__builtin_ldexpf(__uint_as_float(w[2 * j + 1]), -e)) << 16);
    if (r >= valid) continue;
    *reinterpret_cast<uint4*>(dst(r) + 8 * k) = make_uint4(o[0], o[1], o[2], o[3]);
    if (k == 0) *ebyte(r) = (uint8_t)(e + kF16ExpBias);
  }
}

// fp16 factors that bring an h block to its row's common power of two:
// 2^d (d <= 0) as two fp16 multipliers 2^a and 2^b (a = max(d, -24), b =
// max(d - a, -24)), since fp16 holds powers of two down to 2^-24 only; the
// two fp16 bit patterns in one word (low: a).
__device__ __forceinline__ uint32_t f16_pow2_bits(int a) {  // a in [-24, 0]
  return a >= -14 ? (uint32_t)(a + 15) << 10 : 1u << (a + 24);
}
__device__ __forceinline__ uint32_t rescale_word(int d) {
  const int a = d > -24 ? d : -24;
  const int b = d - a > -24 ? d - a : -24;
  return f16_pow2_bits(a) | (f16_pow2_bits(b) << 16);
}
// 8 fp16 values (a 16-byte chunk) times the two multipliers of a rescale word
__device__ __forceinline__ uint4 rescale_f16x8(uint4 v, uint32_t word) {
  const f16x2_t fa = __builtin_bit_cast(f16x2_t, (word & 0xffffu) * 0x10001u);
  const f16x2_t fb = __builtin_bit_cast(f16x2_t, (word >> 16) * 0x10001u);
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) w[j] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, w[j]) * fa * fb);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// ---- the down passes' y: scaled fp16 with an exponent known in advance ----
// A down tile's 256 output columns are two blocks of 128, and each block's
// weights share one scale per 128 K (the scale grid's 128 x 128 blocks), so
// with |A| <= amax_a(row) elementwise the output obeys
//   |y| <= amax_a(row) * 448 * 128 * S(b),  S(b) = sum over K blocks of s(b, kb)
// (|code| <= 448). With 2^g(row) >= amax_a(row) / 2^15 (bf16 pass: the h
// row's common power of two, h' < 2^15; FP8 pass: the largest of the row's h
// block exponents, codes <= 448 folded into q) and 2^q(b) > 448 * 128 * S(b)
// (* 448 / 2^15 for the FP8 pass), y is stored as fp16(y * 2^-ey) with
// ey = g(row) + q(b), below 2^15 by construction: no maximum has to be found
// across the tile. The bound is loose by the usual cancellation of a sum
// (typically 2^8 - 2^10), which still leaves every y value down to 2^-20 or
// so of its block's largest with the full fp16 significand; the exponent
// byte is ey + 127, clamped to [0, 254] (only beyond fp32's own range).
__device__ __forceinline__ int y_block_q(const float* srow, int nkb, float coef) {
  float sum = 0.f;
  for (int kb = 0; kb < nkb; ++kb) sum += srow[kb];
  // 2^q > coef * sum: q = binary exponent (frexp) of the product, 0 for 0
  const float b = coef * sum;
  return b > 0.f ? __builtin_amdgcn_frexp_expf(b) : 0;
}
__device__ __forceinline__ int clamp_exp(int e) { return e < -127 ? -127 : (e > 127 ? 127 : e); }

// The down tile's fp16 y through LDS (a tile of 256 fp16 columns, row r at
// rows(r), 16-byte chunk c at slot c ^ oswz(r)), every row then stored as
// whole 16-byte chunks by slot (orow), with the exponent bytes. acc holds
// the wavefront's MW x 2 MFMA tiles; value (row, block b) is stored as
// acc * unit[nb] * 2^(G(row) - ey), ey = clamp(g(row) + q(b)), where G is
// the power of two acc is expressed in (the bf16 pass: g; FP8: 0).
template <int RA, int MW, int H, bool GISG, class Rows>
__device__ __forceinline__ void store_y_tile(const f32x16_t (&acc)[MW][2], const float* unit,
                                             const int* rowg, const int* yq, int arow0, int wn,
                                             bool idle, int valid, int n0, const int* orow,
                                             int wave, Rows rows, uint16_t* y,
                                             uint8_t* yexps) {
  constexpr int ORB = 256 * 2, OCH = ORB / 16;
  auto oswz = [](int r) { return ((r & 1) | (((r >> 2) & 1) << 1)) << 2; };
  const int ln = (int)__lane_id(), q = ln >> 5, l32 = ln & 31;
  const bool odd = l32 & 1;
  if (!idle) {
#pragma unroll
    for (int m = 0; m < MW; ++m)
#pragma unroll
      for (int v = 0; v < 16; v += 2) {
        const int row = arow0 + 32 * m + 8 * (v >> 2) + 4 * q + (v & 3);
        const int g0 = rowg[row], g1 = rowg[row + 1];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const int col0 = 64 * wn + 32 * nb, b = col0 >> 7;
          const int s0 = (GISG ? g0 : 0) - clamp_exp(g0 + yq[b]);
          const int s1 = (GISG ? g1 : 0) - clamp_exp(g1 + yq[b]);
          const uint32_t a = f32_to_f16(__builtin_ldexpf(acc[m][nb][v] * unit[nb], s0));
          const uint32_t c = f32_to_f16(__builtin_ldexpf(acc[m][nb][v + 1] * unit[nb], s1));
          // lanes exchange one value with their neighbour (DPP quad_perm
          // 1,0,3,2): an even lane writes two columns of row R, an odd lane
          // two columns of row R + 1
          const uint32_t send = odd ? a : c;
          const uint32_t recv = (uint32_t)__builtin_amdgcn_mov_dpp((int)send, 0xb1, 0xf, 0xf, false);
          const int r = row + (odd ? 1 : 0);
          const int col = col0 + l32 - (odd ? 1 : 0);
          const uint32_t word = odd ? (recv | (c << 16)) : (a | (recv << 16));
          *reinterpret_cast<uint32_t*>(rows(r) + 16 * (((2 * col) >> 4) ^ oswz(r)) +
                                       ((2 * col) & 15)) = word;
        }
      }
  }
  __syncthreads();
  const int tid = 64 * wave + ln;
  static_assert((RA * OCH) % kPassThreadsDecl == 0, "output chunks per thread");
#pragma unroll
  for (int i = 0; i < RA * OCH / kPassThreadsDecl; ++i) {
    const int idx = tid + kPassThreadsDecl * i, r = idx / OCH, c = idx % OCH;
    if (r >= valid) continue;
    const uint4 val = *reinterpret_cast<const uint4*>(rows(r) + 16 * (c ^ oswz(r)));
    *reinterpret_cast<uint4*>(y + (size_t)orow[r] * H + n0 + 8 * c) = val;
  }
  if (tid < 2 * RA) {
    const int r = tid % RA, b = tid / RA;
    if (r < valid)
      yexps[(size_t)orow[r] * (H / 128) + n0 / 128 + b] =
          (uint8_t)(clamp_exp(rowg[r] + yq[b]) + kF16ExpBias);
  }
}

// Outputs of a bf16 pass: gate/up writes h (scaled fp16 [P][I]) and its
// exponent bytes; down reads h's exponent bytes and writes y (scaled fp16
// [P][H], by slot) and its exponent bytes.
struct PassIO {
  void* out;
  uint8_t* oexps;
  const uint8_t* hexps;
};

// Grouped pass, one template for both projections.
//
// A workgroup (512 threads, 8 wavefronts as 2 x 4) computes one tile: up to
// kMfmaBM = 128 rows of one group against 256 weight rows, on 32x32x16 MFMAs
// (v_mfma_f32_32x32x16_*). Registers are held to 128 per lane and LDS to 64
// KiB per workgroup, so two workgroups (four wavefronts per SIMD) share a
// compute unit and hide each other's LDS and memory latency.
//   gate/up (GU): the 256 weight rows are gate rows n0 .. n0 + 127 then the
//     matching up rows; wavefront wn holds gate rows 32 wn .. 32 wn + 31 and
//     the matching up rows, so SwiGLU pairs accumulator tiles of one
//     wavefront. A = bf16 activation rows gathered by token; bf16 MFMA.
//   down: weight rows n0 .. n0 + 255 are output columns; wavefront wn holds
//     64 of them. A = fp16 h rows (a group's rows are contiguous); fp16 MFMA.
// Two tile shapes, chosen per tile:
//   full (more than 64 rows): wavefront (wm, wn) takes rows 64 wm .. + 63
//     (two 32-row MFMA tiles). K runs in stages of 64 (half a scale block),
//     a stage's A tile (128 rows) and B tile (256 x 64 bytes) going through
//     one of two LDS buffers, one stage ahead, one barrier per stage.
//     gate/up (pass_tile_gu_dma) loads them straight from global memory
//     into LDS (buffer_load ... lds), with no register round trip; down
//     fetches them into registers and writes them to LDS after the current
//     stage's MFMAs, bringing each h block to its row's common power of two
//     on the way.
//   thin (at most 64 rows, where the pass streams weights): rows 32 wm ..
//     + 31 (one MFMA tile); the A tile has 64 rows. gate/up: K runs in
//     stages of 128 (one scale block), so every weight row is read 128
//     bytes at a time, which the memory system streams faster than 64-byte
//     pieces of 256 rows; two stages are in flight in registers, and the
//     stage (16 KiB of A, 32 KiB of B) goes through one LDS buffer, with a
//     barrier before and after its MFMAs. down (K = I, a few stages): 64-k
//     stages in two LDS buffers, four fetched ahead.
// Loads are never conditional (a stage index past the end is clamped, rows
// past the group's end repeat its last row), so the compiler can wait for
// exactly the loads a write needs. In LDS the 16-byte chunks of a row are
// XOR-swizzled with the row index (64-k stages: A chunk c of row r at slot
// c ^ ((r >> 1) & 7), B at c ^ ((r >> 2) & 3); 128-k stages: A at c ^ (r &
// 15), B at c ^ ((r >> 1) & 7)), which makes the 32-row fragment reads and
// the tile writes free of bank conflicts.
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
// fp32 rounding (the ratio costs about two roundings per block). A block
// with scale 0 adds nothing: its codes are zeroed when the tile is written to
// LDS. The tile's scales (two scale rows, K / 128 each) are copied to LDS
// once at the start: read from global memory inside the loop, each would be
// a vector load issued behind the weight prefetches, and as vector loads
// complete in order, waiting for it would wait for every stage in flight.
// Rows past the group's end are computed with the rest (they repeat the last
// row) and never stored; a wavefront whose rows all lie past it skips its
// MFMAs. The results go out through LDS, so that every output row is stored
// as whole 16-byte chunks.
constexpr int kTN = 256;            // weight rows per tile
constexpr int kXcds = 8;            // accelerator complex dies (one L2 each)
constexpr int kPassThreads = kPassThreadsDecl;
constexpr int kLdsBytes = 65536;    // stage buffers of one workgroup
static_assert(kMfmaBM == 128, "tile geometry assumes 128-row tiles");

template <bool GU, int H, int I>
struct PassShape {
  static constexpr int K = GU ? H : I;         // contraction length
  static constexpr int COLS = GU ? 128 : 256;  // output columns per tile
  static constexpr int NOUT = GU ? I : H;      // output row length
};


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
  // thin gate/up tiles (K = H) take 128-k stages through one LDS buffer; the
  // down pass's K (= I) is short enough that the deeper pipeline of 64-k
  // stages in two buffers pays more than the longer row pieces
  static constexpr bool WIDE = THIN && GU;
  static constexpr int RA = THIN ? 64 : 128;  // A rows fetched per stage
  static constexpr int KS = WIDE ? 128 : 64;  // k per stage
  static constexpr int CA = KS * 2 / 16;      // 16-byte chunks per A row (bf16/fp16)
  static constexpr int CB = KS / 16;          // 16-byte chunks per B row (E4M3)
  static constexpr int AC = RA * CA / kPassThreads;   // A chunks per thread per stage
  static constexpr int BC = kTN * CB / kPassThreads;  // B chunks per thread per stage
  static constexpr int ASTAGE = RA * KS * 2;  // bytes of a stage's A tile
  static constexpr int BSTAGE = kTN * KS;     // bytes of a stage's B tile
  static constexpr int BUFS = WIDE ? 1 : 2;   // LDS stage buffers
  static constexpr int MW = THIN ? 1 : 2;     // 32-row MFMA tiles per wavefront
  static constexpr int NBW = 2;               // 32-column MFMA tiles per wavefront
  static constexpr int DEPTH = WIDE ? 2 : (THIN ? 4 : 1);  // stages fetched ahead
  static_assert(BUFS * (ASTAGE + BSTAGE) <= kLdsBytes, "stage buffers exceed the LDS block");
  static_assert(AC * kPassThreads == RA * CA && BC * kPassThreads == kTN * CB, "fetch map");
  // tile-relative first row of this wavefront's rows
  static __device__ __forceinline__ int arow0(int wm) { return (THIN ? 32 : 64) * wm; }
  // tile-relative weight row of this wavefront's MFMA tile nb
  static __device__ __forceinline__ int brow(int wn, int nb) {
    if (GU) return nb == 0 ? 32 * wn : kTN / 2 + 32 * wn;
    return 64 * wn + 32 * nb;
  }
  // LDS slot of chunk c of A row r / B row r
  static __device__ __forceinline__ int aswz(int r) { return CA == 16 ? (r & 15) : ((r >> 1) & 7); }
  static __device__ __forceinline__ int bswz(int r) { return CB == 8 ? ((r >> 1) & 7) : ((r >> 2) & 3); }
};

template <bool GU, int H, int I, bool THIN>
__device__ __forceinline__ void pass_tile(const uint16_t* __restrict__ act, const uint8_t* W,
                                          const float* ss, const int* arow, const int* orow,
                                          const uint32_t* hfac, const int* herow, const int* yq,
                                          int valid, int r0, int n0, uint8_t* lds, uint8_t* ldsb,
                                          PassIO io) {
  using P = PassShape<GU, H, I>;
  using O = Op<GU>;
  using S = TileShape<GU, THIN>;
  // LDS: two separate halves, lds and ldsb. Full tiles take
  // pass_tile_gu_dma / pass_tile_down_dma; the thin gate/up stage (one
  // buffer) has its A tile in lds and its B tile in ldsb; the thin down
  // pass's stage buffer b is lds (b = 0) or ldsb (b = 1), A then B.
  static_assert(THIN, "full tiles load their B tiles through LDS-DMA");
  static_assert(GU ? (S::ASTAGE <= kLdsBytes / 2 && S::BSTAGE <= kLdsBytes / 2)
                   : S::ASTAGE + S::BSTAGE <= kLdsBytes / 2, "stage buffers fit the LDS halves");
  static_assert(S::RA * 512 <= kLdsBytes / 2, "output tile fits one LDS half");
  auto abuf = [&](int buf) -> uint8_t* { return GU || buf == 0 ? lds : ldsb; };
  auto bbuf = [&](int buf) -> uint8_t* { return GU ? ldsb : abuf(buf) + S::ASTAGE; };
  constexpr int K = P::K, KS = S::KS, NS = K / KS, AC = S::AC, BC = S::BC, MW = S::MW,
                NBW = S::NBW, CA = S::CA, CB = S::CB;
  constexpr int NKB = K / kBK;
  static_assert(K % KS == 0 && kBK % KS == 0, "stages must tile the scale blocks");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches only
  const int wm = wave >> 2, wn = wave & 3;

  // fetch map: A chunk qq = tid + 512 i is row qq / CA, chunk qq % CA; B chunk
  // qq = tid + 512 i is tile weight row qq / CB, chunk qq % CB. Moving qq by
  // 512 moves the row by a multiple of 32, which leaves the swizzle alone, so
  // the LDS targets and the sources of i > 0 are constant offsets from those
  // of i = 0 (GU: tile rows 128 .. 255 are the up rows I + n0 ..). Byte
  // offsets from the wave-uniform bases fit in 32 bits (checked on the host
  // for the activation rows; a weight matrix is below 2 GiB).
  const __amdgpu_buffer_rsrc_t arsrc = buffer_rsrc(act, 0xffffffffu);
  const __amdgpu_buffer_rsrc_t brsrc = buffer_rsrc(W, (uint32_t)((GU ? 2 * I : H) * K));
  constexpr int ARS = kPassThreads / CA, BRS = kPassThreads / CB;  // row step per i
  uint32_t asrc[AC];
  const int ar0 = tid / CA, ac0 = tid % CA;
  const int adst0 = ar0 * (KS * 2) + 16 * (ac0 ^ S::aswz(ar0));
#pragma unroll
  for (int i = 0; i < AC; ++i) asrc[i] = (uint32_t)arow[ar0 + ARS * i] * (K * 2) + 16 * ac0;
  const int br0 = tid / CB, bc0 = tid % CB;
  const int bdst0 = br0 * KS + 16 * (bc0 ^ S::bswz(br0));
  const uint32_t bsrc0 = (uint32_t)(n0 + br0) * K + 16 * bc0;
  // weight row offset (in rows) of chunk group i's tile row BRS i
  auto brow_of = [](int i) -> int {
    const int tr = BRS * i;
    return GU ? (tr < kTN / 2 ? tr : I + tr - kTN / 2) : tr;
  };
  struct Regs {
    uint4 a[AC], b[BC];
  };
  // scale rows (in LDS) of this thread's B chunks: chunk group i lies in the
  // tile's scale row (BRS i) / 128 (GU: the gate block, then the up block;
  // down: rows n0 .. + 127, then n0 + 128 .. + 255), so these are uniform; a
  // block of scale 0 has its codes zeroed when written to LDS
  const float* bscale[BC];
#pragma unroll
  for (int i = 0; i < BC; ++i) bscale[i] = ss + (BRS * i / kBK) * NKB;
  auto fetch = [&](Regs& R, int st) {
    st = st < NS ? st : NS - 1;  // past the end: a harmless repeat, never stored
#pragma unroll
    for (int i = 0; i < AC; ++i) R.a[i] = buffer_ld16(arsrc, asrc[i], (uint32_t)(st * KS * 2));
#pragma unroll
    // thin gate/up tiles stream weights read once, a whole 128-byte line per
    // row and stage: non-temporal. (64-k stages read half lines, whose other
    // half the next stage finds in L2 only if the line was kept.)
    for (int i = 0; i < BC; ++i)
      R.b[i] = buffer_ld16<S::WIDE ? kBufNonTemporal : 0>(brsrc, bsrc0,
                                                          (uint32_t)(brow_of(i) * K + st * KS));
  };
  auto put = [&](Regs& R, int buf, int st) {
    uint8_t* A = abuf(buf);
    uint8_t* B = bbuf(buf);
    const int kb = st * KS / kBK;
    bool zero = false;
#pragma unroll
    for (int i = 0; i < BC; ++i) zero |= bscale[i][kb] == 0.f;
    if (zero) {  // rare: a zero block scale (uniform branch)
#pragma unroll
      for (int i = 0; i < BC; ++i)
        if (bscale[i][kb] == 0.f) R.b[i] = make_uint4(0, 0, 0, 0);
    }
    if (!GU) {  // h rows to their row's common power of two
#pragma unroll
      for (int i = 0; i < AC; ++i) R.a[i] = rescale_f16x8(R.a[i], hfac[(ar0 + ARS * i) * NKB + kb]);
    }
#pragma unroll
    for (int i = 0; i < AC; ++i) *reinterpret_cast<uint4*>(A + adst0 + ARS * (KS * 2) * i) = R.a[i];
#pragma unroll
    for (int i = 0; i < BC; ++i) *reinterpret_cast<uint4*>(B + bdst0 + BRS * KS * i) = R.b[i];
  };

  // this wavefront's fragments: A rows arow0 + 32 m + lane % 32; B rows
  // brow(nb) + lane % 32. The row offsets are multiples of 32, so the swizzle
  // of a fragment read depends on lane % 32 only.
  const int q = lane >> 5, l32 = lane & 31;
  const int afr = (S::arow0(wm) + l32) * (KS * 2), asw = S::aswz(l32);
  const int bfr = l32 * KS, bsw = S::bswz(l32);
  // scale row (in LDS) of each MFMA tile: its weight rows lie in the tile's
  // scale row brow / 128
  const float* srow[NBW];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) srow[nb] = ss + (S::brow(wn, nb) / kBK) * NKB;

  f32x16_t acc[MW][NBW];
#pragma unroll
  for (int m = 0; m < MW; ++m)
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[m][nb][v] = 0.f;
  float unit[NBW];   // scale the accumulators are expressed in
  float snext[NBW];  // scales of the next block, read one block ahead
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) {
    unit[nb] = 0.f;
    snext[nb] = srow[nb][0];
  }

  // One stage. Every MFMA tile is computed even when rows past the group's
  // end fill it (their results are not stored); nothing inside is
  // conditional, so the compiler schedules the MFMAs and LDS reads freely.
  // K order inside a stage: the contraction does not depend on the order of
  // k, as long as A and B use the same one. Lane group q = lane / 32 reads
  // 16 B bytes (16 k) of chunk 2p + q for step pair p and uses its halves in
  // steps 2p and 2p + 1; the A fragment of step 2p + h for group q is then 8
  // k at chunk 4p + 2q + h (8 bf16 per A chunk).
  // a wavefront whose rows all lie past the group's end (a thin tile of at
  // most 32 rows) skips its MFMAs; it still fetches and stores its share of
  // the stage and takes part in every barrier (uniform per wavefront)
  const bool idle = S::arow0(wm) >= valid;
  auto compute = [&](int buf, int st) {
    if (idle) return;
    if ((st * KS) % kBK == 0) {  // entering scale block kb
      const int kb = st * KS / kBK;
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) {
        const float sn = snext[nb];
        if (kb + 1 < NKB) snext[nb] = srow[nb][kb + 1];
        const bool on = sn != 0.f;
        // unit 0 (nothing added yet): the accumulators are 0 and stay 0; a
        // block of scale 0 (codes zeroed in LDS) leaves the unit as it is
        const float r = on ? scale_ratio(unit[nb], sn) : 1.f;
#pragma unroll
        for (int m = 0; m < MW; ++m)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[m][nb][v] *= r;
        unit[nb] = on ? sn : unit[nb];
      }
    }
    const uint8_t* A = abuf(buf);
    const uint8_t* B = bbuf(buf);
    // the stage's MFMAs run at raised wave priority, so that a wavefront
    // ready to compute issues ahead of those waiting on loads and barriers
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int p = 0; p < KS / 32; ++p) {
      uint4 braw[NBW];
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb)
        braw[nb] = *reinterpret_cast<const uint4*>(B + S::brow(wn, nb) * KS + bfr +
                                                   16 * ((2 * p + q) ^ bsw));
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        typename O::T bf[NBW];
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb)
          bf[nb] = hh ? O::cvt(braw[nb].z, braw[nb].w) : O::cvt(braw[nb].x, braw[nb].y);
#pragma unroll
        for (int m = 0; m < MW; ++m) {
          const uint4 af = *reinterpret_cast<const uint4*>(A + afr + 32 * m * (KS * 2) +
                                                           16 * ((4 * p + 2 * q + hh) ^ asw));
#pragma unroll
          for (int nb = 0; nb < NBW; ++nb) acc[m][nb] = O::mma(af, bf[nb], acc[m][nb]);
        }
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };

  if (S::BUFS == 2) {
    // two LDS buffers and a ring of DEPTH register sets: while stage st is
    // computed, stages st + 1 .. st + DEPTH are in flight (stage s lives in
    // set s % DEPTH); the loop is unrolled by DEPTH so the sets are fixed
    // registers; one barrier per stage
    constexpr int D = S::DEPTH;
    static_assert(NS % D == 0, "stage count must be a multiple of the prefetch depth");
    Regs R[D];
    // the prologue issues the stages in order, as the loop does: the waits the
    // compiler places at the loop head must hold for both ways in, and loads
    // of different stages interleaved here would make them wait for nearly
    // every load in flight
#pragma unroll
    for (int j = 0; j < D; ++j) {
      fetch(R[j], j);
      __builtin_amdgcn_sched_barrier(0);
    }
    put(R[0], 0, 0);
    __syncthreads();
    for (int st0 = 0; st0 < NS; st0 += D) {
#pragma unroll
      for (int j = 0; j < D; ++j) {
        const int st = st0 + j;
        fetch(R[j], st + D);  // set j held stage st, written to LDS before this stage
        compute(st & 1, st);
        if (st + 1 < NS) put(R[(j + 1) % D], (st + 1) & 1, st + 1);
        __syncthreads();
      }
    }
  } else {
    // one LDS buffer and a ring of DEPTH register sets (as above), with a
    // barrier before and after each stage's MFMAs
    constexpr int D = S::DEPTH;
    static_assert(NS % D == 0, "stage count must be a multiple of the prefetch depth");
    Regs R[D];
#pragma unroll
    for (int j = 0; j < D; ++j) {  // in stage order (see above)
      fetch(R[j], j);
      __builtin_amdgcn_sched_barrier(0);
    }
    for (int st0 = 0; st0 < NS; st0 += D) {
#pragma unroll
      for (int j = 0; j < D; ++j) {
        const int st = st0 + j;
        put(R[j], 0, st);     // the previous stage's reads ended at the last barrier
        fetch(R[j], st + D);  // set j is free once written
        __syncthreads();
        compute(0, st);
        __syncthreads();
      }
    }
  }

  // Epilogue through LDS (free after the loop's last barrier) as fp32 tiles
  // of 128 columns, stored as scaled fp16 rows (store_f16_rows). D layout
  // (32x32): lane L holds column L % 32; value v is row 8 (v / 4) + 4 (L / 32)
  // + v % 4. gate/up: the tile's 128 h columns in one round; down: 256
  // output columns in two rounds of 128 (wavefronts wn = 0, 1, then 2, 3),
  // the h row's common power of two applied to the fp32 results.
  static_assert(S::RA * 512 <= kLdsBytes, "output tile exceeds the LDS block");
  // the lane's position, rebuilt here rather than kept live through the loop
  const int eln = (int)__lane_id(), eq = eln >> 5, el32 = eln & 31;
  if (GU) {
    if (!idle) {
#pragma unroll
      for (int m = 0; m < MW; ++m)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = S::arow0(wm) + 32 * m + 8 * (v >> 2) + 4 * eq + (v & 3);
          put_f32(lds, row, S::brow(wn, 0) + el32,
                  silu(acc[m][0][v] * unit[0]) * (acc[m][1][v] * unit[1]));
        }
    }
    __syncthreads();
    uint16_t* h = static_cast<uint16_t*>(io.out);
    store_f16_rows<S::RA>(
        [&](int r) { return lds + r * 512; }, valid, wave,
        [&](int r) { return h + (size_t)(r0 + r) * I + n0; },
        [&](int r) { return io.oexps + (size_t)(r0 + r) * (I / kBK) + n0 / kBK; });
  } else {
    store_y_tile<S::RA, MW, H, true>(acc, unit, herow, yq, S::arow0(wm), wn, idle, valid, n0,
                                     orow, wave, [&](int r) { return lds + r * 512; },
                                     static_cast<uint16_t*>(io.out), io.oexps);
  }
}

// A full gate/up tile (more than 64 rows; shape and K order as pass_tile's
// full tiles) whose stages go from global memory straight into LDS
// (buffer_load_dwordx4 ... lds): lane l of a wavefront's load writes its 16
// bytes at the wavefront's LDS base + 16 l, so a load fills 1 KiB of LDS in
// lane order and the swizzle is applied on the source side (the lane at
// slot s of row r fetches chunk s ^ swz(r)). Stage st (64 k) goes to buffer
// st % 2: its A tile (128 rows x 128 bytes) at offset 0, its B tile (256 rows
// x 64 bytes: gate rows n0 .., then the matching up rows) at 16 KiB; each
// wavefront issues two 1 KiB loads of each. The two buffers are separate
// LDS objects, so the compiler sees that loads into one do not touch the
// other while its fragments are read. Stage st + 1 is issued before stage
// st's MFMAs; each wavefront waits for its own loads (vmcnt 0) before the
// barrier that ends the stage, after which the whole stage is in LDS and
// the buffer just read is free. A block of scale 0 has its B fragments
// zeroed as they are read. The epilogue goes through the two buffers as one
// fp32 tile (rows 0 .. 63 in the first).
template <int H, int I>
__device__ __forceinline__ void pass_tile_gu_dma(const uint16_t* __restrict__ act,
                                                 const uint8_t* W, const float* ss,
                                                 const int* arow, int valid, int r0, int n0,
                                                 uint8_t* lds0, uint8_t* lds1, PassIO io) {
  using O = Op<true>;
  constexpr int K = H, KS = 64, NS = K / KS, NKB = K / kBK;
  constexpr int ABYTES = kMfmaBM * KS * 2, BBYTES = kTN * KS;
  static_assert(NS % 2 == 0 && kBK % KS == 0, "stages come in pairs and tile the scale blocks");
  static_assert(ABYTES + BBYTES <= kLdsBytes / 2 && kMfmaBM * 512 <= kLdsBytes,
                "stage and output tile fit the two LDS halves");
  static_assert(ABYTES == 2 * 16 * kPassThreads && BBYTES == 2 * 16 * kPassThreads,
                "two 16-byte loads per lane and tile");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform
  const int wm = wave >> 2, wn = wave & 3;
  const __amdgpu_buffer_rsrc_t arsrc = buffer_rsrc(act, 0xffffffffu);
  const __amdgpu_buffer_rsrc_t brsrc = buffer_rsrc(W, (uint32_t)(2 * I * K));
  // load i of this lane fills LDS slot qq = tid + 512 i of the tile: A row
  // qq / 8 (slot qq % 8), B tile row qq / 4 (slot qq % 4); tile B rows
  // 0 .. 127 are gate rows n0 .., rows 128 .. 255 the up rows I + n0 ..
  uint32_t aoff[2], boff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int qq = tid + kPassThreads * i;
    const int r = qq >> 3, c = (qq & 7) ^ ((r >> 1) & 7);
    aoff[i] = (uint32_t)arow[r] * (K * 2) + 16 * c;
    const int rb = qq >> 2, cb = (qq & 3) ^ ((rb >> 2) & 3);
    const int wrow = rb < kTN / 2 ? n0 + rb : I + n0 + rb - kTN / 2;
    boff[i] = (uint32_t)wrow * K + 16 * cb;
  }
  // load i of wavefront w fills bytes 16 (512 i + 64 w) .. + 1023 of its tile
  constexpr int kLoadBytes = 16 * kPassThreads;  // LDS bytes of one load over the workgroup
  auto issue = [&](uint8_t* buf, int st) {
    st = st < NS ? st : NS - 1;  // past the end: a harmless repeat, never read
#pragma unroll
    for (int i = 0; i < 2; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(arsrc, buf + kLoadBytes * i + 1024 * wave, 16,
                                               aoff[i], (uint32_t)(st * KS * 2), 0, 0);
#pragma unroll
    for (int i = 0; i < 2; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(brsrc, buf + ABYTES + kLoadBytes * i + 1024 * wave,
                                               16, boff[i], (uint32_t)(st * KS), 0, 0);
  };
  // fragments (as pass_tile): A rows 64 wm + 32 m + lane % 32, B tile rows
  // brow(nb) + lane % 32; row offsets are multiples of 32, so the swizzle of
  // a fragment read depends on lane % 32 only
  const int q = lane >> 5, l32 = lane & 31;
  const int afr = (64 * wm + l32) * (KS * 2), asw = (l32 >> 1) & 7;
  const int bfr = ABYTES + l32 * KS, bsw = (l32 >> 2) & 3;
  auto brow = [&](int nb) { return nb == 0 ? 32 * wn : kTN / 2 + 32 * wn; };
  const float* srow[2] = {ss, ss + NKB};  // gate block, up block
  f32x16_t acc[2][2];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[m][nb][v] = 0.f;
  float unit[2] = {0.f, 0.f};  // scale the accumulators are expressed in
  bool on[2] = {true, true};   // the current block's scale is not 0
  auto compute = [&](const uint8_t* buf, int st) {
    if ((st * KS) % kBK == 0) {  // entering scale block kb (as pass_tile)
      const int kb = st * KS / kBK;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const float sn = srow[nb][kb];
        on[nb] = sn != 0.f;
        const float r = on[nb] ? scale_ratio(unit[nb], sn) : 1.f;
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[m][nb][v] *= r;
        unit[nb] = on[nb] ? sn : unit[nb];
      }
    }
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int p = 0; p < KS / 32; ++p) {
      uint4 braw[2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        braw[nb] = *reinterpret_cast<const uint4*>(buf + bfr + brow(nb) * KS +
                                                   16 * ((2 * p + q) ^ bsw));
        if (!on[nb]) braw[nb] = make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        typename O::T bf[2];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          bf[nb] = hh ? O::cvt(braw[nb].z, braw[nb].w) : O::cvt(braw[nb].x, braw[nb].y);
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const uint4 af = *reinterpret_cast<const uint4*>(buf + afr + 32 * m * (KS * 2) +
                                                           16 * ((4 * p + 2 * q + hh) ^ asw));
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) acc[m][nb] = O::mma(af, bf[nb], acc[m][nb]);
        }
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };
  constexpr int kWaitVm0 = 0x0F70;  // s_waitcnt vmcnt(0) (lgkm and exp counts not waited on)
  issue(lds0, 0);
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __syncthreads();
#pragma unroll 1
  for (int st = 0; st < NS; st += 2) {
    issue(lds1, st + 1);
    compute(lds0, st);
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
    issue(lds0, st + 2);
    compute(lds1, st + 1);
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
  }
  // epilogue (as pass_tile's): the fp32 tile, rows 0 .. 63 in lds0 and
  // 64 .. 127 in lds1, then scaled fp16 rows
  const int eln = (int)__lane_id(), eq = eln >> 5, el32 = eln & 31;
  auto rows = [&](int r) { return (r < 64 ? lds0 : lds1) + (r & 63) * 512; };
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int row = 64 * wm + 32 * m + 8 * (v >> 2) + 4 * eq + (v & 3);
      put_f32_row(rows(row), row, brow(0) + el32,
                  silu(acc[m][0][v] * unit[0]) * (acc[m][1][v] * unit[1]));
    }
  __syncthreads();
  uint16_t* h = static_cast<uint16_t*>(io.out);
  store_f16_rows<kMfmaBM>(
      rows, valid, wave, [&](int r) { return h + (size_t)(r0 + r) * I + n0; },
      [&](int r) { return io.oexps + (size_t)(r0 + r) * (I / kBK) + n0 / kBK; });
}

// A full down tile (more than 64 rows; shape and K order as pass_tile's full
// tiles, K = I): B tiles (256 weight rows x 64 bytes per stage) go straight
// into LDS as in pass_tile_gu_dma; A tiles (h rows, fp16) go through
// registers, where each h block is brought to its row's common power of two
// (rescale words in hfac) before it is written to LDS. Stage st uses buffer
// st % 2 (lds or ldsb: A at offset 0, B at 16 KiB). A block of scale 0 has
// its B fragments zeroed as they are read.
template <int H, int I>
__device__ __forceinline__ void pass_tile_down_dma(const uint16_t* __restrict__ act,
                                                   const uint8_t* W, const float* ss,
                                                   const int* arow, const int* orow,
                                                   const uint32_t* hfac, const int* herow,
                                                   const int* yq, int valid, int r0, int n0,
                                                   uint8_t* lds0, uint8_t* lds1, PassIO io) {
  using O = Op<false>;
  constexpr int K = I, KS = 64, NS = K / KS, NKB = K / kBK;
  constexpr int ABYTES = kMfmaBM * KS * 2, BBYTES = kTN * KS;
  static_assert(NS % 2 == 0 && kBK % KS == 0, "stages come in pairs and tile the scale blocks");
  static_assert(ABYTES + BBYTES <= kLdsBytes / 2 && kMfmaBM * 512 <= kLdsBytes,
                "stage and output tile fit the two LDS halves");
  static_assert(ABYTES == 2 * 16 * kPassThreads && BBYTES == 2 * 16 * kPassThreads,
                "two 16-byte chunks per lane and tile");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform
  const int wm = wave >> 2, wn = wave & 3;
  const __amdgpu_buffer_rsrc_t arsrc = buffer_rsrc(act, 0xffffffffu);
  const __amdgpu_buffer_rsrc_t brsrc = buffer_rsrc(W, (uint32_t)(H * K));
  // A: chunk i of this thread is tile row ar0 + 64 i (8 chunks of 16 bytes
  // per row and stage), written at its swizzled slot; moving the row by 64
  // leaves the swizzle alone. B: load i fills tile slot qq = tid + 512 i
  // (weight row n0 + qq / 4, slot qq % 4), as pass_tile_gu_dma.
  const int ar0 = tid >> 3, ac0 = tid & 7;
  const int adst0 = ar0 * (KS * 2) + 16 * (ac0 ^ ((ar0 >> 1) & 7));
  uint32_t asrc[2], boff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    asrc[i] = (uint32_t)arow[ar0 + 64 * i] * (K * 2) + 16 * ac0;
    const int qq = tid + kPassThreads * i;
    const int rb = qq >> 2, cb = (qq & 3) ^ ((rb >> 2) & 3);
    boff[i] = (uint32_t)(n0 + rb) * K + 16 * cb;
  }
  constexpr int kLoadBytes = 16 * kPassThreads;  // LDS bytes of one load over the workgroup
  uint4 ra[2];
  auto fetch = [&](uint8_t* buf, int st) {  // A into registers, B into buf
    st = st < NS ? st : NS - 1;  // past the end: a harmless repeat, never read
#pragma unroll
    for (int i = 0; i < 2; ++i) ra[i] = buffer_ld16(arsrc, asrc[i], (uint32_t)(st * KS * 2));
#pragma unroll
    for (int i = 0; i < 2; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(brsrc, buf + ABYTES + kLoadBytes * i + 1024 * wave,
                                               16, boff[i], (uint32_t)(st * KS), 0, 0);
  };
  auto put = [&](uint8_t* buf, int st) {  // A to LDS, each h block to its row's power of two
    st = st < NS ? st : NS - 1;  // as fetch
    const int kb = st * KS / kBK;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      *reinterpret_cast<uint4*>(buf + adst0 + 64 * (KS * 2) * i) =
          rescale_f16x8(ra[i], hfac[(ar0 + 64 * i) * NKB + kb]);
  };
  const int q = lane >> 5, l32 = lane & 31;
  const int afr = (64 * wm + l32) * (KS * 2), asw = (l32 >> 1) & 7;
  const int bfr = ABYTES + l32 * KS, bsw = (l32 >> 2) & 3;
  auto brow = [&](int nb) { return 64 * wn + 32 * nb; };
  const float* srow[2] = {ss + (brow(0) / kBK) * NKB, ss + (brow(1) / kBK) * NKB};
  f32x16_t acc[2][2];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[m][nb][v] = 0.f;
  float unit[2] = {0.f, 0.f};
  bool on[2] = {true, true};
  auto compute = [&](const uint8_t* buf, int st) {
    if ((st * KS) % kBK == 0) {  // entering scale block kb (as pass_tile)
      const int kb = st * KS / kBK;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const float sn = srow[nb][kb];
        on[nb] = sn != 0.f;
        const float r = on[nb] ? scale_ratio(unit[nb], sn) : 1.f;
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[m][nb][v] *= r;
        unit[nb] = on[nb] ? sn : unit[nb];
      }
    }
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int p = 0; p < KS / 32; ++p) {
      uint4 braw[2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        braw[nb] = *reinterpret_cast<const uint4*>(buf + bfr + brow(nb) * KS +
                                                   16 * ((2 * p + q) ^ bsw));
        if (!on[nb]) braw[nb] = make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        typename O::T bf[2];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          bf[nb] = hh ? O::cvt(braw[nb].z, braw[nb].w) : O::cvt(braw[nb].x, braw[nb].y);
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const uint4 af = *reinterpret_cast<const uint4*>(buf + afr + 32 * m * (KS * 2) +
                                                           16 * ((4 * p + 2 * q + hh) ^ asw));
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) acc[m][nb] = O::mma(af, bf[nb], acc[m][nb]);
        }
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };
  // each wavefront waits for its own loads (vmcnt 0; the A loads are also
  // waited for by the LDS writes) before the barrier that ends the stage
  // before theirs
  constexpr int kWaitVm0 = 0x0F70;  // s_waitcnt vmcnt(0)
  fetch(lds0, 0);
  put(lds0, 0);
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __syncthreads();
#pragma unroll 1
  for (int st = 0; st < NS; st += 2) {
    fetch(lds1, st + 1);
    compute(lds0, st);
    put(lds1, st + 1);
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
    fetch(lds0, st + 2);
    compute(lds1, st + 1);
    put(lds0, st + 2);  // past the end: a repeat, never read
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
  }
  store_y_tile<kMfmaBM, 2, H, true>(
      acc, unit, herow, yq, 64 * wm, wn, false, valid, n0, orow, wave,
      [&](int r) { return (r < 64 ? lds0 : lds1) + (r & 63) * 512; },
      static_cast<uint16_t*>(io.out), io.oexps);
}

constexpr int kChunkTiles = 512;  // tile lists at least this long are dealt in chunks
static_assert(kXcds == kXcdCount, "one XCD count");

// The row tile of this workgroup (its column block is j % NCB), or -1 for a
// slot without one. XCD-aware: workgroups are dispatched round-robin over
// the XCDs (each with its own L2), so workgroup L runs on XCD L % 8, and XCD
// x takes, for each of its tiles, all NCB column blocks in a row, so that a
// tile's activation rows are fetched into one L2 and reused from it. On
// long tile lists XCD x takes a contiguous chunk of tiles, so the row tiles
// of a hot expert share few L2s; the permutation cuts the chunks at equal
// cost (tile_cost), so every XCD gets a like share of the work. On short
// ones it takes tiles x, x + 8, ... The launch gives every XCD
// mfma_chunk_tiles slots (long lists can occur) or a round-robin share.
template <int NCB>
__device__ __forceinline__ int pass_tile_of(const int32_t* __restrict__ meta, int bid, int& j) {
  const int xcd = bid % kXcds;
  j = bid / kXcds;
  // loaded together (clamped indices): no load waits for another
  const int nt = meta[1];
  const int lo = meta[kMetaXcdBounds + (xcd > 0 ? xcd - 1 : 0)];
  const int hi = meta[kMetaXcdBounds + (xcd < kXcds - 1 ? xcd : 0)];
  if (nt >= kChunkTiles) {
    const int t = (xcd > 0 ? lo : 0) + j / NCB;
    return t < (xcd < kXcds - 1 ? hi : nt) ? t : -1;
  }
  const int t = (j / NCB) * kXcds + xcd;
  return t < nt ? t : -1;
}

// LDS of a pass workgroup. lds, ldsb: stage buffers and the output tile, two
// separate arrays, so that the compiler sees that loads into one leave the
// other alone; arow: source row of each tile row; orow (down): the y row
// (slot) of each tile row; ss: the tile's two weight scale rows; hfac, herow
// (down): the h rows' rescale words per block and their common exponents;
// yq (down): the two output column blocks' bound exponents; go: the
// outcome of a one-launch down item's wait.
struct PassLds {
  uint8_t* lds;
  uint8_t* ldsb;
  int* arow;
  int* orow;
  float* ss;
  uint32_t* hfac;
  int* herow;
  int* yq;
  int* go;
};

// One-launch hand-over of h (mfma_layer): word 0 is the give-up word, word
// 1 + t tile t's counter (bits 0-5: gate/up items done; bits 6 (1 + x) ..
// 6 (1 + x) + 5: those done on XCD x). Null in the two-launch passes.
struct LayerSync {
  uint64_t* words;
  uint32_t* status;
  uint32_t spin;  // polls before a wait gives up
};
constexpr uint32_t kLayerSpin = 1u << 21;  // default poll bound (about a second)

// XCD of the calling wavefront: hardware register XCC_ID, bits 0-3 (0-7
// on this 8-XCD chip; masked to 3 bits so that a counter field is never
// shifted out of its 64-bit word)
__device__ __forceinline__ int xcc_id() {
  return (int)(__builtin_amdgcn_s_getreg((3 << 11) | 20) & (uint32_t)(kXcds - 1));
}
static_assert(6 * (1 + kXcds) <= 64, "one six-bit count per XCD after the total");

// Down workgroup of mfma_layer: wait until every gate/up item of the tile
// has published (thread 0 polls at the point of coherence, bounded), and
// check that they ran on this XCD: h goes between them through the XCD's
// L2, which another XCD does not see. false: give up the tile (a wait of
// the call gave up; the status word says so).
template <int NGU>
__device__ __forceinline__ bool layer_wait(const LayerSync& ls, int tile, int* flag) {
  static_assert(NGU < 64, "a tile's gate/up item count fits six bits");
  if (threadIdx.x == 0) {
    uint64_t* ctr = ls.words + 1 + tile;
    uint64_t v = ld_coherent(ctr);
    bool ok = true;
    for (uint32_t it = 0; (int)(v & 63u) < NGU; ++it) {
      if (it >= ls.spin || ((it & 255u) == 255u && ld_coherent(ls.words) != 0ull)) {
        atomicOr(ls.status, kStatusLayerWait);
        st_coherent(ls.words, (uint64_t)1);
        ok = false;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
      v = ld_coherent(ctr);
    }
    if (ok && (int)((v >> (6 * (1 + xcc_id()))) & 63u) != NGU) atomicOr(ls.status, kStatusLayerXcd);
    *flag = ok;
  }
  __syncthreads();
  return *flag != 0;
}

// Gate/up workgroup of mfma_layer: once this item's h and exponents are
// stored (every wavefront's stores complete, so they are in the XCD's L2),
// count it on its tile.
__device__ __forceinline__ void layer_publish(const LayerSync& ls, int tile) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0)
    __hip_atomic_fetch_add(ls.words + 1 + tile, 1ull + (1ull << (6 * (1 + xcc_id()))),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One work item of a grouped pass: workgroup bid's row tile and column
// block (pass_tile_of). ls.words non-null: the one-launch layer (a down
// item first waits for its tile's gate/up items; a gate/up item publishes).
template <bool GU, int H, int I>
__device__ __forceinline__ void pass_item(int bid, const uint16_t* __restrict__ act, MfmaBank bk,
                                          const int32_t* __restrict__ meta,
                                          const int32_t* __restrict__ tiles,
                                          const int32_t* __restrict__ offsets,
                                          const int32_t* __restrict__ rtok,
                                          const int32_t* __restrict__ pair, int E, PassIO io,
                                          PassLds L, LayerSync ls) {
  using P = PassShape<GU, H, I>;
  static_assert(P::K % kBK == 0 && P::NOUT % P::COLS == 0, "MFMA tiling");
  constexpr int NKB = P::K / kBK;  // scale blocks along K
  constexpr int NCB = P::NOUT / P::COLS;
  constexpr int NGU = I / PassShape<true, H, I>::COLS;  // gate/up items per tile
  uint8_t *lds = L.lds, *ldsb = L.ldsb;
  int *arow = L.arow, *orow = L.orow, *herow = L.herow, *yq = L.yq;
  float* ss = L.ss;
  uint32_t* hfac = L.hfac;
  int j;
  const int tile = pass_tile_of<NCB>(meta, bid, j);
  if (tile < 0) return;
  if (!GU && ls.words && !layer_wait<NGU>(ls, tile, L.go)) return;
  const int g = tiles[2 * tile], r0 = tiles[2 * tile + 1];
  const int valid = min(kMfmaBM, offsets[g + 1] - r0);
  const int tid = threadIdx.x;
  const int n0 = (j % NCB) * P::COLS;
  const bool sh = g == E;
  if (bk.slot && bk.slot[g] < 0) return;  // a streamed expert outside this round
  const int gs = bk.slot && !sh ? bk.slot[g] : g;
  const uint8_t* W;
  const float* Sc;
  if (GU) {
    W = sh ? bk.sh_wgu : bk.wgu + (size_t)gs * 2 * I * H;
    Sc = sh ? bk.sh_sgu : bk.sgu + (size_t)gs * (2 * I / kBK) * (H / kBK);
  } else {
    W = sh ? bk.sh_wd : bk.wd + (size_t)gs * H * I;
    Sc = sh ? bk.sh_sd : bk.sd + (size_t)gs * (H / kBK) * (I / kBK);
  }
  // Everything the tile needs before its first stage, loaded in one round
  // (no load below depends on another):
  // source row of each tile row (GU: the token; down: the h row)
  if (tid < kMfmaBM) {
    const int rr = tid < valid ? tid : valid - 1;
    arow[tid] = GU ? rtok[r0 + rr] : r0 + rr;
    if (!GU) {
      // y is stored by slot (row r's output goes to y row pair[r]), so the
      // combine reads a token's outputs without the inverse permutation
      orow[tid] = pair[r0 + rr];
      // the h row's common power of two: the largest of its block
      // exponents; its blocks are brought to it by rescale words (exact
      // unless a block lies more than 2^14 below the row's largest block)
      // (one launch: read past this CU's L1, which may hold a line of them
      // from a neighbouring tile's rows, fetched before this tile's gate/up
      // items had written theirs)
      const uint8_t* eb = io.hexps + (size_t)(r0 + rr) * NKB;
      int b[NKB], emax = 0;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        b[kb] = ls.words ? ld_coherent(eb + kb) : eb[kb];
        emax = max(emax, b[kb]);
      }
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) hfac[tid * NKB + kb] = rescale_word(b[kb] - emax);
      herow[tid] = emax - kF16ExpBias;
    }
  }
  // scale rows of the tile's weight rows: GU: the gate block of rows n0 ..
  // n0 + 127 and the matching up block; down: rows n0 .. and n0 + 128 ..
  if (tid >= 256 && tid < 256 + 2 * NKB) {
    const int i = (tid - 256) / NKB, kb = (tid - 256) % NKB;
    const int wrow = GU ? (i == 0 ? n0 : I + n0) : n0 + 128 * i;
    ss[i * NKB + kb] = Sc[(size_t)(wrow / kBK) * NKB + kb];
  }
  // down: the output column blocks' bound exponents (|h'| <= 2^15 and
  // |code| <= 448: 2^q > 448 * 128 * S(b), the 2^15 of h' cancelling)
  if (!GU && tid >= 320 && tid < 322)
    yq[tid - 320] = y_block_q(Sc + (size_t)((n0 + 128 * (tid - 320)) / kBK) * NKB, NKB,
                              448.f * 128.f);
  __syncthreads();
  if (tid < 2) drop_far_blocks(ss + tid * NKB, NKB);
  __syncthreads();
  if (valid <= 64)
    pass_tile<GU, H, I, true>(act, W, ss, arow, orow, hfac, herow, yq, valid, r0, n0, lds, ldsb,
                              io);
  else if constexpr (GU)
    pass_tile_gu_dma<H, I>(act, W, ss, arow, valid, r0, n0, lds, ldsb, io);
  else
    pass_tile_down_dma<H, I>(act, W, ss, arow, orow, hfac, herow, yq, valid, r0, n0, lds, ldsb,
                             io);
  if (GU && ls.words) layer_publish(ls, tile);
}

// A grouped pass on its own (the FP8-free two-launch form, which a streamed
// bank takes: its rounds run the passes once per round)
template <bool GU, int H, int I>
__global__ __launch_bounds__(kPassThreads) __attribute__((amdgpu_waves_per_eu(4)))
void mfma_pass(const uint16_t* __restrict__ act, MfmaBank bk, const int32_t* __restrict__ meta,
               const int32_t* __restrict__ tiles, const int32_t* __restrict__ offsets,
               const int32_t* __restrict__ rtok, const int32_t* __restrict__ pair, int E,
               PassIO io) {
  constexpr int NKB = PassShape<GU, H, I>::K / kBK;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes / 2];
  __shared__ __attribute__((aligned(16))) uint8_t ldsb[kLdsBytes / 2];
  __shared__ int arow[kMfmaBM];
  __shared__ int orow[GU ? 1 : kMfmaBM];
  __shared__ float ss[2 * NKB];
  __shared__ uint32_t hfac[GU ? 1 : kMfmaBM * NKB];
  __shared__ int herow[GU ? 1 : kMfmaBM];
  __shared__ int yq[2];
  pass_item<GU, H, I>(blockIdx.x, act, bk, meta, tiles, offsets, rtok, pair, E, io,
                      PassLds{lds, ldsb, arow, orow, ss, hfac, herow, yq, nullptr},
                      LayerSync{nullptr, nullptr, 0u});
}

// Both grouped passes in one launch: workgroups 0 .. n_gu - 1 are gate/up
// items, the rest down items in the same tile order, so a tile's items of
// both passes land on one XCD (bid % 8). Workgroups are dispatched in order
// on each XCD, so a waiting down item never holds back a gate/up item it
// waits for: every gate/up item of its XCD has been dispatched before it,
// and a gate/up item never waits. The down items of a tile start while
// other tiles' gate/up items still run (no drain between the passes).
template <int H, int I>
__global__ __launch_bounds__(kPassThreads) __attribute__((amdgpu_waves_per_eu(4)))
void mfma_layer(const uint16_t* __restrict__ x, const uint16_t* __restrict__ h, MfmaBank bk,
                const int32_t* __restrict__ meta, const int32_t* __restrict__ tiles,
                const int32_t* __restrict__ offsets, const int32_t* __restrict__ rtok,
                const int32_t* __restrict__ pair, int E, PassIO hio, PassIO yio, int n_gu,
                LayerSync ls) {
  constexpr int NKG = H / kBK, NKD = I / kBK;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes / 2];
  __shared__ __attribute__((aligned(16))) uint8_t ldsb[kLdsBytes / 2];
  __shared__ int arow[kMfmaBM];
  __shared__ int orow[kMfmaBM];
  __shared__ float ss[2 * (NKG > NKD ? NKG : NKD)];
  __shared__ uint32_t hfac[kMfmaBM * NKD];
  __shared__ int herow[kMfmaBM];
  __shared__ int yq[2];
  __shared__ int go;
  const PassLds L{lds, ldsb, arow, orow, ss, hfac, herow, yq, &go};
  const int b = blockIdx.x;
  if (b < n_gu)
    pass_item<true, H, I>(b, x, bk, meta, tiles, offsets, rtok, pair, E, hio, L, ls);
  else
    pass_item<false, H, I>(b - n_gu, h, bk, meta, tiles, offsets, rtok, pair, E, yio, L, ls);
}

// ---------------------------------------------------------------------------
// FP8 passes: the variant that runs both expert contractions with E4M3 on
// both sides, on v_mfma_scale_f32_32x32x64_f8f6f4. gate/up reads the
// activations quantised by moe_quantize_act_e4m3 (one power-of-two scale per
// token and 128 columns); its epilogue quantises h the same way (a tile's
// 128 h columns are one block) into E4M3 codes and exponents, which the down
// pass reads.
//   Lane l supplies A row l % 32 and B column (weight row) l % 32, each as the
//   32 bytes of K of its lane half (bytes 32 (l / 32) .. + 31 of the 64-k
//   step: two 16-byte LDS chunks). A and B take K in the same order, so the
//   contraction does not depend on the order in which the instruction walks K.
//   The A scale rides in the instruction: lane l's E8M0 byte scales A row
//   l % 32 over its 32 K, all inside one 128-column block, so every lane of a
//   row passes that block's exponent; B's scale byte is 127 (1). The weights'
//   fp32 block scales are applied in the ratio form of the bf16 passes.
// Tiles as in the bf16 passes with half the A bytes: full tiles (more than 64
// rows) take 64-k stages through two LDS buffers (A 8 KiB, B 16 KiB), one
// stage fetched ahead; thin tiles take 128-k stages (one scale block) through
// one 40 KiB buffer, two stages in flight in registers. A and B rows are both
// KS bytes of E4M3 and share one swizzle (chunk c of row r at slot
// c ^ ((r >> 2) & 3) for 64-k stages, c ^ ((r >> 1) & 7) for 128-k stages).
template <bool GU, bool THIN>
struct F8Shape {
  static constexpr int RA = THIN ? 64 : 128;          // A rows per stage
  static constexpr int KS = THIN ? 128 : 64;          // k per stage
  static constexpr int CH = KS / 16;                  // 16-byte chunks per A or B row
  static constexpr int AC = RA * CH / kPassThreads;   // A chunks per thread per stage
  static constexpr int BC = kTN * CH / kPassThreads;  // B chunks per thread per stage
  static constexpr int ASTAGE = RA * KS;
  static constexpr int BSTAGE = kTN * KS;
  static constexpr int BUFS = THIN ? 1 : 2;
  static constexpr int MW = THIN ? 1 : 2;             // 32-row MFMA tiles per wavefront
  static constexpr int NBW = 2;                       // 32-column MFMA tiles per wavefront
  static constexpr int DEPTH = THIN ? 2 : 1;
  static_assert(BUFS * (ASTAGE + BSTAGE) <= kLdsBytes, "stage buffers exceed the LDS block");
  static_assert(AC * kPassThreads == RA * CH && BC * kPassThreads == kTN * CH, "fetch map");
  static __device__ __forceinline__ int arow0(int wm) { return (THIN ? 32 : 64) * wm; }
  // gate/up: gate rows 32 wn .., then the matching up rows; down: 64 wn + 32 nb
  static __device__ __forceinline__ int brow(int wn, int nb) {
    if (GU) return nb == 0 ? 32 * wn : kTN / 2 + 32 * wn;
    return 64 * wn + 32 * nb;
  }
  static __device__ __forceinline__ int swz(int r) { return CH == 8 ? ((r >> 1) & 7) : ((r >> 2) & 3); }
};

typedef int i32x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ i32x8_t f8_operand(const uint8_t* row, int c0, int c1) {
  const uint4 a = *reinterpret_cast<const uint4*>(row + 16 * c0);
  const uint4 b = *reinterpret_cast<const uint4*>(row + 16 * c1);
  i32x8_t v;
  v[0] = (int)a.x; v[1] = (int)a.y; v[2] = (int)a.z; v[3] = (int)a.w;
  v[4] = (int)b.x; v[5] = (int)b.y; v[6] = (int)b.z; v[7] = (int)b.w;
  return v;
}

// Outputs of an FP8 pass: gate/up writes h as E4M3 codes [P][I] and E8M0
// exponents [P][I/128]; down writes y (fp16, by slot).
struct F8Out {
  uint8_t* hcodes;
  uint8_t* hexps;
  uint16_t* y;
  uint8_t* yexps;
};

template <bool GU, int H, int I, bool THIN>
__device__ __forceinline__ void pass_tile_f8(const uint8_t* __restrict__ act, const uint8_t* W,
                                             const float* ss, const uint8_t* sx, const int* arow,
                                             const int* orow, const int* rowg, const int* yq,
                                             int valid, int r0, int n0, uint8_t* lds, F8Out out) {
  using S = F8Shape<GU, THIN>;
  constexpr int K = GU ? H : I, KS = S::KS, NS = K / KS, AC = S::AC, BC = S::BC, MW = S::MW,
                NBW = S::NBW, CH = S::CH;
  constexpr int NKB = K / kBK;
  static_assert(K % KS == 0 && kBK % KS == 0, "stages must tile the scale blocks");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches only
  const int wm = wave >> 2, wn = wave & 3;

  // fetch map: chunk qq = tid + 512 i is row qq / CH, chunk qq % CH (A and B
  // alike); moving qq by 512 moves the row by a multiple of 32, which leaves
  // the swizzle alone (gate/up: tile rows 128 .. 255 are the up rows I + n0 ..)
  const __amdgpu_buffer_rsrc_t arsrc = buffer_rsrc(act, 0xffffffffu);
  const __amdgpu_buffer_rsrc_t brsrc = buffer_rsrc(W, (uint32_t)((GU ? 2 * I : H) * K));
  constexpr int RS = kPassThreads / CH;  // row step per chunk group
  const int rt = tid / CH, ct = tid % CH;
  const int dst0 = rt * KS + 16 * (ct ^ S::swz(rt));
  uint32_t asrc[AC];
#pragma unroll
  for (int i = 0; i < AC; ++i) asrc[i] = (uint32_t)arow[rt + RS * i] * K + 16 * ct;
  const uint32_t bsrc0 = (uint32_t)(n0 + rt) * K + 16 * ct;
  auto brow_of = [](int i) -> int {
    const int tr = RS * i;
    return GU ? (tr < kTN / 2 ? tr : I + tr - kTN / 2) : tr;
  };
  struct Regs {
    uint4 a[AC], b[BC];
  };
  const float* bscale[BC];
#pragma unroll
  for (int i = 0; i < BC; ++i) bscale[i] = ss + (RS * i / kBK) * NKB;
  auto fetch = [&](Regs& R, int st) {
    st = st < NS ? st : NS - 1;  // past the end: a harmless repeat, never stored
#pragma unroll
    for (int i = 0; i < AC; ++i) R.a[i] = buffer_ld16(arsrc, asrc[i], (uint32_t)(st * KS));
#pragma unroll
    for (int i = 0; i < BC; ++i)
      R.b[i] = buffer_ld16<THIN ? kBufNonTemporal : 0>(brsrc, bsrc0,
                                                       (uint32_t)(brow_of(i) * K + st * KS));
  };
  auto put = [&](Regs& R, int buf, int st) {
    uint8_t* A = lds + buf * (S::ASTAGE + S::BSTAGE);
    uint8_t* B = A + S::ASTAGE;
    const int kb = st * KS / kBK;
    bool zero = false;
#pragma unroll
    for (int i = 0; i < BC; ++i) zero |= bscale[i][kb] == 0.f;
    if (zero) {  // rare: a zero block scale (uniform branch)
#pragma unroll
      for (int i = 0; i < BC; ++i)
        if (bscale[i][kb] == 0.f) R.b[i] = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < AC; ++i) *reinterpret_cast<uint4*>(A + dst0 + RS * KS * i) = R.a[i];
#pragma unroll
    for (int i = 0; i < BC; ++i) *reinterpret_cast<uint4*>(B + dst0 + RS * KS * i) = R.b[i];
  };

  // fragments: A rows arow0 + 32 m + lane % 32, B rows brow(nb) + lane % 32;
  // the row offsets are multiples of 32, so the swizzle depends on lane % 32
  const int q = lane >> 5, l32 = lane & 31;
  const int sw = S::swz(l32);
  const int afr = (S::arow0(wm) + l32) * KS, bfr = l32 * KS;
  const float* srow[NBW];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) srow[nb] = ss + (S::brow(wn, nb) / kBK) * NKB;
  const uint8_t* sxr[MW];  // this lane's rows' A exponents
#pragma unroll
  for (int m = 0; m < MW; ++m) sxr[m] = sx + (S::arow0(wm) + 32 * m + l32) * NKB;

  f32x16_t acc[MW][NBW];
#pragma unroll
  for (int m = 0; m < MW; ++m)
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[m][nb][v] = 0.f;
  float unit[NBW], snext[NBW];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) {
    unit[nb] = 0.f;
    snext[nb] = srow[nb][0];
  }
  const bool idle = S::arow0(wm) >= valid;
  auto compute = [&](int buf, int st) {
    if (idle) return;
    const int kb = st * KS / kBK;
    if ((st * KS) % kBK == 0) {  // entering weight scale block kb (ratio form)
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) {
        const float sn = snext[nb];
        if (kb + 1 < NKB) snext[nb] = srow[nb][kb + 1];
        const bool on = sn != 0.f;
        const float r = on ? scale_ratio(unit[nb], sn) : 1.f;
#pragma unroll
        for (int m = 0; m < MW; ++m)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[m][nb][v] *= r;
        unit[nb] = on ? sn : unit[nb];
      }
    }
    int sc[MW];
#pragma unroll
    for (int m = 0; m < MW; ++m) sc[m] = sxr[m][kb];
    const uint8_t* A = lds + buf * (S::ASTAGE + S::BSTAGE);
    const uint8_t* B = A + S::ASTAGE;
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int p = 0; p < KS / 64; ++p) {
      const int c0 = (4 * p + 2 * q) ^ sw, c1 = (4 * p + 2 * q + 1) ^ sw;
      // A fragments first, then one B fragment at a time: fewer live registers
      i32x8_t af[MW];
#pragma unroll
      for (int m = 0; m < MW; ++m) af[m] = f8_operand(A + afr + 32 * m * KS, c0, c1);
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) {
        const i32x8_t bf = f8_operand(B + S::brow(wn, nb) * KS + bfr, c0, c1);
#pragma unroll
        for (int m = 0; m < MW; ++m)
          acc[m][nb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[m], bf, acc[m][nb], 0, 0,
                                                                      0, sc[m], 0, 127);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };

  if (S::DEPTH == 1) {
    static_assert(NS % 2 == 0, "stages come in pairs");
    Regs R;
    fetch(R, 0);
    put(R, 0, 0);
    __syncthreads();
#pragma unroll 1
    for (int st = 0; st < NS; st += 2) {
      fetch(R, st + 1);
      compute(0, st);
      put(R, 1, st + 1);
      __syncthreads();
      fetch(R, st + 2);
      compute(1, st + 1);
      if (st + 2 < NS) put(R, 0, st + 2);
      __syncthreads();
    }
  } else {
    constexpr int D = S::DEPTH;
    static_assert(NS % D == 0, "stage count must be a multiple of the prefetch depth");
    Regs R[D];
#pragma unroll
    for (int j = 0; j < D; ++j) {  // in stage order, as the loop issues them
      fetch(R[j], j);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll 1  // a fully unrolled ring spills at 128 registers
    for (int st0 = 0; st0 < NS; st0 += D) {
#pragma unroll
      for (int j = 0; j < D; ++j) {
        const int st = st0 + j;
        put(R[j], 0, st);     // the previous stage's reads ended at the last barrier
        fetch(R[j], st + D);  // set j is free once written
        __syncthreads();
        compute(0, st);
        __syncthreads();
      }
    }
  }

  // D layout (32x32): lane L holds column L % 32; value v is row
  // 8 (v / 4) + 4 (L / 32) + v % 4
  if (GU) {
    // h through LDS as fp32 (512 bytes per tile row; 16-byte chunk c of row r
    // at slot c ^ (((r >> 2) & 1) << 3), so the two row groups of one write
    // use different banks), then quantised per row of the tile's 128 columns
    // (one scale block): 16 lanes (a DPP row) per tile row, 8 values each
    constexpr int HRB = 128 * 4;
    static_assert(S::RA * HRB <= kLdsBytes, "h tile exceeds the LDS block");
    auto hswz = [](int r) { return ((r >> 2) & 1) << 3; };
    if (!idle) {
#pragma unroll
      for (int m = 0; m < MW; ++m)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = S::arow0(wm) + 32 * m + 8 * (v >> 2) + 4 * q + (v & 3);
          const int col = S::brow(wn, 0) + l32;
          *reinterpret_cast<float*>(lds + row * HRB + 16 * ((col >> 2) ^ hswz(row)) +
                                    4 * (col & 3)) =
              silu(acc[m][0][v] * unit[0]) * (acc[m][1][v] * unit[1]);
        }
    }
    __syncthreads();
    static_assert((S::RA * 16) % kPassThreads == 0, "h rows per thread");
#pragma unroll
    for (int i = 0; i < S::RA * 16 / kPassThreads; ++i) {
      const int idx = tid + kPassThreads * i, r = idx >> 4, k = idx & 15;
      const uint4 a = *reinterpret_cast<const uint4*>(lds + r * HRB + 16 * ((2 * k) ^ hswz(r)));
      const uint4 b = *reinterpret_cast<const uint4*>(lds + r * HRB + 16 * ((2 * k + 1) ^ hswz(r)));
      const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
      uint32_t mx = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) mx = max(mx, w[j] & 0x7fffffffu);
      const int e = act_exponent(__uint_as_float(row16_max_u32(mx)));
      uint32_t c[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) c[j] = e4m3_rne(__builtin_ldexpf(__uint_as_float(w[j]), -e));
      if (r >= valid) continue;
      *reinterpret_cast<uint2*>(out.hcodes + (size_t)(r0 + r) * I + n0 + 8 * k) =
          make_uint2(c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24),
                     c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24));
      if (k == 0) out.hexps[(size_t)(r0 + r) * (I / kBK) + n0 / kBK] = (uint8_t)(e + 127);
    }
  } else {
    // y as scaled fp16 by slot (acc is y itself: the h exponents ride in the
    // instruction), as in the bf16 down pass
    static_assert(S::RA * 512 <= kLdsBytes, "output tile exceeds the LDS block");
    store_y_tile<S::RA, MW, H, false>(acc, unit, rowg, yq, S::arow0(wm), wn, idle, valid, n0,
                                      orow, wave, [&](int r) { return lds + r * 512; }, out.y,
                                      out.yexps);
  }
}

// LDS of an FP8 pass workgroup: lds, the stage buffers and output tile;
// arow: source row of each tile row; orow (down): the y row (slot) of each
// tile row; ss: the tile's two weight scale rows; sx: the tile rows' A
// exponents; rowg (down): each row's largest h exponent; yq (down): the
// output column blocks' bound exponents; go: a one-launch down item's wait
// outcome.
struct PassLdsF8 {
  uint8_t* lds;
  int* arow;
  int* orow;
  float* ss;
  uint8_t* sx;
  int* rowg;
  int* yq;
  int* go;
};

// One work item of an FP8 pass (as pass_item: ls.words non-null in the
// one-launch layer, mfma_layer_f8).
template <bool GU, int H, int I>
__device__ __forceinline__ void pass_item_f8(int bid, const uint8_t* __restrict__ codes,
                                             const uint8_t* __restrict__ exps, MfmaBank bk,
                                             const int32_t* __restrict__ meta,
                                             const int32_t* __restrict__ tiles,
                                             const int32_t* __restrict__ offsets,
                                             const int32_t* __restrict__ rtok,
                                             const int32_t* __restrict__ pair, int E, F8Out out,
                                             PassLdsF8 L, LayerSync ls) {
  constexpr int K = GU ? H : I, NKB = K / kBK;
  constexpr int COLS = GU ? 128 : 256, NCB = (GU ? I : H) / COLS;
  constexpr int NGU = I / 128;  // gate/up items per tile
  uint8_t* lds = L.lds;
  uint8_t* sx = L.sx;
  int *arow = L.arow, *orow = L.orow, *rowg = L.rowg, *yq = L.yq;
  float* ss = L.ss;
  int j;  // XCD-aware, as mfma_pass
  const int tile = pass_tile_of<NCB>(meta, bid, j);
  if (tile < 0) return;
  if (!GU && ls.words && !layer_wait<NGU>(ls, tile, L.go)) return;
  const int g = tiles[2 * tile], r0 = tiles[2 * tile + 1];
  const int valid = min(kMfmaBM, offsets[g + 1] - r0);
  const int tid = threadIdx.x;
  const int n0 = (j % NCB) * COLS;
  const bool sh = g == E;
  if (bk.slot && bk.slot[g] < 0) return;  // a streamed expert outside this round
  const int gs = bk.slot && !sh ? bk.slot[g] : g;
  const uint8_t* W;
  const float* Sc;
  if (GU) {
    W = sh ? bk.sh_wgu : bk.wgu + (size_t)gs * 2 * I * H;
    Sc = sh ? bk.sh_sgu : bk.sgu + (size_t)gs * (2 * I / kBK) * (H / kBK);
  } else {
    W = sh ? bk.sh_wd : bk.wd + (size_t)gs * H * I;
    Sc = sh ? bk.sh_sd : bk.sd + (size_t)gs * (H / kBK) * (I / kBK);
  }
  // source row of each tile row (gate/up: the token; down: the h row); the
  // down pass also takes its rows' h exponents in the same round of loads
  if (tid < kMfmaBM) {
    const int rr = tid < valid ? tid : valid - 1;
    arow[tid] = GU ? rtok[r0 + rr] : r0 + rr;
    if (!GU) {
      orow[tid] = pair[r0 + rr];
      int emax = 0;
      for (int kb = 0; kb < NKB; ++kb) {
        // (one launch: past this CU's L1, as the bf16 down items read them)
        const uint8_t* ep = exps + (size_t)(r0 + rr) * NKB + kb;
        const int b = ls.words ? ld_coherent(ep) : *ep;
        sx[tid * NKB + kb] = (uint8_t)b;
        emax = max(emax, b);
      }
      rowg[tid] = emax - 127;
    }
  }
  // weight scale rows: gate/up: the gate block of rows n0 .. n0 + 127 and the
  // matching up block; down: rows n0 .. + 127, then n0 + 128 .. + 255
  if (tid >= 256 && tid < 256 + 2 * NKB) {
    const int i = (tid - 256) / NKB, kb = (tid - 256) % NKB;
    const int wrow = GU ? (i == 0 ? n0 : I + n0) : n0 + 128 * i;
    ss[i * NKB + kb] = Sc[(size_t)(wrow / kBK) * NKB + kb];
  }
  // down: |h| <= 448 * 2^g and |code| <= 448: 2^(q + 15) > 448 * 448 * 128 * S(b)
  if (!GU && tid >= 320 && tid < 322)
    yq[tid - 320] = y_block_q(Sc + (size_t)((n0 + 128 * (tid - 320)) / kBK) * NKB, NKB,
                              448.f * 448.f * 128.f) - 15;
  __syncthreads();
  if (tid < 2) drop_far_blocks(ss + tid * NKB, NKB);
  __syncthreads();
  if (GU) {  // gate/up: the activation exponents of each row's token
    for (int i = tid; i < kMfmaBM * NKB; i += kPassThreads)
      sx[i] = exps[(size_t)arow[i / NKB] * NKB + i % NKB];
    __syncthreads();
  }
  if (valid <= 64)
    pass_tile_f8<GU, H, I, true>(codes, W, ss, sx, arow, orow, rowg, yq, valid, r0, n0, lds, out);
  else
    pass_tile_f8<GU, H, I, false>(codes, W, ss, sx, arow, orow, rowg, yq, valid, r0, n0, lds, out);
  if (GU && ls.words) layer_publish(ls, tile);
}

// An FP8 pass on its own (a streamed bank's rounds)
template <bool GU, int H, int I>
__global__ __launch_bounds__(kPassThreads) __attribute__((amdgpu_waves_per_eu(4)))
void mfma_pass_f8(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ exps,
                  MfmaBank bk, const int32_t* __restrict__ meta,
                  const int32_t* __restrict__ tiles, const int32_t* __restrict__ offsets,
                  const int32_t* __restrict__ rtok, const int32_t* __restrict__ pair, int E,
                  F8Out out) {
  constexpr int NKB = (GU ? H : I) / kBK;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];
  __shared__ int arow[kMfmaBM];
  __shared__ int orow[GU ? 1 : kMfmaBM];
  __shared__ float ss[2 * NKB];
  __shared__ uint8_t sx[kMfmaBM * NKB];
  __shared__ int rowg[GU ? 1 : kMfmaBM];
  __shared__ int yq[2];
  pass_item_f8<GU, H, I>(blockIdx.x, codes, exps, bk, meta, tiles, offsets, rtok, pair, E, out,
                         PassLdsF8{lds, arow, orow, ss, sx, rowg, yq, nullptr},
                         LayerSync{nullptr, nullptr, 0u});
}

// Both FP8 passes in one launch, as mfma_layer: gate/up items (workgroups
// 0 .. n_gu - 1) publish per tile after their h codes and exponents are
// stored; down items wait for their tile's.
template <int H, int I>
__global__ __launch_bounds__(kPassThreads) __attribute__((amdgpu_waves_per_eu(4)))
void mfma_layer_f8(const uint8_t* __restrict__ acodes, const uint8_t* __restrict__ aexps,
                   const uint8_t* __restrict__ hcodes, const uint8_t* __restrict__ hexps,
                   MfmaBank bk, const int32_t* __restrict__ meta,
                   const int32_t* __restrict__ tiles, const int32_t* __restrict__ offsets,
                   const int32_t* __restrict__ rtok, const int32_t* __restrict__ pair, int E,
                   F8Out hout, F8Out yout, int n_gu, LayerSync ls) {
  constexpr int NKG = H / kBK, NKD = I / kBK, NKM = NKG > NKD ? NKG : NKD;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];
  __shared__ int arow[kMfmaBM];
  __shared__ int orow[kMfmaBM];
  __shared__ float ss[2 * NKM];
  __shared__ uint8_t sx[kMfmaBM * NKM];
  __shared__ int rowg[kMfmaBM];
  __shared__ int yq[2];
  __shared__ int go;
  const PassLdsF8 L{lds, arow, orow, ss, sx, rowg, yq, &go};
  const int b = blockIdx.x;
  if (b < n_gu)
    pass_item_f8<true, H, I>(b, acodes, aexps, bk, meta, tiles, offsets, rtok, pair, E, hout, L,
                             ls);
  else
    pass_item_f8<false, H, I>(b - n_gu, hcodes, hexps, bk, meta, tiles, offsets, rtok, pair, E,
                              yout, L, ls);
}

// ---------------------------------------------------------------------------
template <int H, int I, int B>
static void run_mfma(const Dims& d, const void* x, const MfmaBank& bk, const Work& w,
                     hipStream_t s, KernelEvents ev) {
  static_assert(B == kBK, "MFMA passes take 128 x 128 scale blocks");
  // tile slots: every XCD gets the longest chunk it can be dealt (long tile
  // lists) or its round-robin share; slots without a tile exit
  const int64_t mt = max_mfma_tiles(d);
  const unsigned nt8 =
      (unsigned)(kXcds * (mt >= kChunkTiles ? mfma_chunk_tiles(d) : (mt + kXcds - 1) / kXcds));
  const dim3 grid(nt8 * (I / PassShape<true, H, I>::COLS));
  const uint16_t* xa = reinterpret_cast<const uint16_t*>(x);
  const int32_t *meta = w.meta, *tiles = w.tiles, *offsets = w.offsets, *rtok = w.rtok,
                *pair = w.pair;
  if (d.f8) {  // both contractions on E4M3 operands; h goes between them as E4M3
    const F8Out hout{static_cast<uint8_t*>(w.h), w.hexps, nullptr, nullptr};
    const F8Out yout{nullptr, nullptr, static_cast<uint16_t*>(w.y), w.yexps};
    if (!bk.slot) {  // one launch, as the bf16 passes
      const LayerSync ls{static_cast<uint64_t*>(w.sync), w.status, layer_wait_limit(kLayerSpin)};
      const int n_gu = (int)grid.x;
      const dim3 g2(grid.x + nt8 * (H / PassShape<false, H, I>::COLS));
      const uint8_t* hc = static_cast<const uint8_t*>(w.h);
      if (ev.any())
        hipExtLaunchKernelGGL(mfma_layer_f8<H, I>, g2, dim3(kPassThreads), 0, s, ev.begin, ev.end,
                              0, w.acodes, w.aexps, hc, w.hexps, bk, meta, tiles, offsets, rtok,
                              pair, d.E, hout, yout, n_gu, ls);
      else
        mfma_layer_f8<H, I><<<g2, kPassThreads, 0, s>>>(w.acodes, w.aexps, hc, w.hexps, bk, meta,
                                                        tiles, offsets, rtok, pair, d.E, hout,
                                                        yout, n_gu, ls);
      return;
    }
    if (ev.any())
      hipExtLaunchKernelGGL(mfma_pass_f8<true, H, I>, grid, dim3(kPassThreads), 0, s, ev.begin,
                            ev.end, 0, w.acodes, w.aexps, bk, meta, tiles, offsets, rtok, pair,
                            d.E, hout);
    else
      mfma_pass_f8<true, H, I><<<grid, kPassThreads, 0, s>>>(w.acodes, w.aexps, bk, meta, tiles,
                                                             offsets, rtok, pair, d.E, hout);
    mfma_pass_f8<false, H, I><<<nt8 * (H / PassShape<false, H, I>::COLS), kPassThreads, 0, s>>>(
        static_cast<const uint8_t*>(w.h), w.hexps, bk, meta, tiles, offsets, rtok, pair, d.E,
        yout);
    return;
  }
  const PassIO hio{w.h, w.hexps, nullptr};
  const PassIO yio{w.y, w.yexps, w.hexps};
  const uint16_t* hin = reinterpret_cast<const uint16_t*>(w.h);
  const unsigned n_down = nt8 * (H / PassShape<false, H, I>::COLS);
  if (!bk.slot) {  // one launch; the permutation cleared its counters and status
    const LayerSync ls{static_cast<uint64_t*>(w.sync), w.status, layer_wait_limit(kLayerSpin)};
    const int n_gu = (int)grid.x;
    const dim3 g2(grid.x + n_down);
    if (ev.any())
      hipExtLaunchKernelGGL(mfma_layer<H, I>, g2, dim3(kPassThreads), 0, s, ev.begin, ev.end, 0,
                            xa, hin, bk, meta, tiles, offsets, rtok, pair, d.E, hio, yio, n_gu,
                            ls);
    else
      mfma_layer<H, I><<<g2, kPassThreads, 0, s>>>(xa, hin, bk, meta, tiles, offsets, rtok, pair,
                                                   d.E, hio, yio, n_gu, ls);
    return;
  }
  if (ev.any()) {  // the events take the kernel's own start and end times
    hipExtLaunchKernelGGL(mfma_pass<true, H, I>, grid, dim3(kPassThreads), 0, s, ev.begin, ev.end,
                          0, xa, bk, meta, tiles, offsets, rtok, pair, d.E, hio);
  } else {
    mfma_pass<true, H, I><<<grid, kPassThreads, 0, s>>>(xa, bk, meta, tiles, offsets, rtok, pair,
                                                        d.E, hio);
  }
  mfma_pass<false, H, I><<<n_down, kPassThreads, 0, s>>>(hin, bk, meta, tiles, offsets, rtok,
                                                        pair, d.E, yio);
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
                               KernelEvents gate_up_events, const int32_t* slot) {
  MfmaBank bk{routed.w_gate_up, routed.w_down, routed.s_gate_up, routed.s_down,
              shared ? shared->w_gate_up : nullptr, shared ? shared->w_down : nullptr,
              shared ? shared->s_gate_up : nullptr, shared ? shared->s_down : nullptr, slot};
#define X(hh, ii, bb)                                    \
  if (d.H == hh && d.I == ii && d.B == bb) {             \
    run_mfma<hh, ii, bb>(d, x, bk, w, s, gate_up_events); \
    return hipGetLastError();                            \
  }
  MOE_MFMA_SHAPES(X)
#undef X
  return hipErrorInvalidValue;
}

}  // namespace moe
