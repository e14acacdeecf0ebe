// expert_mfma.hip — the expert passes for prefill-sized groups, as grouped
// bf16 MFMA GEMMs over block-FP8 weights.
//
// With tens to thousands of tokens per expert the passes are dense
// contractions, so they run on the matrix cores (v_mfma_f32_16x16x32_bf16).
// Following the colizig page ("Features": dequantisation fused into the dot
// products), E4M3 weights are converted in registers right after their
// 16-byte global load; every E4M3 value is a bf16 value, so the conversion
// (v_cvt_scalef32_pk_bf16_fp8 with a unit scale) is exact and the products
// are exact in fp32. A block's fp32 scale multiplies the partial sum of its
// 128 columns (one accumulator per scale block, folded into the running
// total), never single weights.
//
// Work list: the permutation emits one (group, first row) entry per tile of
// kMfmaBM = 64 rows of a group; blockIdx.y indexes it (entries past the count
// exit at once) and blockIdx.x picks a block of output columns.
//
//   gate/up: a workgroup owns 64 gate columns and the 64 matching up columns;
//            each of its 4 wavefronts owns 16 of each, so SwiGLU is applied to
//            accumulator registers directly. bf16 MFMA: activations are bf16
//            and the weights exact in bf16, so nothing is rounded on the way
//            in. h is written as fp16 [P][I] (11-bit significand; saturated
//            at +-65504).
//   down:    fp16 MFMA on h (weights are exact in fp16 as well); a workgroup
//            owns 128 output columns (32 per wavefront); y is written as fp32
//            [P][H].
// h is the one intermediate rounded below fp32. fp16 rather than bf16 keeps
// its relative error at 2^-11, which leaves the layer's output well inside
// its tolerance (max error <= 1e-2 x RMS); bf16 would use up most of it.
// The 64 x 128 activation tile of the current scale block is staged in LDS
// (rows padded by 16 bytes, so the 16 rows a wavefront reads in one step fall
// in different banks); each wavefront loads its weight rows directly.
//
// MFMA operand layout (16x16x32 bf16): lane L supplies row L%16 of A and
// column L%16 of B, each as 8 consecutive k of the 32 (k = 8*(L/16) .. +7).
// The contraction is the same for any permutation of k applied to A and B
// alike, so a lane loads 16 consecutive bytes of a weight row (k = 16*(L/16)
// .. +15 of a 64-wide span) and uses them for two MFMA steps; its A reads use
// the same k positions.
#include "device.hpp"
#include "layer.hpp"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

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
constexpr int kLda = kBK + 8;       // LDS row stride of the A tile, in bf16

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

__device__ __forceinline__ f16x8_t lds_f16x8(const uint16_t* p) {
  return __builtin_bit_cast(f16x8_t, *reinterpret_cast<const uint4*>(p));
}

__device__ __forceinline__ f32x4_t mfma16_f16(f16x8_t a, f16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8_t lds_bf16x8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(p));
}

__device__ __forceinline__ f32x4_t mfma16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Stage rows [0, 64) x k-columns [k0, k0 + 128) of the tile's activations into
// LDS; rows at or past `valid` are zero. src(row) gives the row's base.
template <typename RowPtr>
__device__ __forceinline__ void stage_a(uint16_t* As, RowPtr src, int valid, int k0) {
  const int tid = threadIdx.x;
  uint4 v[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = tid + 256 * j;        // 16-byte chunk: 64 rows x 16 chunks
    const int row = c >> 4, c16 = c & 15;
    v[j] = row < valid ? ld16(src(row) + k0 + 8 * c16) : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = tid + 256 * j;
    const int row = c >> 4, c16 = c & 15;
    *reinterpret_cast<uint4*>(As + row * kLda + 8 * c16) = v[j];
  }
}

template <int H, int I, int B>
__global__ __launch_bounds__(256) void mfma_gate_up(const uint16_t* __restrict__ x, MfmaBank bk,
                                                   const int32_t* __restrict__ meta,
                                                   const int32_t* __restrict__ tiles,
                                                   const int32_t* __restrict__ offsets,
                                                   const int32_t* __restrict__ rtok, int E,
                                                   uint16_t* __restrict__ h) {
  static_assert(B == kBK && H % kBK == 0 && I % 64 == 0, "MFMA tiling");
  __shared__ uint16_t As[kMfmaBM * kLda];
  __shared__ int toks[kMfmaBM];
  const int tile = blockIdx.y;
  if (tile >= meta[1]) return;
  const int g = tiles[2 * tile], r0 = tiles[2 * tile + 1];
  const int valid = min(kMfmaBM, offsets[g + 1] - r0);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n0 = blockIdx.x * 64 + wave * 16;  // this wavefront's 16 gate columns
  const bool sh = g == E;
  const uint8_t* W = sh ? bk.sh_wgu : bk.wgu + (size_t)g * 2 * I * H;
  const float* Sc = sh ? bk.sh_sgu : bk.sgu + (size_t)g * (2 * I / B) * (H / B);
  if (threadIdx.x < kMfmaBM) toks[threadIdx.x] = threadIdx.x < valid ? rtok[r0 + threadIdx.x] : 0;
  __syncthreads();

  const uint8_t* wg_row = W + (size_t)(n0 + (lane & 15)) * H + 16 * (lane >> 4);
  const uint8_t* wu_row = W + (size_t)(I + n0 + (lane & 15)) * H + 16 * (lane >> 4);
  const float* sg_row = Sc + (size_t)(n0 / B) * (H / B);
  const float* su_row = Sc + (size_t)((I + n0) / B) * (H / B);
  auto xrow = [&](int row) { return x + (size_t)toks[row] * H; };

  f32x4_t accg[4], accu[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) accg[m] = accu[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int kb = 0; kb < H / kBK; ++kb) {
    const int k0 = kb * kBK;
    uint4 wgv[2], wuv[2];
#pragma unroll
    for (int sp = 0; sp < 2; ++sp) {
      wgv[sp] = ld16(wg_row + k0 + 64 * sp);
      wuv[sp] = ld16(wu_row + k0 + 64 * sp);
    }
    const float sg = sg_row[kb], su = su_row[kb];
    __syncthreads();  // the previous block's LDS reads are done
    stage_a(As, xrow, valid, k0);
    __syncthreads();

    f32x4_t bg[4], bu[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) bg[m] = bu[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int sp = 0; sp < 2; ++sp) {
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const bf16x8_t bgf = st ? e4m3x8_to_bf16x8(wgv[sp].z, wgv[sp].w)
                                : e4m3x8_to_bf16x8(wgv[sp].x, wgv[sp].y);
        const bf16x8_t buf = st ? e4m3x8_to_bf16x8(wuv[sp].z, wuv[sp].w)
                                : e4m3x8_to_bf16x8(wuv[sp].x, wuv[sp].y);
        const int kc = 64 * sp + 16 * (lane >> 4) + 8 * st;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const bf16x8_t af = lds_bf16x8(As + (16 * m + (lane & 15)) * kLda + kc);
          bg[m] = mfma16(af, bgf, bg[m]);
          bu[m] = mfma16(af, buf, bu[m]);
        }
      }
    }
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        accg[m][i] = fmaf(sg, bg[m][i], accg[m][i]);
        accu[m][i] = fmaf(su, bu[m][i], accu[m][i]);
      }
  }
  // D layout: lane L holds rows 4*(L/16) + i of column L%16
  const int col = n0 + (lane & 15);
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * m + 4 * (lane >> 4) + i;
      if (row < valid) h[(size_t)(r0 + row) * I + col] = f32_to_f16_sat(silu(accg[m][i]) * accu[m][i]);
    }
}

template <int H, int I, int B>
__global__ __launch_bounds__(256) void mfma_down(MfmaBank bk, const int32_t* __restrict__ meta,
                                                const int32_t* __restrict__ tiles,
                                                const int32_t* __restrict__ offsets, int E,
                                                const uint16_t* __restrict__ h,
                                                float* __restrict__ y) {
  static_assert(B == kBK && I % kBK == 0 && H % 128 == 0, "MFMA tiling");
  __shared__ uint16_t As[kMfmaBM * kLda];
  const int tile = blockIdx.y;
  if (tile >= meta[1]) return;
  const int g = tiles[2 * tile], r0 = tiles[2 * tile + 1];
  const int valid = min(kMfmaBM, offsets[g + 1] - r0);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n0 = blockIdx.x * 128 + wave * 32;  // this wavefront's 32 output columns
  const bool sh = g == E;
  const uint8_t* W = sh ? bk.sh_wd : bk.wd + (size_t)g * H * I;
  const float* Sc = sh ? bk.sh_sd : bk.sd + (size_t)g * (H / B) * (I / B);
  const uint8_t* w_row[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
    w_row[nb] = W + (size_t)(n0 + 16 * nb + (lane & 15)) * I + 16 * (lane >> 4);
  const float* s_row = Sc + (size_t)(n0 / B) * (I / B);  // 32 columns share a scale row
  auto hrow = [&](int row) { return h + (size_t)(r0 + row) * I; };

  f32x4_t acc[4][2];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) acc[m][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int kb = 0; kb < I / kBK; ++kb) {
    const int k0 = kb * kBK;
    uint4 wv[2][2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int sp = 0; sp < 2; ++sp) wv[nb][sp] = ld16(w_row[nb] + k0 + 64 * sp);
    const float sc = s_row[kb];
    __syncthreads();
    stage_a(As, hrow, valid, k0);
    __syncthreads();

    f32x4_t b[4][2];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) b[m][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int sp = 0; sp < 2; ++sp) {
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        f16x8_t bf[2];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          bf[nb] = st ? e4m3x8_to_f16x8(wv[nb][sp].z, wv[nb][sp].w)
                      : e4m3x8_to_f16x8(wv[nb][sp].x, wv[nb][sp].y);
        const int kc = 64 * sp + 16 * (lane >> 4) + 8 * st;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const f16x8_t af = lds_f16x8(As + (16 * m + (lane & 15)) * kLda + kc);
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) b[m][nb] = mfma16_f16(af, bf[nb], b[m][nb]);
        }
      }
    }
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[m][nb][i] = fmaf(sc, b[m][nb][i], acc[m][nb][i]);
  }
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * m + 4 * (lane >> 4) + i;
      if (row < valid) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          y[(size_t)(r0 + row) * H + n0 + 16 * nb + (lane & 15)] = acc[m][nb][i];
      }
    }
}

// ---------------------------------------------------------------------------
template <int H, int I, int B>
static void run_mfma(const Dims& d, const void* x, const MfmaBank& bk, const Work& w,
                     hipStream_t s, hipEvent_t after_gate_up) {
  const unsigned ntiles = (unsigned)max_mfma_tiles(d);
  mfma_gate_up<H, I, B><<<dim3(I / 64, ntiles), 256, 0, s>>>(
      reinterpret_cast<const uint16_t*>(x), bk, w.meta, w.tiles, w.offsets, w.rtok, d.E,
      reinterpret_cast<uint16_t*>(w.h));
  if (after_gate_up) (void)hipEventRecord(after_gate_up, s);
  mfma_down<H, I, B><<<dim3(H / 128, ntiles), 256, 0, s>>>(
      bk, w.meta, w.tiles, w.offsets, d.E, reinterpret_cast<const uint16_t*>(w.h), w.y);
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
