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

#include "gemv_body.hpp"

namespace moe {

// grid: (slab groups, group slots); slots past the last group exit at once.
template <int H, int I, int B, int NT, int M, bool XBF16>
__global__ __launch_bounds__(256) void gemv_gate_up(const void* __restrict__ x, BankPtrs bk,
                                                   const int4* __restrict__ gdesc,
                                                   const int32_t* __restrict__ rtok, int E,
                                                   float* __restrict__ h) {
  __shared__ __attribute__((aligned(16))) uint8_t xs[GateUpShape<H, I, B, NT, M, XBF16>::LDS];
  gate_up_item<H, I, B, NT, M, XBF16>(x, bk, gdesc[blockIdx.y], blockIdx.x, rtok, E, h, xs);
}

// The combine's inputs when the down kernel also combines (complete_rows).
struct FoldCombine {
  int32_t* cmb;         // (token, row block) counters, zeroed by the selection kernel
  const float* gates;   // [T][k]
  const int32_t* rtok;  // token of each permuted row
  void* out;            // [T][H]
  int T, k, S;
};

// COMBINE: 0 the down pass alone (y for the combine kernel); 1 / 2: each item
// then combines the (token, row block)s it completes into fp32 / bf16 out.
template <int H, int I, int B, int NT, int COMBINE>
__global__ __launch_bounds__(256) void gemv_down(BankPtrs bk, const int4* __restrict__ gdesc,
                                                int E, const float* __restrict__ h,
                                                const int32_t* __restrict__ pair,
                                                float* __restrict__ y, FoldCombine fc) {
  __shared__ __attribute__((aligned(16))) uint16_t hs[NT * I];  // scaled fp16 h rows
  __shared__ uint32_t hmax[NT];
  __shared__ int hexp[NT];
  __shared__ int marks[kGemvMaxTokens + 1];
  const int4 gd = gdesc[blockIdx.y];
  down_item<H, I, B, NT, false, COMBINE != 0>(bk, gd, blockIdx.x, E, h, pair, y, hs, hmax, hexp);
  if (COMBINE != 0 && gd.x >= 0)
    complete_rows<H, DownShape<H, I>::ROWS, DownShape<H, I>::ITEMS, COMBINE == 2>(
        gd, blockIdx.x, fc.rtok, fc.cmb, fc.gates, y, fc.T, fc.k, fc.S, fc.out, marks,
        marks + kGemvMaxTokens);
}

// ---------------------------------------------------------------------------
template <int H, int I, int B, int NT, bool XBF16>
static void run_gemv(const Dims& d, const void* x, const BankPtrs& bk, const Work& w,
                     hipStream_t s, KernelEvents ev, void* out) {
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
  const dim3 dgrid((SPG2 + 3) / 4, groups);
  float* y = static_cast<float*>(w.y);
  const FoldCombine fc{static_cast<int32_t*>(w.sync), w.gates, w.rtok, out, (int)d.T, d.k, d.S};
  if (!out)
    gemv_down<H, I, B, NT, 0><<<dgrid, 256, 0, s>>>(bk, gdesc, d.E, h, w.pair, y, fc);
  else if (d.out_bf16)
    gemv_down<H, I, B, NT, 2><<<dgrid, 256, 0, s>>>(bk, gdesc, d.E, h, w.pair, y, fc);
  else
    gemv_down<H, I, B, NT, 1><<<dgrid, 256, 0, s>>>(bk, gdesc, d.E, h, w.pair, y, fc);
}

template <int H, int I, int B>
static void run_gemv_nt(const Dims& d, const void* x, const BankPtrs& bk, const Work& w,
                        hipStream_t s, KernelEvents ev, void* out) {
  // tokens per pass: up to 4 (fp32 activations of wide rows: 1, which keeps
  // their LDS stage at 16 KiB); larger groups take several passes over the
  // weights held in registers
  constexpr int NTF = H <= 1024 ? 4 : 1;
  if (d.x_bf16) {
    if (d.T <= 1) run_gemv<H, I, B, 1, true>(d, x, bk, w, s, ev, out);
    else if (d.T <= 2) run_gemv<H, I, B, 2, true>(d, x, bk, w, s, ev, out);
    else run_gemv<H, I, B, 4, true>(d, x, bk, w, s, ev, out);
  } else {
    if (d.T <= 1) run_gemv<H, I, B, 1, false>(d, x, bk, w, s, ev, out);
    else run_gemv<H, I, B, NTF, false>(d, x, bk, w, s, ev, out);
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

int gemv_down_items(const Dims& d) {
#define X(h, i, b) \
  if (d.H == h && d.I == i && d.B == b) return DownShape<h, i>::ITEMS;
  MOE_GEMV_SHAPES(X)
#undef X
  return 0;
}

size_t fold_combine_bytes(const Dims& d) {
  return d.fold_combine ? (size_t)d.T * gemv_down_items(d) * kCmbStride * 4 : 0;
}

hipError_t launch_experts_gemv(const Dims& d, const void* x, const moe_expert_bank& routed,
                               const moe_expert_bank* shared, const Work& w, hipStream_t s,
                               KernelEvents gate_up_events, const int32_t* slot, void* out) {
  if (out && !d.fold_combine) return hipErrorInvalidValue;
  BankPtrs bk{routed.w_gate_up, routed.w_down, routed.s_gate_up, routed.s_down,
              shared ? shared->w_gate_up : nullptr, shared ? shared->w_down : nullptr,
              shared ? shared->s_gate_up : nullptr, shared ? shared->s_down : nullptr, slot};
#define X(h, i, b)                                       \
  if (d.H == h && d.I == i && d.B == b) {                \
    run_gemv_nt<h, i, b>(d, x, bk, w, s, gate_up_events, out); \
    return hipGetLastError();                            \
  }
  MOE_GEMV_SHAPES(X)
#undef X
  return hipErrorInvalidValue;
}

}  // namespace moe
