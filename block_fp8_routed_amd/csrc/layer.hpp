// layer.hpp — host-side description of one layer call, shared by the C ABI
// (moe_api.hip) and the kernel launchers. Internal to libmoe_fp8.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe_fp8.h"

namespace moe {

constexpr int kMaxExperts = 1024;  // permute keeps per-wave expert counters in LDS
constexpr int kMaxTopK = 16;       // top-k keeps the selection in registers
constexpr int kGemvMaxTokens = 16; // decode sizes: one-workgroup selection + permutation
// AUTO takes the wavefront GEMV family up to this many tokens (bf16 x; fp32
// x always): measured faster than the grouped MFMA family through 48 tokens
// on both the 128- and the 512-expert layer, slower from 56-64 on
constexpr int kAutoGemvTokens = 48;
constexpr int kMfmaBM = 128;       // rows (tokens) of one grouped-MFMA tile
constexpr size_t kAlign = 256;

struct Dims {
  int64_t T;     // tokens
  int H, E, I;   // hidden, routed experts, intermediate
  int k, B, S;   // top-k, block edge, shared expert count (0/1)
  int64_t P;     // rows of the permuted problem: T*k + S*T
  bool x_bf16, out_bf16;
  bool mfma;     // expert family: grouped bf16 MFMA (true) or wavefront GEMV
  bool f8;       // grouped family with E4M3 operands in both expert contractions
  bool fused;    // GEMV family with the whole layer in one launch (decode_fused.hip)
  bool fold_combine;  // decode GEMV path: the combine runs inside the down kernel
};

// Router kernels and partial logits. The router writes partial logits per
// slice of H; the top-k kernel sums the slices in slice order.
//  * decode and small batches (T <= 16, or T x E <= kRouterDecodeWork):
//    wavefront dot products over slices of kRouterSlice columns (one slice
//    when H < kRouterSlice), 16 tokens per workgroup (measured faster than
//    the MFMA tiles through 256 tokens of 128 experts and 64 of 512, slower
//    at 128 of 512);
//  * prefill with bf16 activations (H a multiple of 64): MFMA tiles of
//    kRouterTile tokens x kRouterTile experts over the router weights split
//    exactly into three bf16 planes; H is cut into as many slices (a power of
//    two, each a multiple of 128 columns, at most max_router_slices) as
//    brings the tile count x slices to about 512 workgroups, so that small
//    batches still spread over the compute units;
//  * otherwise (fp32 activations at prefill sizes): the fp32 tiled GEMM, one
//    slice.
constexpr int kRouterSlice = 512;
constexpr int kRouterTile = 128;
constexpr int64_t kRouterDecodeWork = 32768;  // tokens x experts
enum RouterKind { kRouterDecode, kRouterMfma, kRouterGemm, kRouterNone };
inline RouterKind router_kind(const Dims& d) {
  const bool slices_ok = d.H < kRouterSlice || d.H % kRouterSlice == 0;
  if (slices_ok && (d.T <= kGemvMaxTokens || d.T * d.E <= kRouterDecodeWork))
    return kRouterDecode;
  if (d.T <= kGemvMaxTokens) return kRouterGemm;
  if (d.x_bf16 && d.H % 64 == 0) return kRouterMfma;
  return kRouterGemm;
}
// slices the top-k kernel sums without a loop: 16 when a lane holds at most
// two experts (E <= 128), else 8
inline int max_router_slices(const Dims& d) { return d.E <= 128 ? 16 : 8; }
// number of partial-logit slices (>= 1)
inline int router_slices(const Dims& d) {
  switch (router_kind(d)) {
    case kRouterDecode:
      return d.H % kRouterSlice == 0 ? d.H / kRouterSlice : 1;
    case kRouterMfma: {
      const int64_t tiles = ((d.T + kRouterTile - 1) / kRouterTile) *
                            ((d.E + kRouterTile - 1) / kRouterTile);
      int ns = 1;
      while (2 * ns <= max_router_slices(d) && tiles * ns < 512 && d.H % (2 * ns * 128) == 0)
        ns *= 2;
      return ns;
    }
    default:
      return 1;
  }
}

constexpr int kMetaPermCounter = 9;    // multi-block permutation's completion counter
// meta[kMetaXcdBounds + x - 1], x = 1 .. kXcdCount - 1: first MFMA row tile of
// XCD x's contiguous range when the tile list is dealt in chunks (XCD 0
// starts at tile 0, the last range ends at meta[1])
constexpr int kMetaXcdBounds = 2;
constexpr int kXcdCount = 8;           // accelerator complex dies (one L2 each)
static_assert(kMetaXcdBounds + kXcdCount - 1 <= kMetaPermCounter, "meta layout");
// Relative cost of a row tile when the chunks are cut: a thin tile (at most
// kMfmaBM / 2 rows) reads the same weights as a full one with half its MFMA
// work. Every range then holds less than C / (8 kTileCostThin) + 1 tiles, C
// the list's total cost (mfma_chunk_tiles).
constexpr int kTileCostFull = 3, kTileCostThin = 2;
__host__ __device__ constexpr int tile_cost(int rows) {
  return rows > kMfmaBM / 2 ? kTileCostFull : kTileCostThin;
}
constexpr int kPermMaxBlocksHost = 16; // blocks of the multi-block permutation (at most)

// Carved workspace. Every region is kAlign-aligned.
struct Work {
  float* logits;     // [slices][T][E] partial router logits (bias not added)
  int32_t* topk;     // [T][k]
  float* gates;      // [T][k]
  int32_t* offsets;  // [E+2]
  int32_t* meta;     // [16]: meta[0] = active groups, meta[1] = MFMA tiles,
                     // meta[kMetaPermCounter]: multi-block permutation's completion count
  int32_t* gdesc;    // [E+2][4] per non-empty group: (group, first row, rows, 0);
                     // group = -1 past the last one (shared group = E)
  int32_t* rtok;     // [P] token of each permuted row
  int32_t* pair;     // [P] row -> slot
  int32_t* inv;      // [P] slot -> row
  int32_t* tiles;    // [max_tiles][2] (group, first row) of each MFMA row tile
  void* h;           // [P][I] SwiGLU output in permuted row order: fp32 (GEMV
                     // family), fp16 scaled per 128 columns by hexps (bf16 MFMA),
                     // E4M3 codes scaled by hexps (FP8 variant)
  void* y;           // [P][H] expert outputs by slot: fp32 (GEMV family), fp16
                     // scaled per 128 columns by yexps (grouped families)
  int32_t* pblock;   // [2][16][E] per-block expert counts, then per-block bases
  uint8_t* acodes;   // [T][H] E4M3 activations (FP8 variant only, else empty)
  uint8_t* aexps;    // [T][H/128] their E8M0 exponents (FP8 variant only)
  uint8_t* hexps;    // [P][I/128] exponent bytes of h (grouped families)
  uint8_t* yexps;    // [P][H/128] exponent bytes of y (grouped families)
  int32_t* slotmap;  // [E+1] slot map of a streamed bank (moe_forward_streamed)
  void* sync;        // single-launch decode layer: flags and counters (decode_fused.hip);
                     // decode GEMV path: the combine's (token, row block) counters
  uint32_t* status;  // single-launch decode layer: error bits of its waits (0: none)
};

inline int64_t max_mfma_tiles(const Dims& d) {
  return d.P / kMfmaBM + d.E + d.S + 1;
}
// The grouped paths (bf16 and FP8) run gate/up and down in one launch
// (expert_mfma.hip, mfma_layer and mfma_layer_f8): the down workgroups wait
// for their tile's gate/up items through one 64-bit counter per row tile in
// the workspace, after a give-up word (word 0; tile t's counter is word
// 1 + t; bits 0-5: items done, bits 6 (1 + x) .. + 5: items done on XCD x).
// The permutation clears the give-up word, the counters of the call's tiles
// and the status word. A streamed bank keeps two launches.
inline bool layer_one_launch(const Dims& d) { return d.mfma; }
inline size_t layer_sync_bytes(const Dims& d) {
  return (size_t)(max_mfma_tiles(d) + 1) * 8;
}
// status bits of the one-launch grouped paths (the single-launch decode
// layer's are 1, 2 and 4): a down workgroup gave up waiting for its tile's
// gate/up items; a tile's gate/up items ran on an XCD other than its down
// workgroup's (h would not be coherent between them)
constexpr uint32_t kStatusLayerWait = 8u, kStatusLayerXcd = 16u;
// poll bound of those waits: dflt, unless moe_set_wait_limit set one
uint32_t layer_wait_limit(uint32_t dflt);

// tile slots per XCD that cover the longest cost-balanced chunk of any tile
// list of this problem (at most max_mfma_tiles tiles, each of cost at most
// kTileCostFull and at least kTileCostThin)
inline int64_t mfma_chunk_tiles(const Dims& d) {
  return max_mfma_tiles(d) * kTileCostFull / (kXcdCount * kTileCostThin) + 1;
}

// Validation shared by the entry points (host only, no HIP call).
moe_status basic_dims(const moe_config* c, Dims* d);
moe_status expert_family_ok(const Dims& d);
bool bank_ok(const moe_expert_bank* b);
moe_status check_workspace(const Dims& d, void* ws, size_t bytes);
// Router, selection and permutation (and the FP8 variant's activation
// quantiser) for one call, with the optional phase events START and ROUTED.
moe_status enqueue_routing(const Dims& d, const void* x, const float* router_w,
                           const float* router_bias, const struct Work& w,
                           const moe_phase_events* events, hipStream_t s);

// Sum of region sizes; carve() lays them out in this order.
size_t workspace_bytes(const Dims& d);
Work carve(const Dims& d, void* base);

// ---- launchers (each returns hipGetLastError() of its launches) ----------
hipError_t launch_router(const Dims& d, const void* x, const float* wr, const Work& w,
                         hipStream_t s);
// Sums the router slices, adds the bias, selects and gates; optionally writes
// the final logits.
// zero_word (may be null): a workspace word the multi-block permutation that
// follows uses as its completion counter; the top-k kernel zeroes it.
hipError_t launch_topk(const Dims& d, const float* plogits, const float* bias, int32_t* topk,
                       float* gates, float* logits_out, int32_t* zero_word, hipStream_t s);
// counter_zeroed: the completion counter (meta[kMetaPermCounter]) was zeroed
// by an earlier kernel on the stream; otherwise a one-thread kernel zeroes it.
hipError_t launch_permute(const Dims& d, const int32_t* topk, const Work& w, int tile_rows,
                          bool counter_zeroed, hipStream_t s);
// Decode sizes: top-k + gates + permutation in one kernel of one workgroup
// (one wavefront per token).
bool small_select_permute(const Dims& d);
hipError_t launch_select_permute_small(const Dims& d, const float* plog, const float* bias,
                                       const Work& w, int tile_rows, hipStream_t s);
// Events attached to the gate/up kernel's own dispatch (either may be null):
// begin takes the kernel's start time, end its end time.
struct KernelEvents {
  hipEvent_t begin, end;
  bool any() const { return begin != nullptr || end != nullptr; }
};
// expert passes; returns hipErrorInvalidValue if no instantiation matches
// slot (device, may be null): for a streamed bank, the slot of each routed
// expert in `routed` (-1: skipped in this launch) and entry E: 0 when the
// shared group runs in this launch, -1 when it is skipped
// out (may be null): with d.fold_combine, the down kernel also combines into
// out (no combine launch follows); null runs the down kernel alone.
hipError_t launch_experts_gemv(const Dims& d, const void* x, const moe_expert_bank& routed,
                               const moe_expert_bank* shared, const Work& w, hipStream_t s,
                               KernelEvents gate_up_events, const int32_t* slot = nullptr,
                               void* out = nullptr);
hipError_t launch_experts_mfma(const Dims& d, const void* x, const moe_expert_bank& routed,
                               const moe_expert_bank* shared, const Work& w, hipStream_t s,
                               KernelEvents gate_up_events, const int32_t* slot = nullptr);
bool has_gemv_instance(const Dims& d);
// Decode GEMV path with the combine inside the down kernel: its (token, row
// block) counters, zeroed by the selection kernel (bytes, 0 when unused).
size_t fold_combine_bytes(const Dims& d);
int gemv_down_items(const Dims& d);
// The single-launch decode layer (decode_fused.hip): whether it covers d
// (GEMV family, 1 <= T <= 16, decode router, E <= 512, a GEMV instance), the
// bytes of its sync region (0 when it does not), and its launch. PERMUTED and
// GATE_UP events, when given, take the kernel's start and end.
bool fused_decode_ok(const Dims& d);
size_t fused_sync_bytes(const Dims& d);
hipError_t launch_decode_fused(const Dims& d, const void* x, const float* router_w,
                               const float* router_bias, const moe_expert_bank& routed,
                               const moe_expert_bank* shared, const Work& w, void* out,
                               hipStream_t s, KernelEvents ev);
bool has_mfma_instance(const Dims& d);
hipError_t launch_combine(const Dims& d, const Work& w, void* out, hipStream_t s);
// x [T][H] bf16 -> E4M3 codes [T][H] and E8M0 exponents [T][H/128]
hipError_t launch_quant_act(const void* x, int64_t T, int H, uint8_t* codes, uint8_t* exps,
                            hipStream_t s);

}  // namespace moe
