// moe_api.hip — the C ABI of libmoe_fp8.so (declared in include/moe_fp8.h):
// argument validation, workspace layout and the launch sequence of one layer.
//
// Nothing here allocates or synchronises the host; the only state kept
// between calls is the poll bound a test may set (moe_set_wait_limit).
// Every check runs on the host before the first launch, following the colizig
// page's rule (Status / Contributing) that an unsupported or invalid request
// returns an error instead of a plausible-looking wrong number.
#include <algorithm>
#include <atomic>

#include "layer.hpp"

namespace moe {

static size_t al(size_t n) { return (n + kAlign - 1) / kAlign * kAlign; }

static std::atomic<uint32_t> g_wait_limit{0};  // 0: each wait's default bound
uint32_t layer_wait_limit(uint32_t dflt) {
  const uint32_t v = g_wait_limit.load(std::memory_order_relaxed);
  return v ? v : dflt;
}

// Region sizes in carve order.
constexpr int kRegions = 20;

static void region_sizes(const Dims& d, size_t* sz) {
  sz[0] = (size_t)router_slices(d) * d.T * d.E * 4;  // partial router logits
  sz[1] = (size_t)d.T * d.k * 4;          // topk
  sz[2] = (size_t)d.T * d.k * 4;          // gates
  sz[3] = (size_t)(d.E + 2) * 4;          // offsets
  sz[4] = 16 * 4;                         // meta
  sz[5] = (size_t)(d.E + 2) * 16;         // group descriptors
  sz[6] = (size_t)d.P * 4;                // rtok
  sz[7] = (size_t)d.P * 4;                // pair
  sz[8] = (size_t)d.P * 4;                // inv
  sz[9] = (size_t)max_mfma_tiles(d) * 8;  // tiles
  // h and y: fp32 on the decode (GEMV) family; fp16 (h of the FP8 variant:
  // E4M3 bytes) with exponent bytes per 128 columns on the grouped families
  sz[10] = (size_t)d.P * d.I * (d.mfma ? (d.f8 ? 1 : 2) : 4);  // h
  sz[11] = (size_t)d.P * d.H * (d.mfma ? 2 : 4);               // y
  sz[12] = (size_t)2 * kPermMaxBlocksHost * d.E * 4;  // permutation block counts and bases
  sz[13] = d.f8 ? (size_t)d.T * d.H : 0;              // E4M3 activations
  sz[14] = d.f8 ? (size_t)d.T * (d.H / 128) : 0;      // their exponents
  sz[15] = d.mfma ? (size_t)d.P * (d.I / 128) : 0;    // exponents of h
  sz[16] = d.mfma ? (size_t)d.P * (d.H / 128) : 0;    // exponents of y
  sz[17] = (size_t)(d.E + 1) * 4;                     // slot map of a streamed bank
  // flags and counters: the single-launch decode layer's, the one-launch
  // grouped path's per-tile counters, or the decode combine fold's
  sz[18] = d.fused              ? fused_sync_bytes(d)
           : layer_one_launch(d) ? layer_sync_bytes(d)
                                 : fold_combine_bytes(d);
  // status word (then the decode layer's give-up tag)
  sz[19] = d.fused || layer_one_launch(d) ? 16 : 0;
}

size_t workspace_bytes(const Dims& d) {
  size_t sz[kRegions], b = 0;
  region_sizes(d, sz);
  for (size_t v : sz) b += al(v);
  return b;
}

Work carve(const Dims& d, void* base) {
  size_t sz[kRegions];
  region_sizes(d, sz);
  char* p = static_cast<char*>(base);
  void* r[kRegions];
  for (int i = 0; i < kRegions; ++i) {
    r[i] = p;
    p += al(sz[i]);
  }
  Work w;
  w.logits = static_cast<float*>(r[0]);
  w.topk = static_cast<int32_t*>(r[1]);
  w.gates = static_cast<float*>(r[2]);
  w.offsets = static_cast<int32_t*>(r[3]);
  w.meta = static_cast<int32_t*>(r[4]);
  w.gdesc = static_cast<int32_t*>(r[5]);
  w.rtok = static_cast<int32_t*>(r[6]);
  w.pair = static_cast<int32_t*>(r[7]);
  w.inv = static_cast<int32_t*>(r[8]);
  w.tiles = static_cast<int32_t*>(r[9]);
  w.h = r[10];
  w.y = r[11];
  w.pblock = static_cast<int32_t*>(r[12]);
  w.acodes = static_cast<uint8_t*>(r[13]);
  w.aexps = static_cast<uint8_t*>(r[14]);
  w.hexps = static_cast<uint8_t*>(r[15]);
  w.yexps = static_cast<uint8_t*>(r[16]);
  w.slotmap = static_cast<int32_t*>(r[17]);
  w.sync = r[18];
  w.status = static_cast<uint32_t*>(r[19]);
  return w;
}

// Shape checks shared by every entry point (no HIP call).
moe_status basic_dims(const moe_config* c, Dims* d) {
  if (!c) return MOE_ERR_NULL;
  if (c->tokens < 0 || c->hidden <= 0 || c->experts <= 0 || c->inter <= 0 || c->top_k <= 0 ||
      c->block <= 0)
    return MOE_ERR_SHAPE;
  if (c->top_k > c->experts) return MOE_ERR_SHAPE;
  if (c->hidden % c->block != 0 || c->inter % c->block != 0) return MOE_ERR_SHAPE;
  if (c->has_shared != 0 && c->has_shared != 1) return MOE_ERR_SHAPE;
  if ((c->x_dtype != MOE_F32 && c->x_dtype != MOE_BF16) ||
      (c->out_dtype != MOE_F32 && c->out_dtype != MOE_BF16))
    return MOE_ERR_SHAPE;
  if (c->path != MOE_PATH_AUTO && c->path != MOE_PATH_GEMV && c->path != MOE_PATH_MFMA &&
      c->path != MOE_PATH_MFMA_FP8 && c->path != MOE_PATH_GEMV_FUSED)
    return MOE_ERR_SHAPE;
  if (c->experts > kMaxExperts || c->top_k > kMaxTopK) return MOE_ERR_UNSUPPORTED;
  if (c->hidden % 16 != 0 || c->inter % 16 != 0) return MOE_ERR_UNSUPPORTED;
  const int64_t P = c->tokens * (int64_t)(c->top_k + c->has_shared);
  if (P >= ((int64_t)1 << 31) || c->tokens * (int64_t)c->experts >= ((int64_t)1 << 40))
    return MOE_ERR_UNSUPPORTED;
  d->T = c->tokens;
  d->H = c->hidden;
  d->E = c->experts;
  d->I = c->inter;
  d->k = c->top_k;
  d->B = c->block;
  d->S = c->has_shared;
  d->P = P;
  d->x_bf16 = c->x_dtype == MOE_BF16;
  d->out_bf16 = c->out_dtype == MOE_BF16;
  d->f8 = c->path == MOE_PATH_MFMA_FP8;
  d->mfma = c->path == MOE_PATH_MFMA || d->f8 ||
            (c->path == MOE_PATH_AUTO && d->x_bf16 && c->tokens > kAutoGemvTokens);
  // the single-launch decode layer only when asked for: the five-launch
  // GEMV path measures faster on MI355X at every decode size
  d->fused = c->path == MOE_PATH_GEMV_FUSED && fused_decode_ok(*d);
  // the combine inside the down kernel: each item waits for its coherent y
  // stores and counts its tokens, which lengthens every down workgroup by a
  // few microseconds; that pays for the combine launch only while the down
  // grid is one round of workgroups (measured: one token -1.0 us per step;
  // c1 at 4 and 16 tokens +1.0 and +2.3 us, c3 at 8 tokens +6.4 us)
  d->fold_combine = !d->mfma && !d->fused && d->T >= 1 && small_select_permute(*d) &&
                    has_gemv_instance(*d) &&
                    (std::min<int64_t>(d->E, d->T * d->k) + d->S) * gemv_down_items(*d) <= 1024;
  return MOE_OK;
}

moe_status expert_family_ok(const Dims& d) {
  if (d.fused) return MOE_OK;
  if (d.mfma) {
    if (!d.x_bf16) return MOE_ERR_UNSUPPORTED;
    if (d.f8 && (d.H % 128 != 0 || d.I % 128 != 0 ||
                 d.T * (int64_t)(d.H / 128) >= ((int64_t)1 << 27)))
      return MOE_ERR_UNSUPPORTED;
    if (max_mfma_tiles(d) > 65535) return MOE_ERR_UNSUPPORTED;  // bounded tile list
    // the passes address activation and h rows with 32-bit byte offsets
    if ((uint64_t)d.T * d.H * 2 > 0xffffffffull || (uint64_t)d.P * d.I * 2 > 0xffffffffull)
      return MOE_ERR_UNSUPPORTED;
    return has_mfma_instance(d) ? MOE_OK : MOE_ERR_UNSUPPORTED;
  }
  return has_gemv_instance(d) ? MOE_OK : MOE_ERR_UNSUPPORTED;
}

bool bank_ok(const moe_expert_bank* b) {
  return b && b->w_gate_up && b->w_down && b->s_gate_up && b->s_down;
}

moe_status check_workspace(const Dims& d, void* ws, size_t bytes) {
  if (!ws) return MOE_ERR_NULL;
  if (bytes < workspace_bytes(d) || reinterpret_cast<uintptr_t>(ws) % kAlign != 0)
    return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

static bool rec(const moe_phase_events* ev, moe_phase p, hipStream_t s) {
  if (!ev || !ev->ev[p]) return true;
  return hipEventRecord(static_cast<hipEvent_t>(ev->ev[p]), s) == hipSuccess;
}

moe_status enqueue_routing(const Dims& d, const void* x, const float* router_w,
                           const float* router_bias, const Work& w, const moe_phase_events* events,
                           hipStream_t s) {
  if (!rec(events, MOE_EV_START, s)) return MOE_ERR_HIP;
  if (launch_router(d, x, router_w, w, s) != hipSuccess) return MOE_ERR_HIP;
  const int tile_rows = d.mfma ? kMfmaBM : 0;
  if (small_select_permute(d)) {
    // decode sizes: selection and permutation share one launch, so ROUTED
    // marks the end of the router logits here
    if (!rec(events, MOE_EV_ROUTED, s)) return MOE_ERR_HIP;
    if (launch_select_permute_small(d, w.logits, router_bias, w, tile_rows, s) != hipSuccess)
      return MOE_ERR_HIP;
  } else {
    if (launch_topk(d, w.logits, router_bias, w.topk, w.gates, nullptr,
                    w.meta + kMetaPermCounter, s) != hipSuccess)
      return MOE_ERR_HIP;
    if (!rec(events, MOE_EV_ROUTED, s)) return MOE_ERR_HIP;
    if (launch_permute(d, w.topk, w, tile_rows, true, s) != hipSuccess) return MOE_ERR_HIP;
  }
  if (d.f8 && launch_quant_act(x, d.T, d.H, w.acodes, w.aexps, s) != hipSuccess)
    return MOE_ERR_HIP;
  return MOE_OK;
}

}  // namespace moe

using namespace moe;

extern "C" {

size_t moe_workspace_bytes(const moe_config* cfg) {
  Dims d;
  if (basic_dims(cfg, &d) != MOE_OK) return 0;
  return workspace_bytes(d);
}

moe_status moe_forward(const void* x, const float* router_w, const float* router_bias,
                       const moe_expert_bank* experts, const moe_expert_bank* shared,
                       int32_t top_k, void* out, const moe_config* cfg, void* workspace,
                       size_t workspace_bytes_, const moe_phase_events* events, void* stream) {
  Dims d;
  moe_status st = basic_dims(cfg, &d);
  if (st != MOE_OK) return st;
  if (top_k != cfg->top_k) return MOE_ERR_SHAPE;
  if (!x || !router_w || !out || !bank_ok(experts)) return MOE_ERR_NULL;
  if (d.S && !bank_ok(shared)) return MOE_ERR_NULL;
  st = expert_family_ok(d);
  if (st != MOE_OK) return st;
  if (d.T == 0) return MOE_OK;
  if (cfg->path == MOE_PATH_GEMV_FUSED && !d.fused) return MOE_ERR_UNSUPPORTED;
  st = check_workspace(d, workspace, workspace_bytes_);
  if (st != MOE_OK) return st;

  const Work w = carve(d, workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  // PERMUTED and GATE_UP are attached to the gate/up kernel's dispatch (its
  // start and end times), so that pair times that kernel alone
  const KernelEvents ev_gate_up{
      events ? static_cast<hipEvent_t>(events->ev[MOE_EV_PERMUTED]) : nullptr,
      events ? static_cast<hipEvent_t>(events->ev[MOE_EV_GATE_UP]) : nullptr};
  if (d.fused) {
    // one kernel: START and ROUTED before it, PERMUTED and GATE_UP on its
    // dispatch, DOWN and END after it
    if (!rec(events, MOE_EV_START, s) || !rec(events, MOE_EV_ROUTED, s)) return MOE_ERR_HIP;
    if (launch_decode_fused(d, x, router_w, router_bias, *experts, d.S ? shared : nullptr, w,
                            out, s, ev_gate_up) != hipSuccess)
      return MOE_ERR_HIP;
    if (!rec(events, MOE_EV_DOWN, s) || !rec(events, MOE_EV_END, s)) return MOE_ERR_HIP;
    return MOE_OK;
  }
  st = enqueue_routing(d, x, router_w, router_bias, w, events, s);
  if (st != MOE_OK) return st;
  const moe_expert_bank* sh = d.S ? shared : nullptr;
  const hipError_t e =
      d.mfma ? launch_experts_mfma(d, x, *experts, sh, w, s, ev_gate_up)
             : launch_experts_gemv(d, x, *experts, sh, w, s, ev_gate_up, nullptr,
                                   d.fold_combine ? out : nullptr);
  if (e != hipSuccess) return MOE_ERR_HIP;
  if (!rec(events, MOE_EV_DOWN, s)) return MOE_ERR_HIP;
  // (decode GEMV path: the down kernel has combined already)
  if (!d.fold_combine && launch_combine(d, w, out, s) != hipSuccess) return MOE_ERR_HIP;
  if (!rec(events, MOE_EV_END, s)) return MOE_ERR_HIP;
  return MOE_OK;
}

moe_status moe_route(const void* x, const float* router_w, const float* router_bias,
                     int32_t* topk_idx, float* gates, float* logits, const moe_config* cfg,
                     void* workspace, size_t workspace_bytes_, void* stream) {
  Dims d;
  moe_status st = basic_dims(cfg, &d);
  if (st != MOE_OK) return st;
  if (!x || !router_w || !topk_idx || !gates) return MOE_ERR_NULL;
  if (d.T == 0) return MOE_OK;
  st = check_workspace(d, workspace, workspace_bytes_);
  if (st != MOE_OK) return st;
  const Work w = carve(d, workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (launch_router(d, x, router_w, w, s) != hipSuccess) return MOE_ERR_HIP;
  if (launch_topk(d, w.logits, router_bias, topk_idx, gates, logits, nullptr, s) != hipSuccess)
    return MOE_ERR_HIP;
  return MOE_OK;
}

moe_status moe_permute(const int32_t* topk_idx, int32_t* offsets, int32_t* pair, int32_t* inv,
                       const moe_config* cfg, void* workspace, size_t workspace_bytes_,
                       void* stream) {
  Dims d;
  moe_status st = basic_dims(cfg, &d);
  if (st != MOE_OK) return st;
  if (!topk_idx || !offsets || !pair || !inv) return MOE_ERR_NULL;
  if (d.T == 0) return MOE_OK;
  st = check_workspace(d, workspace, workspace_bytes_);
  if (st != MOE_OK) return st;
  Work w = carve(d, workspace);
  w.offsets = offsets;
  w.pair = pair;
  w.inv = inv;
  if (launch_permute(d, topk_idx, w, 0, false, static_cast<hipStream_t>(stream)) != hipSuccess)
    return MOE_ERR_HIP;
  return MOE_OK;
}

moe_status moe_workspace_region(const moe_config* cfg, int32_t region, size_t* offset,
                                size_t* bytes) {
  if (!offset || !bytes) return MOE_ERR_NULL;
  Dims d;
  moe_status st = basic_dims(cfg, &d);
  if (st != MOE_OK) return st;
  // carve-order index of each exported region
  static const int kIndex[MOE_WS_COUNT] = {1, 2, 3, 7, 8, 10, 15, 11, 16, 19};
  if (region < 0 || region >= MOE_WS_COUNT) return MOE_ERR_SHAPE;
  size_t sz[kRegions], off = 0;
  region_sizes(d, sz);
  const int idx = kIndex[region];
  for (int i = 0; i < idx; ++i) off += al(sz[i]);
  *offset = off;
  // STATUS: the status word only (the region also holds an internal give-up tag)
  *bytes = region == MOE_WS_STATUS ? std::min<size_t>(sz[idx], 4) : sz[idx];
  return MOE_OK;
}

const char* moe_status_string(moe_status status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_SHAPE: return "invalid shape or argument";
    case MOE_ERR_UNSUPPORTED: return "no kernel for this shape, dtype or path";
    case MOE_ERR_WORKSPACE: return "workspace too small or misaligned";
    case MOE_ERR_HIP: return "HIP launch failed";
    case MOE_ERR_TOO_LARGE: return "the call needs more scratch than the static scratch holds";
  }
  return "unknown status";
}

moe_status moe_set_wait_limit(uint32_t polls) {
  g_wait_limit.store(polls, std::memory_order_relaxed);
  return MOE_OK;
}

int32_t moe_version(void) { return 100; }

}  // extern "C"
