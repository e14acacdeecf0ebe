// decode_fused.hip — the decode-size layer (T <= 16, wavefront GEMV family)
// in one launch.
//
// The ferrite page describes decode as a fixed graph of operations replayed
// each step; at decode sizes a layer of five kernels spends much of its time
// on kernel boundaries (each a launch, a ramp-up and a drain) rather than on
// moving its expert bytes. Here every step runs in one grid and results pass
// through device memory, ordered by flags and counters instead of kernel
// boundaries. Workgroups by block id:
//   [0, NR)        router items (expert quad, slice of H) -> partial logits;
//                  each sets its flag to the call's epoch and exits
//   NR             select: waits for the NR router flags (and resets them),
//                  sums each logit's slices into LDS, selects every token's
//                  experts and gates, builds the permutation and group
//                  descriptors, zeroes the counters below, and sets every
//                  worker's flag to the epoch
//   [NR+1, +NW)    workers: worker w waits for its flag (and resets it), then
//                  takes gate/up items (group, slab group) w, w + NW, ... in
//                  group order, counting finished items per group, then down
//                  items w, w + NW, ...: it requests a down item's weights,
//                  waits until the item's group has all its gate/up items,
//                  computes y, and counts it for each of its tokens in its
//                  row block; the item that completes a (token, row block)
//                  count (k routed experts plus the shared one) sums that
//                  token's rows into out, in the combine's fixed order.
// A worker's down items start while other workers still run gate/up items,
// with the down weights requested before the wait (the next expert's weights
// prefetched behind the current ones' compute).
//
// Forward progress: routers wait for nothing; the select workgroup waits
// only for routers (lower block ids, dispatched before it); workers wait for
// the select workgroup and for other workers' gate/up items, so the host
// sizes NW to fit on the device beside the select workgroup (from the
// kernel's occupancy), and the routers, which exit without waiting, free
// their slots for workers dispatched after them. Every wait is also bounded
// (kSpinLimit polls): past it the workgroup records an error bit in the
// status word and goes on, so every wavefront exits whatever happens. Flags hold a 64-bit epoch given by the host per call (never 0),
// so stale or arbitrary workspace contents never satisfy a wait; every flag
// is reset to 0 by its consumer within the call, so a captured launch
// replayed with the same epoch also starts from cleared flags. Counters are
// zeroed by the select workgroup before any of their users starts.
//
// Memory order. Cache write-backs and invalidations (agent-scope release and
// acquire fences) cost tens of nanoseconds each and serialise across the
// device, so none is taken per work item: data one workgroup hands to
// another inside the kernel (partial logits, h, y) is stored and read at the
// point of coherence (agent-scope relaxed atomics: sc1), and a producer
// waits for its stores to complete (s_waitcnt 0) before a barrier and the
// signalling atomic. The only fence is the select workgroup's one release of
// the routing results, which it writes with plain stores: every consumer
// reads those lines only after its flag, and no cache holds them before
// (the kernel starts with invalidated caches and nothing reads them
// earlier), so plain loads see the written-back values.
#include <hip/hip_ext.h>

#include <algorithm>
#include <atomic>
#include <chrono>

#include "gemv_body.hpp"
#include "permute.hpp"
#include "router_decode.hpp"
#include "select.hpp"

namespace moe {

constexpr uint32_t kSpinLimit = 1u << 20;  // polls before a wait gives up (about a second)
constexpr int kFusedRouterNT = 4;           // router tokens per wavefront (4 x 4 = 16 tokens)
constexpr uint32_t kStatusRouter = 1u, kStatusExpertFlag = 2u, kStatusGateUp = 4u;
// Flags and counters are spread over separate cache lines (and memory
// channels): polls of one must not queue behind another's updates.
constexpr int kFlagStride = 8;  // uint64 words: 64 bytes
constexpr int kGuStride = 64;   // int32 words: 256 bytes
constexpr int kMaxSlices = 8;   // router slices (H <= 4096 on the GEMV shapes)

struct FusedArgs {
  const void* x;
  const float* wr;
  const float* bias;
  BankPtrs bk;
  void* out;
  float* plog;
  int32_t* topk;
  float* gates;
  int32_t* offsets;
  int32_t* meta;
  int4* gdesc;
  int32_t* rtok;
  int32_t* pair;
  int32_t* inv;
  float* h;
  float* y;
  uint64_t* flags;   // [NR] router flags, then [NW] worker flags (kFlagStride apart)
  int32_t* gu_done;  // [gmax] finished gate/up items per group (kGuStride apart)
  int32_t* cmb;      // [T][down items per group] finished down items (kCmbStride apart)
  uint32_t* status;  // error bits of waits that gave up (0: none), zeroed by select
  uint64_t* failed;  // set to the epoch when a wait of this call gives up
  uint64_t epoch;
  int T, E, k, S, slices, HS, quads, nr, nw, gmax;
};

__device__ __forceinline__ void set_flag(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Bounded waits (one thread). A wait also gives up early once another wait
// of the same call has given up (failed == epoch), so a broken call ends
// after about one spin limit, not one per wait.
struct Waits {
  uint32_t* status;
  uint64_t* failed;
  uint64_t epoch;
  __device__ bool given_up(uint32_t it) const {
    return (it & 1023u) == 1023u &&
           __hip_atomic_load(failed, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == epoch;
  }
  __device__ void fail(uint32_t bit) const {
    atomicOr(status, bit);
    set_flag(failed, epoch);
  }
  __device__ bool flag(uint64_t* p) const {
    for (uint32_t it = 0; it < kSpinLimit && !given_up(it); ++it) {
      if (__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == epoch) return true;
      __builtin_amdgcn_s_sleep(1);
    }
    return false;
  }
  __device__ bool count(int32_t* p, int want) const {
    for (uint32_t it = 0; it < kSpinLimit && !given_up(it); ++it) {
      if (__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= want) return true;
      __builtin_amdgcn_s_sleep(1);
    }
    return false;
  }
};

// Signal after this workgroup's coherent stores: every wavefront waits for
// its stores to complete, then thread 0 runs `signal` after a barrier.
template <class F>
__device__ __forceinline__ void publish(F signal) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) signal();
}

// An expert workgroup's own flag: wait, reset.
__device__ __forceinline__ void take_own_flag(const FusedArgs& a, int slot) {
  if (threadIdx.x == 0) {
    const Waits wt{a.status, a.failed, a.epoch};
    if (!wt.flag(a.flags + (size_t)slot * kFlagStride)) wt.fail(kStatusExpertFlag);
    set_flag(a.flags + (size_t)slot * kFlagStride, 0ull);
  }
  __syncthreads();
}

// ---- select + permute on one 256-thread workgroup -------------------------
// As select_permute_small (permute.hip), with four wavefronts taking tokens
// t = wave, wave + 4, ...: wavefront selection per token (select_token), the
// expert token masks in LDS, the group scan on wavefront 0, then every slot
// placed at its expert's first row plus the number of lower tokens in the
// expert's mask (rows in ascending token order).
template <int NV>
__device__ __forceinline__ void select_permute_block(const FusedArgs& a, uint8_t* smem,
                                                     const float* logits) {
  uint32_t* tmask = reinterpret_cast<uint32_t*>(smem);             // [64 NV]
  int32_t* first = reinterpret_cast<int32_t*>(smem + 256 * NV);    // [64 NV]
  int32_t* routed_rows = reinterpret_cast<int32_t*>(smem + 512 * NV);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int T = a.T, k = a.k, E = a.E, S = a.S;
  for (int e = tid; e < 64 * NV; e += 256) tmask[e] = 0u;
  __syncthreads();
  int my_e[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = wv + 4 * i;
    my_e[i] = -1;
    if (t < T) {
      // the slices are already summed (in slice order) into LDS
      my_e[i] = select_token<NV, 1>(logits, 1, a.bias, T, t, E, k, a.topk, a.gates, nullptr);
      if (lane < k) atomicOr(&tmask[my_e[i]], 1u << t);
    }
  }
  __syncthreads();
  if (wv == 0) {
    uint32_t m[NV];
    int local = 0, nz = 0;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = NV * lane + i;
      m[i] = e < E ? tmask[e] : 0u;
      local += __popc(m[i]);
      nz += m[i] != 0u;
    }
    int total, nact;
    int run = wave_excl_scan(local, &total);
    int apos = wave_excl_scan(nz, &nact);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = NV * lane + i;
      if (e < E) {
        const int c = __popc(m[i]);
        a.offsets[e] = run;
        first[e] = run;
        if (c > 0) a.gdesc[apos++] = make_int4(e, run, c, 0);
        run += c;
      }
    }
    if (lane == 0) {
      a.offsets[E] = total;
      a.offsets[E + 1] = total + S * T;
      if (S) a.gdesc[nact] = make_int4(E, total, T, 0);
      a.meta[0] = nact + S;
      a.meta[1] = 0;
      *routed_rows = total;
    }
    for (int y = nact + S + lane; y < E + 2; y += 64) a.gdesc[y] = make_int4(-1, 0, 0, 0);
  }
  __syncthreads();
  const int TK = T * k;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = wv + 4 * i;
    if (t >= T) break;
    if (lane < k) {
      const int e = my_e[i];
      const int row = first[e] + __popc(tmask[e] & ((1u << t) - 1u));
      const int s = t * k + lane;
      a.pair[row] = s;
      a.inv[s] = row;
      a.rtok[row] = t;
    }
    if (S && lane == 0) {  // the shared group: slot TK + t is token t
      const int row = *routed_rows + t;
      a.pair[row] = TK + t;
      a.inv[TK + t] = row;
      a.rtok[row] = t;
    }
  }
}

// logits[p] = sum over slices s (in slice order) of plog[s][p], p = t E + e,
// for the whole workgroup: Q logits per thread per round, every slice of
// them requested at once (MS: slices held per logit).
template <int MS, int Q>
__device__ __forceinline__ void sum_slices(const FusedArgs& a, float* logits) {
  const int n = a.T * a.E, tid = threadIdx.x;
  for (int base = 0; base < n; base += 256 * Q) {
    float v[Q][MS];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int p = std::min(base + 256 * q + tid, n - 1);
#pragma unroll
      for (int s = 0; s < MS; ++s)
        v[q][s] = ld_coherent(a.plog + (size_t)std::min(s, a.slices - 1) * n + p);
    }
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int p = base + 256 * q + tid;
      float acc = v[q][0];
#pragma unroll
      for (int s = 1; s < MS; ++s)
        if (s < a.slices) acc += v[q][s];
      if (p < n) logits[p] = acc;
    }
  }
}

template <int H, int I>
__device__ __forceinline__ void select_role(const FusedArgs& a, uint8_t* smem) {
  const int tid = threadIdx.x;
  const Waits wt{a.status, a.failed, a.epoch};
  if (tid == 0) __hip_atomic_store(a.status, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  bool ok = true;
  for (int i = tid; i < a.nr; i += 256) ok = wt.flag(a.flags + (size_t)i * kFlagStride) && ok;
  if (!ok) wt.fail(kStatusRouter);
  __syncthreads();
  for (int i = tid; i < a.nr; i += 256) set_flag(a.flags + (size_t)i * kFlagStride, 0ull);
  // LDS: token masks and first rows (4112 bytes), then the T x E logits
  float* logits = reinterpret_cast<float*>(smem + 4112);
  if (a.slices <= 1)
    sum_slices<1, 8>(a, logits);
  else if (a.slices <= 4)
    sum_slices<4, 8>(a, logits);
  else
    sum_slices<kMaxSlices, 4>(a, logits);
  __syncthreads();
  if (a.E <= 64)
    select_permute_block<1>(a, smem, logits);
  else if (a.E <= 128)
    select_permute_block<2>(a, smem, logits);
  else if (a.E <= 256)
    select_permute_block<4>(a, smem, logits);
  else
    select_permute_block<8>(a, smem, logits);
  for (int i = tid; i < a.gmax; i += 256) a.gu_done[(size_t)i * kGuStride] = 0;
  for (int i = tid; i < a.T * DownShape<H, I>::ITEMS; i += 256) a.cmb[(size_t)i * kCmbStride] = 0;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  for (int i = tid; i < a.nw; i += 256)
    set_flag(a.flags + (size_t)(a.nr + i) * kFlagStride, a.epoch);
}

template <int H, int I, int B, int NT, int M, bool XBF16, bool OUT_BF16>
__global__ __launch_bounds__(256) void decode_fused(const FusedArgs a) {
  using GS = GateUpShape<H, I, B, NT, M, XBF16>;
  using DS = DownShape<H, I>;
  // select: token masks and first rows (E <= 512), then T x E logits
  constexpr int kSelBytes = 4112 + kGemvMaxTokens * 512 * 4;
  constexpr int kDownBytes = NT * I * 2 + 2 * NT * 4 + (kGemvMaxTokens + 1) * 4;
  constexpr int kBytes = std::max(GS::LDS, std::max(kSelBytes, kDownBytes));
  __shared__ __attribute__((aligned(16))) uint8_t smem[kBytes];
  const int tid = threadIdx.x;
  int b = blockIdx.x;

  if (b < a.nr) {  // ---- router item
    router_slices_item<kFusedRouterNT, XBF16, true>(a.x, a.wr, a.plog, a.T, H, a.E, a.HS,
                                                    b % a.quads, b / a.quads);
    publish([&] { set_flag(a.flags + (size_t)b * kFlagStride, a.epoch); });
    return;
  }
  b -= a.nr;
  if (b == 0) {  // ---- select + permute
    select_role<H, I>(a, smem);
    return;
  }
  const int w = b - 1;  // ---- worker
  take_own_flag(a, a.nr + w);
  const int nact = a.meta[0];

  // gate/up items. A finished item is counted one item late: the next
  // item's loads were issued after its h stores and vector memory operations
  // complete in issue order, so once the next item has its data (every
  // wavefront past the item's first barrier) those stores are complete; the
  // last item waits for its stores explicitly.
  const int gu_items = nact * GS::ITEMS;
  int prev = -1;  // group of the item finished but not yet counted
  for (int i = w; i < gu_items; i += a.nw) {
    const int gi = i / GS::ITEMS;
    gate_up_item<H, I, B, NT, M, XBF16, true>(a.x, a.bk, a.gdesc[gi], i - gi * GS::ITEMS,
                                              a.rtok, a.E, a.h, smem);
    __syncthreads();  // every wavefront has this item's data, so prev's stores are done
    if (tid == 0 && prev >= 0)
      __hip_atomic_fetch_add(a.gu_done + (size_t)prev * kGuStride, 1, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
    prev = gi;
  }
  if (prev >= 0)
    publish([&] {
      __hip_atomic_fetch_add(a.gu_done + (size_t)prev * kGuStride, 1, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
    });

  // down items, each with its share of the combine
  uint16_t* hs = reinterpret_cast<uint16_t*>(smem);
  uint32_t* hmax = reinterpret_cast<uint32_t*>(smem + NT * I * 2);
  int* hexp = reinterpret_cast<int*>(hmax + NT);
  int* marked = hexp + NT;                // tokens whose row block this item completes
  int* nmarked = marked + kGemvMaxTokens;
  const int dn_items = nact * DS::ITEMS;
  for (int j = w; j < dn_items; j += a.nw) {
    const int gi = j / DS::ITEMS, bx = j - gi * DS::ITEMS;
    const int4 gd = a.gdesc[gi];
    down_item<H, I, B, NT, true>(a.bk, gd, bx, a.E, a.h, a.pair, a.y, hs, hmax, hexp, [&] {
      const Waits wt{a.status, a.failed, a.epoch};
      if (threadIdx.x == 0 && !wt.count(a.gu_done + (size_t)gi * kGuStride, GS::ITEMS))
        wt.fail(kStatusGateUp);
      __syncthreads();
    });
    complete_rows<H, DS::ROWS, DS::ITEMS, OUT_BF16>(gd, bx, a.rtok, a.cmb, a.gates, a.y, a.T,
                                                    a.k, a.S, a.out, marked, nmarked);
  }
}

// ---------------------------------------------------------------- host ---
// Per-call epochs: a process-wide counter started from the clock, so that
// flag words left by another process in reused device memory are not this
// call's epoch either.
static std::atomic<uint64_t> g_epoch{
    (uint64_t)std::chrono::steady_clock::now().time_since_epoch().count() * 0x9E3779B97F4A7C15ull};

template <int H, int I, int B>
struct FusedItems {
  static constexpr int GU = GateUpShape<H, I, B, 1, gate_up_chunks<H>(), true>::ITEMS;
  static constexpr int DN = DownShape<H, I>::ITEMS;
};

#define MOE_FUSED_SHAPES(X) \
  X(64, 32, 32)             \
  X(2048, 768, 128)         \
  X(4096, 1024, 128)

bool fused_decode_ok(const Dims& d) {
  return !d.mfma && d.T >= 1 && d.T <= kGemvMaxTokens && router_kind(d) == kRouterDecode &&
         small_select_permute(d) && has_gemv_instance(d);
}

// Layout of the sync region: flags (NR + every possible expert workgroup),
// gate/up counts per group, down counts per (token, row block).
struct FusedLayout {
  int nr, quads, gmax, gu_items, dn_items, max_workers;
  size_t flags_off, gu_off, cmb_off, bytes;
};

static bool fused_layout(const Dims& d, FusedLayout* L) {
  if (!fused_decode_ok(d)) return false;
  int gu = 0, dn = 0;
#define X(h, i, b)                        \
  if (d.H == h && d.I == i && d.B == b) { \
    gu = FusedItems<h, i, b>::GU;         \
    dn = FusedItems<h, i, b>::DN;         \
  }
  MOE_FUSED_SHAPES(X)
#undef X
  if (gu == 0) return false;
  L->quads = (d.E + 3) / 4;
  L->nr = L->quads * router_slices(d);
  L->gmax = (int)std::min<int64_t>(d.E, d.T * d.k) + d.S;
  L->gu_items = gu;
  L->dn_items = dn;
  const auto al = [](size_t n) { return (n + kAlign - 1) / kAlign * kAlign; };
  L->max_workers = L->gmax * std::max(gu, dn);
  const size_t nflags = (size_t)L->nr + L->max_workers;
  L->flags_off = 0;
  L->gu_off = al(nflags * kFlagStride * 8);
  L->cmb_off = L->gu_off + al((size_t)L->gmax * kGuStride * 4);
  L->bytes = L->cmb_off + al((size_t)d.T * dn * kCmbStride * 4);
  return true;
}

size_t fused_sync_bytes(const Dims& d) {
  FusedLayout L;
  return fused_layout(d, &L) ? L.bytes : 0;
}

// Workgroups of this kernel that fit on the device at once (a grid larger
// than this still completes: later workgroups start as earlier ones end).
template <class K>
static int resident_blocks(K kernel) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 256, 0) != hipSuccess ||
      cus <= 0 || per_cu <= 0)
    return 1024;
  return cus * per_cu;
}

template <int H, int I, int B, int NT, bool XBF16, bool OUT_BF16>
static hipError_t run_fused(const Dims& d, FusedArgs a, const FusedLayout& L, hipStream_t s,
                            KernelEvents ev) {
  constexpr int M = gate_up_chunks<H>();
  auto kernel = decode_fused<H, I, B, NT, M, XBF16, OUT_BF16>;
  static const int cap = resident_blocks(kernel);
  // workers and the select workgroup fit on the device together; a few
  // slots are left for other work
  a.nw = std::max(1, std::min(L.max_workers, cap - 1 - cap / 16));
  const unsigned grid = (unsigned)(a.nr + 1 + a.nw);
  if (ev.any())
    hipExtLaunchKernelGGL(kernel, dim3(grid), dim3(256), 0, s, ev.begin, ev.end, 0, a);
  else
    kernel<<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

template <int H, int I, int B, int NT, bool XBF16>
static hipError_t run_fused_out(const Dims& d, const FusedArgs& a, const FusedLayout& L,
                                hipStream_t s, KernelEvents ev) {
  return d.out_bf16 ? run_fused<H, I, B, NT, XBF16, true>(d, a, L, s, ev)
                    : run_fused<H, I, B, NT, XBF16, false>(d, a, L, s, ev);
}

// tokens per pass as in the per-pass kernels (expert_gemv.hip)
template <int H, int I, int B>
static hipError_t run_fused_nt(const Dims& d, const FusedArgs& a, const FusedLayout& L,
                               hipStream_t s, KernelEvents ev) {
  constexpr int NTF = H <= 1024 ? 4 : 1;
  if (d.x_bf16) {
    if (d.T <= 1) return run_fused_out<H, I, B, 1, true>(d, a, L, s, ev);
    if (d.T <= 2) return run_fused_out<H, I, B, 2, true>(d, a, L, s, ev);
    return run_fused_out<H, I, B, 4, true>(d, a, L, s, ev);
  }
  if (d.T <= 1) return run_fused_out<H, I, B, 1, false>(d, a, L, s, ev);
  return run_fused_out<H, I, B, NTF, false>(d, a, L, s, ev);
}

hipError_t launch_decode_fused(const Dims& d, const void* x, const float* router_w,
                               const float* router_bias, const moe_expert_bank& routed,
                               const moe_expert_bank* shared, const Work& w, void* out,
                               hipStream_t s, KernelEvents ev) {
  FusedLayout L;
  if (!fused_layout(d, &L)) return hipErrorInvalidValue;
  FusedArgs a;
  a.x = x;
  a.wr = router_w;
  a.bias = router_bias;
  a.bk = BankPtrs{routed.w_gate_up, routed.w_down, routed.s_gate_up, routed.s_down,
                  shared ? shared->w_gate_up : nullptr, shared ? shared->w_down : nullptr,
                  shared ? shared->s_gate_up : nullptr, shared ? shared->s_down : nullptr,
                  nullptr};
  a.out = out;
  a.plog = w.logits;
  a.topk = w.topk;
  a.gates = w.gates;
  a.offsets = w.offsets;
  a.meta = w.meta;
  a.gdesc = reinterpret_cast<int4*>(w.gdesc);
  a.rtok = w.rtok;
  a.pair = w.pair;
  a.inv = w.inv;
  a.h = static_cast<float*>(w.h);
  a.y = static_cast<float*>(w.y);
  uint8_t* sync = static_cast<uint8_t*>(w.sync);
  a.flags = reinterpret_cast<uint64_t*>(sync + L.flags_off);
  a.gu_done = reinterpret_cast<int32_t*>(sync + L.gu_off);
  a.cmb = reinterpret_cast<int32_t*>(sync + L.cmb_off);
  a.status = w.status;
  a.failed = reinterpret_cast<uint64_t*>(w.status + 2);
  uint64_t e = g_epoch.fetch_add(1, std::memory_order_relaxed) + 1;
  if (e == 0) e = g_epoch.fetch_add(1, std::memory_order_relaxed) + 1;
  a.epoch = e;
  a.T = (int)d.T;
  a.E = d.E;
  a.k = d.k;
  a.S = d.S;
  a.slices = router_slices(d);
  a.HS = d.H < kRouterSlice ? d.H : kRouterSlice;
  a.quads = L.quads;
  a.nr = L.nr;
  a.gmax = L.gmax;
  a.nw = 0;
#define X(h, i, b)                                       \
  if (d.H == h && d.I == i && d.B == b) return run_fused_nt<h, i, b>(d, a, L, s, ev);
  MOE_FUSED_SHAPES(X)
#undef X
  return hipErrorInvalidValue;
}

}  // namespace moe
