// permute.hip — the token -> expert permutation: the multi-block kernels for
// larger batches (perm_count, perm_scatter), and the fused decode kernel that
// selects every token's experts and then permutes them.
#include "layer.hpp"
#include "permute.hpp"
#include "gemv_body.hpp"
#include "select.hpp"

namespace moe {

// Decode sizes (T <= 16, E <= 512): one workgroup of T wavefronts, which
// selects and permutes without any result leaving the compute unit between
// the steps.
//   1. wavefront t selects token t's experts and gates (select_token); lane
//      j < k sets bit t of its expert's token mask (LDS). With at most 16
//      tokens a mask holds an expert's whole token set, and since a token's
//      experts are distinct every (expert, token) bit is set once.
//   2. wavefront 0: lane L owns experts NV L .. NV L + NV - 1 (ascending
//      with L); the group sizes are the masks' popcounts, their exclusive
//      scan gives the groups' first rows, and a scan of the non-empty flags
//      places the group descriptors (and, for the MFMA family, one row tile
//      per group: a group has at most 16 < tile_rows rows).
//   3. the slot of token t's j-th choice e goes to row first[e] + (tokens
//      below t in e's mask): rows keep ascending token order (stable).
// Same results as topk_softmax + the multi-block permutation. U: partial
// logits requested together per expert (the slice count when it is 1, 4 or
// 8, so that no request repeats a clamped slice).
template <int NV, int U>
__global__ __launch_bounds__(64 * kGemvMaxTokens) void select_permute_small(
    const float* __restrict__ plog, int slices, const float* __restrict__ bias, int64_t T, int k,
    int E, int S, int32_t* __restrict__ topk, float* __restrict__ gates,
    int32_t* __restrict__ offsets, int32_t* __restrict__ pair, int32_t* __restrict__ inv,
    int32_t* __restrict__ rtok, int32_t* __restrict__ meta, int4* __restrict__ gdesc,
    int32_t* __restrict__ tiles, int tile_rows, int32_t* __restrict__ cmb, int ncmb,
    uint64_t* __restrict__ lsync, int nlsync, uint32_t* __restrict__ status) {
  static_assert(kGemvMaxTokens <= 32, "a token mask is one 32-bit word");
  // the down kernel's combine counters (when it combines), or the one-launch
  // grouped passes' give-up word, per-tile counters and status: zero for
  // this call
  for (int i = threadIdx.x; i < ncmb; i += blockDim.x) cmb[(size_t)i * kCmbStride] = 0;
  for (int i = threadIdx.x; i < nlsync; i += blockDim.x) lsync[i] = 0ull;
  if (nlsync > 0 && threadIdx.x == 0) *status = 0u;
  __shared__ uint32_t tmask[64 * NV];  // bit t: token t chose the expert
  __shared__ int32_t first[64 * NV];   // first row of each expert's group
  __shared__ int32_t routed_rows;
  const int t = threadIdx.x >> 6, lane = threadIdx.x & 63;  // blockDim.x = 64 T
  for (int e = threadIdx.x; e < 64 * NV; e += blockDim.x) tmask[e] = 0u;
  __syncthreads();
  const int my_e = select_token<NV, U>(plog, slices, bias, T, t, E, k, topk, gates, nullptr);
  if (lane < k) atomicOr(&tmask[my_e], 1u << t);
  __syncthreads();
  if (t == 0) {
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
        offsets[e] = run;
        first[e] = run;
        if (c > 0) {
          gdesc[apos] = make_int4(e, run, c, 0);
          if (tile_rows > 0) {
            tiles[2 * apos] = e;
            tiles[2 * apos + 1] = run;
          }
          ++apos;
        }
        run += c;
      }
    }
    if (lane == 0) {
      offsets[E] = total;
      offsets[E + 1] = total + S * (int)T;
      if (S) {
        gdesc[nact] = make_int4(E, total, (int)T, 0);
        if (tile_rows > 0) {
          tiles[2 * nact] = E;
          tiles[2 * nact + 1] = total;
        }
      }
      meta[0] = nact + S;
      meta[1] = tile_rows > 0 ? nact + S : 0;
      // XCD chunks of the tile list (every tile here is thin: equal counts)
      const int ntl = tile_rows > 0 ? nact + S : 0;
      for (int x = 1; x < kXcdCount; ++x) meta[kMetaXcdBounds + x - 1] = x * ntl / kXcdCount;
      routed_rows = total;
    }
    for (int y = nact + S + lane; y < E + 2; y += 64) gdesc[y] = make_int4(-1, 0, 0, 0);
  }
  __syncthreads();
  const int TK = (int)(T * k);
  if (lane < k) {
    const int row = first[my_e] + __popc(tmask[my_e] & ((1u << t) - 1u));
    const int s = t * k + lane;
    pair[row] = s;
    inv[s] = row;
    rtok[row] = t;
  }
  if (S && lane == 0) {  // the shared group: slot TK + t is token t
    const int row = routed_rows + t;
    pair[row] = TK + t;
    inv[TK + t] = row;
    rtok[row] = t;
  }
}

bool small_select_permute(const Dims& d) {
  static_assert(kGemvMaxTokens <= kMfmaBM, "a decode group fits one MFMA row tile");
  return d.T <= kGemvMaxTokens && d.E <= 64 * 8;
}

hipError_t launch_select_permute_small(const Dims& d, const float* plog, const float* bias,
                                       const Work& w, int tile_rows, hipStream_t s) {
  const int ns = router_slices(d);
  const int nv = (d.E + 63) / 64;
  const unsigned threads = (unsigned)(64 * d.T);
  int32_t* cmb = d.fold_combine ? static_cast<int32_t*>(w.sync) : nullptr;
  const int ncmb = d.fold_combine ? (int)d.T * gemv_down_items(d) : 0;
  const bool one = tile_rows > 0 && layer_one_launch(d);
  uint64_t* lsync = one ? static_cast<uint64_t*>(w.sync) : nullptr;
  const int nlsync = one ? (int)(layer_sync_bytes(d) / 8) : 0;
#define MOE_SPU(NV, U)                                                                        \
  select_permute_small<NV, U><<<1, threads, 0, s>>>(plog, ns, bias, d.T, d.k, d.E, d.S,       \
                                                    w.topk, w.gates, w.offsets, w.pair, w.inv, \
                                                    w.rtok, w.meta,                            \
                                                    reinterpret_cast<int4*>(w.gdesc), w.tiles, \
                                                    tile_rows, cmb, ncmb, lsync, nlsync,       \
                                                    w.status)
#define MOE_SP(NV)            \
  if (ns == 1)                \
    MOE_SPU(NV, 1);           \
  else if (ns == 4)           \
    MOE_SPU(NV, 4);           \
  else if (ns == 8)           \
    MOE_SPU(NV, 8);           \
  else                        \
    MOE_SPU(NV, NV <= 2 ? 16 : 8)
  if (nv <= 1) {
    MOE_SP(1);
  } else if (nv <= 2) {
    MOE_SP(2);
  } else if (nv <= 4) {
    MOE_SP(4);
  } else {
    MOE_SP(8);
  }
#undef MOE_SP
#undef MOE_SPU
  return hipGetLastError();
}

// ------------------------------------------------------ multi-block (T > 16)
// The token -> expert permutation, spread over NB blocks of consecutive
// slots so that large batches are not serialised on one compute unit.
//   perm_count: block b histograms its slots (LDS counters) into
//     bcnt[b][E]; then it publishes them (device-scope release, one atomic
//     increment of *counter) and the block that completes the count
//     (acquire) turns the histograms into offsets, per-block bases
//     bbase[b][e] = offsets[e] + (rows of e in blocks before b), group
//     descriptors and MFMA row tiles. No block waits for another. *counter
//     must be zero at launch. Up to kPermOneBlock slots run as one block,
//     which takes the counts straight from LDS (no hand-over); up to
//     kPermPlaceSlots it then places every slot itself (place_slots), so no
//     second launch follows.
//   perm_scatter: block b places its slots (place_slots): its wavefronts
//     take consecutive sub-ranges, count per (wavefront, expert), take
//     exclusive prefixes over wavefronts on top of bbase[b][e] (after a
//     one-block count, block b is its 1024-slot chunk b, whose bases the
//     count took from a histogram per chunk), and walk their slots in order
//     with ballot peer ranks, so rows keep slot order.
constexpr int kPermBlockSlots = 512;  // slots per block (at most kPermMaxBlocks blocks)
constexpr int kPermBatch = 4;         // slot loads per thread issued together
constexpr int kPermMaxBlocks = kPermMaxBlocksHost;

constexpr int kPermOneBlock = 4096;   // up to this many slots: one block, no hand-over
constexpr int kPermPlaceSlots = 1024; // up to this many: that block also places them
inline int perm_blocks(int64_t TK) {
  if (TK <= kPermOneBlock) return 1;
  int64_t nb = (TK + kPermBlockSlots - 1) / kPermBlockSlots;
  return (int)(nb < 1 ? 1 : (nb > kPermMaxBlocks ? kPermMaxBlocks : nb));
}

// Places slots [blo, bhi) of the permutation with the calling block (1024
// threads): wavefront w takes a consecutive sub-range, counts its experts in
// wcnt[w][e] (LDS, 16 x E), the exclusive prefixes over wavefronts are taken
// on top of base(e) (the block's first row of expert e), and each wavefront
// walks its slots in order with ballot peer ranks, so rows keep slot order.
template <class Base>
__device__ __forceinline__ void place_slots(const int32_t* __restrict__ topk, int k, int E,
                                            int64_t blo, int64_t bhi, Base base, int32_t* wcnt,
                                            int32_t* __restrict__ pair, int32_t* __restrict__ inv,
                                            int32_t* __restrict__ rtok) {
  constexpr int W = 16;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t wper = (bhi - blo + W - 1) / W;
  const int64_t lo = blo + w * wper < bhi ? blo + w * wper : bhi;
  const int64_t hi = lo + wper < bhi ? lo + wper : bhi;
  for (int i = tid; i < W * E; i += 1024) wcnt[i] = 0;
  __syncthreads();
  // the wavefront's slots, kPermBatch rounds of 64 at a time: loaded (clamped,
  // unconditional) before any is used, kept for the walk below when the
  // wavefront has at most kPermBatch rounds
  int ev[kPermBatch];
#pragma unroll
  for (int i = 0; i < kPermBatch; ++i) ev[i] = 0;
  for (int64_t s0 = lo + lane; s0 < hi; s0 += 64 * kPermBatch) {
#pragma unroll
    for (int i = 0; i < kPermBatch; ++i) {
      const int64_t s = s0 + 64 * i;
      ev[i] = topk[s < hi ? s : hi - 1];
    }
#pragma unroll
    for (int i = 0; i < kPermBatch; ++i)
      if (s0 + 64 * i < hi && (unsigned)ev[i] < (unsigned)E) atomicAdd(&wcnt[w * E + ev[i]], 1);
  }
  __syncthreads();
  // exclusive prefix over wavefronts on top of the block's base
  for (int e = tid; e < E; e += 1024) {
    int run = base(e);
    for (int ww = 0; ww < W; ++ww) {
      const int c = wcnt[ww * E + e];
      wcnt[ww * E + e] = run;
      run += c;
    }
  }
  __syncthreads();
  const int ebits = E > 1 ? 32 - __clz(E - 1) : 0;
  const bool held = hi - lo <= 64 * kPermBatch;  // uniform: ev holds every round
  for (int64_t b0 = lo; b0 < hi; b0 += 64) {
    const int64_t s = b0 + lane;
    int e_in = 0;
    if (held) {
#pragma unroll
      for (int i = 0; i < kPermBatch; ++i)
        if (b0 == lo + 64 * i) e_in = ev[i];
    } else if (s < hi) {
      e_in = topk[s];
    }
    const bool ok = s < hi && (unsigned)e_in < (unsigned)E;
    const int e = ok ? e_in : 0;
    if (s < hi && !ok) inv[s] = -1;
    unsigned long long peers = __ballot(ok);
    for (int b = 0; b < ebits; ++b) {
      const bool bit = (e >> b) & 1;
      const unsigned long long m = __ballot(ok && bit);
      peers &= bit ? m : ~m;
    }
    if (!ok) peers = 0;
    const int rank = __popcll(peers & ((1ull << lane) - 1ull));
    const int leader = ok ? (__ffsll((long long)peers) - 1) : lane;
    int old = 0;
    if (ok && lane == leader) old = atomicAdd(&wcnt[w * E + e], __popcll(peers));
    old = __shfl(old, leader, 64);
    if (ok) {
      const int pos = old + rank;
      pair[pos] = (int)s;
      inv[s] = pos;
      rtok[pos] = (int)(s / k);
    }
  }
}

// The shared group's rows: slot TK + t is token t, at row total + t.
__device__ __forceinline__ void place_shared(int64_t T, int64_t TK, int total,
                                             int32_t* __restrict__ pair,
                                             int32_t* __restrict__ inv,
                                             int32_t* __restrict__ rtok) {
  for (int64_t t = threadIdx.x; t < T; t += 1024) {
    pair[total + t] = (int)(TK + t);
    inv[TK + t] = (int)(total + t);
    rtok[total + t] = (int)t;
  }
}

__global__ __launch_bounds__(1024) void perm_count(
    const int32_t* __restrict__ topk, int64_t T, int k, int E, int S, int nb,
    int32_t* bcnt, int32_t* counter, int32_t* __restrict__ offsets, int32_t* bbase,
    int32_t* __restrict__ meta, int4* __restrict__ gdesc, int32_t* __restrict__ tiles,
    int tile_rows, uint64_t* __restrict__ lsync, uint32_t* __restrict__ status, int32_t* pair,
    int32_t* inv, int32_t* rtok, int place_all) {
  // place_all (uniform, one block only): this block also places every slot
  // (place_slots), with the dynamic LDS as its 16 x E wavefront counters
  extern __shared__ int32_t wcnt[];
  __shared__ int32_t cnt[kMaxExperts];
  // one block: a histogram per 1024-slot chunk (the placing blocks' ranges)
  __shared__ int32_t cntc[kPermBatch][kMaxExperts];
  __shared__ int32_t tmp[4 * 64];
  __shared__ int last;
  const int tid = threadIdx.x;
  const int64_t TK = T * k;
  const int64_t per = (TK + nb - 1) / nb;
  const int64_t lo = (int64_t)blockIdx.x * per, hi = lo + per < TK ? lo + per : TK;
  static_assert(kPermOneBlock == 1024 * kPermBatch, "one block: one load round, chunk i = batch i");
  for (int e = tid; e < E; e += 1024) {
    cnt[e] = 0;
#pragma unroll
    for (int i = 0; i < kPermBatch; ++i) cntc[i][e] = 0;
  }
  __syncthreads();
  // kPermBatch slots per thread are loaded before any is counted (indices
  // clamped, so the loads are unconditional and go out together); one block
  // counts slot tid + 1024 i into chunk i's histogram
  for (int64_t s0 = lo + tid; s0 < hi; s0 += 1024 * kPermBatch) {
    int ev[kPermBatch];
#pragma unroll
    for (int i = 0; i < kPermBatch; ++i) {
      const int64_t s = s0 + 1024 * i;
      ev[i] = topk[s < hi ? s : hi - 1];
    }
#pragma unroll
    for (int i = 0; i < kPermBatch; ++i)
      if (s0 + 1024 * i < hi && (unsigned)ev[i] < (unsigned)E)
        atomicAdd(nb == 1 ? &cntc[i][ev[i]] : &cnt[ev[i]], 1);
  }
  __syncthreads();
  const int e = tid;  // from here on one expert per thread (E <= 1024)
  // per-block bases for the placing blocks: one per counting block, or
  // after a one-block count one per 1024-slot chunk
  const int nbases = nb == 1 ? (int)((TK + 1023) / 1024) : nb;
  int c = 0;
  int32_t pre[kPermMaxBlocks];
  if (nb == 1) {  // uniform: the one block holds every count, per chunk
#pragma unroll
    for (int b = 0; b < kPermMaxBlocks; ++b) {
      const int v = (e < E && b < kPermBatch) ? cntc[b < kPermBatch ? b : 0][e < E ? e : 0] : 0;
      pre[b] = c;
      c += v;
    }
  } else {
    for (int i = tid; i < E; i += 1024) bcnt[(size_t)blockIdx.x * E + i] = cnt[i];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __syncthreads();
    if (tid == 0)
      last = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
             nb - 1;
    __syncthreads();
    if (!last) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    // prefix over blocks, in block order; every count is requested before
    // any is summed (clamped indices)
#pragma unroll
    for (int b = 0; b < kPermMaxBlocks; ++b)
      pre[b] = bcnt[(size_t)(b < nb ? b : nb - 1) * E + (e < E ? e : E - 1)];
#pragma unroll
    for (int b = 0; b < kPermMaxBlocks; ++b) {
      const int v = (e < E && b < nb) ? pre[b] : 0;
      pre[b] = c;
      c += v;
    }
  }
  // non-empty groups and MFMA row tiles, ascending expert, shared last
  const int nf = (e < E && c > 0) ? 1 : 0;
  const int nt = (e < E && tile_rows > 0) ? (c + tile_rows - 1) / tile_rows : 0;
  // the tiles' cost (all but the last are full)
  const int cost = nt > 0 ? (nt - 1) * kTileCostFull + tile_cost(c - (nt - 1) * tile_rows) : 0;
  const int sv[4] = {c, nf, nt, cost};
  int sx[4], st[4];
  block_excl_scan<16, 4>(sv, sx, st, tmp);
  const int off = sx[0], apos = sx[1], tpos = sx[2], pcost = sx[3];
  const int total = st[0], nact = st[1], ntile = st[2];
  if (e < E) {
    offsets[e] = off;
#pragma unroll
    for (int b = 0; b < kPermMaxBlocks; ++b)
      if (b < nbases) bbase[(size_t)b * E + e] = off + pre[b];
    cnt[e] = off;  // (thread e's own counter, read back by thread e only)
  }
  if (tid == 0) {
    offsets[E] = total;
    offsets[E + 1] = (int)(total + S * T);
  }
  if (nf) gdesc[apos] = make_int4(e, off, c, 0);
  for (int m = 0, tp = tpos; m < nt; ++m, ++tp) {
    tiles[2 * tp] = e;
    tiles[2 * tp + 1] = off + m * tile_rows;
  }
  int nshared_tiles = 0;
  if (S && tile_rows > 0) {
    nshared_tiles = (int)((T + tile_rows - 1) / tile_rows);
    for (int i = tid; i < nshared_tiles; i += 1024) {
      tiles[2 * (ntile + i)] = E;
      tiles[2 * (ntile + i) + 1] = (int)(total + (int64_t)i * tile_rows);
    }
  }
  // Cost-balanced chunks of the tile list, one per XCD: chunk x starts at
  // the first tile t with 8 * (cost of the tiles before t) >= x * C. The
  // prefix cost is a step function of the tile index; the target of chunk x
  // lies in exactly one group's cost interval (8 pc, 8 (pc + cost)] (the
  // shared group's last), and that group's thread (thread 0 for the shared
  // group) places the start among its tiles.
  const int64_t shared_cost =
      nshared_tiles > 0 ? (int64_t)(nshared_tiles - 1) * kTileCostFull +
                              tile_cost((int)(T - (int64_t)(nshared_tiles - 1) * tile_rows))
                        : 0;
  const int64_t C = (int64_t)st[3] + shared_cost;
  auto place = [&](int64_t X, int64_t pc, int64_t cst, int n, int first, int x) {
    // X = x * C in (8 pc, 8 (pc + cst)]: smallest m in [1, n] with
    // 8 (cost of the group's first m tiles) >= X
    if (X <= 8 * pc || X > 8 * (pc + cst)) return;
    int64_t m = (X - 8 * pc + 8 * kTileCostFull - 1) / (8 * kTileCostFull);
    if (m > n) m = n;
    meta[kMetaXcdBounds + x - 1] = first + (int)m;
  };
  for (int x = 1; x < kXcdCount; ++x) {
    if (C == 0) {
      if (tid == 0) meta[kMetaXcdBounds + x - 1] = 0;
      continue;
    }
    place((int64_t)x * C, pcost, cost, nt, tpos, x);
    if (tid == 0) place((int64_t)x * C, st[3], shared_cost, nshared_tiles, ntile, x);
  }
  if (tid == 0) {
    if (S) gdesc[nact] = make_int4(E, total, (int)T, 0);
    meta[0] = nact + S;
    meta[1] = ntile + nshared_tiles;
  }
  // the one-launch grouped passes' per-tile counters, give-up word and
  // status: cleared for this call's tiles
  if (lsync) {
    const int ntot = ntile + nshared_tiles;
    for (int i = tid; i <= ntot; i += 1024) lsync[i] = 0ull;
    if (tid == 0) *status = 0u;
  }
  for (int y = nact + S + tid; y < E + 2; y += 1024) gdesc[y] = make_int4(-1, 0, 0, 0);
  if (place_all) {
    place_slots(topk, k, E, 0, TK, [&](int ex) { return cnt[ex]; }, wcnt, pair, inv, rtok);
    if (S) place_shared(T, TK, total, pair, inv, rtok);
  }
}

// lds: 16 * E int32. Block b places slots [b per, (b + 1) per) on top of
// its bases bbase[b][e].
__global__ __launch_bounds__(1024) void perm_scatter(
    const int32_t* __restrict__ topk, int64_t T, int k, int E, int S, int64_t per,
    const int32_t* __restrict__ bbase, const int32_t* __restrict__ offsets,
    int32_t* __restrict__ pair, int32_t* __restrict__ inv, int32_t* __restrict__ rtok) {
  extern __shared__ int32_t wcnt[];  // [16][E]
  const int64_t TK = T * k;
  const int64_t blo = (int64_t)blockIdx.x * per, bhi = blo + per < TK ? blo + per : TK;
  place_slots(topk, k, E, blo, bhi, [&](int e) { return bbase[(size_t)blockIdx.x * E + e]; },
              wcnt, pair, inv, rtok);
  if (S && blockIdx.x == 0) place_shared(T, TK, offsets[E], pair, inv, rtok);
}

__global__ void zero_word(int32_t* p) { *p = 0; }

hipError_t launch_permute(const Dims& d, const int32_t* topk, const Work& w, int tile_rows,
                          bool counter_zeroed, hipStream_t s) {
  int32_t* counter = w.meta + kMetaPermCounter;
  if (!counter_zeroed) zero_word<<<1, 1, 0, s>>>(counter);
  const int64_t TK = d.T * d.k;
  const int nb = perm_blocks(TK);
  // up to kPermPlaceSlots slots (one round of 64 per wavefront) the counting
  // block also places them, with no second launch; above that the placing
  // blocks take the counting blocks' ranges, or after a one-block count its
  // 1024-slot chunks, with the bases perm_count left for each
  const int place_all = TK <= kPermPlaceSlots ? 1 : 0;
  const size_t wlds = (size_t)16 * d.E * sizeof(int32_t);  // at most 64 KiB (E <= 1024)
  perm_count<<<nb, 1024, place_all ? wlds : 0, s>>>(
      topk, d.T, d.k, d.E, d.S, nb, w.pblock, counter, w.offsets,
      w.pblock + (size_t)kPermMaxBlocks * d.E, w.meta, reinterpret_cast<int4*>(w.gdesc), w.tiles,
      tile_rows,
      tile_rows > 0 && layer_one_launch(d) ? static_cast<uint64_t*>(w.sync) : nullptr, w.status,
      w.pair, w.inv, w.rtok, place_all);
  if (!place_all) {
    const int64_t per = nb == 1 ? 1024 : (TK + nb - 1) / nb;
    const int nbs = (int)((TK + per - 1) / per);
    perm_scatter<<<nbs, 1024, wlds, s>>>(topk, d.T, d.k, d.E, d.S, per,
                                         w.pblock + (size_t)kPermMaxBlocks * d.E, w.offsets,
                                         w.pair, w.inv, w.rtok);
  }
  return hipGetLastError();
}

}  // namespace moe
