// permute.hpp — token -> expert permutation helpers (the per-expert fan-out of
// the colizig page's "Features": experts are evaluated one group at a time,
// and the threaded result is bit-identical to the serial one).
//
// Slot s = t*k + j is the j-th choice of token t. The permutation groups the
// slots by expert; inside a group the slots stay in ascending order (stable),
// so a group's rows are its tokens in ascending order. The always-on shared
// expert, when present, is group E with slots T*k + t.
//
// Every kernel that builds it counts per expert (LDS counters), takes
// exclusive scans for the groups' first rows, and places slots in slot order:
// lanes with the same expert find each other with one ballot per expert-id
// bit and take their rank among lower lanes, and the group's first lane
// advances the counter. It also emits a descriptor (group, first row, rows)
// per non-empty group (ascending, shared last, then group = -1 up to E+2
// entries) and, for the MFMA family, one (group, first row) entry per tile of
// tile_rows rows, and the token of every permuted row (rtok).
// Expert ids outside [0, E) (possible only through moe_permute's caller) are
// left out of every group with inv = -1; the shared group then starts right
// after the last valid routed row. Nothing is accessed out of bounds.
#pragma once

#include "device.hpp"

namespace moe {

template <int W>
__device__ int block_excl_scan(int v, int* tmp, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int n = __shfl_up(inc, o, 64);
    if (lane >= o) inc += n;
  }
  if (lane == 63) tmp[w] = inc;
  __syncthreads();
  if (w == 0) {
    const int t = lane < W ? tmp[lane] : 0;
    int ti = t;
#pragma unroll
    for (int o = 1; o < W; o <<= 1) {
      const int n = __shfl_up(ti, o, 64);
      if (lane >= o) ti += n;
    }
    if (lane < W) tmp[32 + lane] = ti - t;
    if (lane == W - 1) tmp[63] = ti;
  }
  __syncthreads();
  const int res = inc - v + tmp[32 + w];
  *total = tmp[63];
  __syncthreads();
  return res;
}

// Exclusive prefix sum over the 64 lanes of a wavefront; *total gets the sum.
__device__ __forceinline__ int wave_excl_scan(int v, int* total) {
  const int inc = wave_incl_scan(v);
  *total = __builtin_amdgcn_readlane(inc, 63);
  return inc - v;
}

// Orders this wavefront's LDS accesses before and after the call.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// The same permutation as permute_body, computed by one wavefront, for small
// problems (T*k <= 64 * kWaveSlotsPerLane slots, E <= 64 * kWaveExpertsPerLane):
// per-expert counters in LDS, wave scans, and the ballot peer ranks taken
// over the slots 64 at a time in slot order. cnt: E int32 of shared memory.
constexpr int kWaveExpertsPerLane = 8;
__device__ __forceinline__ void permute_wave(
    const int32_t* topk, int64_t T, int k, int E, int S, int32_t* __restrict__ offsets,
    int32_t* __restrict__ pair, int32_t* __restrict__ inv, int32_t* __restrict__ rtok,
    int32_t* __restrict__ meta, int4* __restrict__ gdesc, int32_t* __restrict__ tiles,
    int tile_rows, int32_t* cnt) {
  const int lane = threadIdx.x & 63;
  const int TK = (int)(T * k);
  for (int e = lane; e < E; e += 64) cnt[e] = 0;
  wave_lds_sync();
  for (int s = lane; s < TK; s += 64) {
    const int e = topk[s];
    if ((unsigned)e < (unsigned)E) atomicAdd(&cnt[e], 1);
  }
  wave_lds_sync();
  // lane owns experts [lane*EPL, lane*EPL + EPL)
  const int EPL = (E + 63) / 64;
  const int eb = lane * EPL;
  int c[kWaveExpertsPerLane];
  int local = 0, nz = 0, nt = 0;
#pragma unroll
  for (int i = 0; i < kWaveExpertsPerLane; ++i) {
    c[i] = (i < EPL && eb + i < E) ? cnt[eb + i] : 0;
    local += c[i];
    nz += c[i] > 0;
    if (tile_rows > 0) nt += (c[i] + tile_rows - 1) / tile_rows;
  }
  int total, nact, ntile;
  int run = wave_excl_scan(local, &total);
  int apos = wave_excl_scan(nz, &nact);
  int tpos = wave_excl_scan(nt, &ntile);
  wave_lds_sync();
#pragma unroll
  for (int i = 0; i < kWaveExpertsPerLane; ++i) {
    const int e = eb + i;
    if (i < EPL && e < E) {
      offsets[e] = run;
      cnt[e] = run;  // running row of expert e
      if (c[i] > 0) gdesc[apos++] = make_int4(e, run, c[i], 0);
      if (tile_rows > 0)
        for (int m = 0; m < c[i]; m += tile_rows) {
          tiles[2 * tpos] = e;
          tiles[2 * tpos + 1] = run + m;
          ++tpos;
        }
      run += c[i];
    }
  }
  wave_lds_sync();
  // stable scatter, 64 slots at a time in slot order
  const int ebits = E > 1 ? 32 - __clz(E - 1) : 0;
  for (int b0 = 0; b0 < TK; b0 += 64) {
    const int s = b0 + lane;
    const int e_in = s < TK ? topk[s] : 0;
    const bool ok = s < TK && (unsigned)e_in < (unsigned)E;
    const int e = ok ? e_in : 0;
    if (s < TK && !ok) inv[s] = -1;
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
    if (ok && lane == leader) old = atomicAdd(&cnt[e], __popcll(peers));
    old = __shfl(old, leader, 64);
    if (ok) {
      const int pos = old + rank;
      pair[pos] = s;
      inv[s] = pos;
      rtok[pos] = s / k;
    }
  }
  if (S) {  // the shared group: slot TK + t is token t (only when it exists)
    for (int t = lane; t < T; t += 64) {
      pair[total + t] = TK + t;
      inv[TK + t] = total + t;
      rtok[total + t] = t;
    }
  }
  int nshared_tiles = 0;
  if (S && tile_rows > 0) {
    nshared_tiles = (int)((T + tile_rows - 1) / tile_rows);
    for (int i = lane; i < nshared_tiles; i += 64) {
      tiles[2 * (ntile + i)] = E;
      tiles[2 * (ntile + i) + 1] = total + i * tile_rows;
    }
  }
  if (lane == 0) {
    offsets[E] = total;
    offsets[E + 1] = total + S * (int)T;
    if (S) gdesc[nact] = make_int4(E, total, (int)T, 0);
    meta[0] = nact + S;
    meta[1] = ntile + nshared_tiles;
  }
  for (int y = nact + S + lane; y < E + 2; y += 64) gdesc[y] = make_int4(-1, 0, 0, 0);
}

}  // namespace moe
