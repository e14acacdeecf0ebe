// permute.hpp — token -> expert permutation helpers (the per-expert fan-out of
// the colizig page's "Features": experts are evaluated one group at a time,
// and the threaded result is bit-identical to the serial one).
//
// Slot s = t*k + j is the j-th choice of token t. The permutation groups the
// slots by expert; inside a group the slots stay in ascending order (stable),
// so a group's rows are its tokens in ascending order. The always-on shared
// expert, when present, is group E with slots T*k + t.
//
// The multi-block kernels count per expert (LDS counters), take exclusive
// scans for the groups' first rows, and place slots in slot order: lanes with
// the same expert find each other with one ballot per expert-id bit and take
// their rank among lower lanes, and the group's first lane advances the
// counter. (The decode kernel, with at most 16 tokens, ranks by token masks
// instead.) Every builder also emits a descriptor (group, first row, rows)
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

}  // namespace moe
