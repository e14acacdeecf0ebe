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

// Exclusive prefix sums of N values per thread over a workgroup of W
// wavefronts (W <= 32), all N at once: DPP scans inside each wavefront, then
// a DPP scan of the wavefront totals by wavefront 0. tmp: N * 64 int32 of
// shared memory; total[i] gets the workgroup's sum of value i.
template <int W, int N>
__device__ void block_excl_scan(const int (&v)[N], int (&res)[N], int (&total)[N], int* tmp) {
  static_assert(W <= 32, "wavefront totals fit one scan");
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int inc[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    inc[i] = wave_incl_scan(v[i]);
    if (lane == 63) tmp[64 * i + w] = inc[i];
  }
  __syncthreads();
  if (w == 0) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int t = lane < W ? tmp[64 * i + lane] : 0;
      const int ti = wave_incl_scan(t);
      if (lane < W) tmp[64 * i + 32 + lane] = ti - t;
      if (lane == W - 1) tmp[64 * i + 63] = ti;
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < N; ++i) {
    res[i] = inc[i] - v[i] + tmp[64 * i + 32 + w];
    total[i] = tmp[64 * i + 63];
  }
  __syncthreads();
}

// Exclusive prefix sum over the 64 lanes of a wavefront; *total gets the sum.
__device__ __forceinline__ int wave_excl_scan(int v, int* total) {
  const int inc = wave_incl_scan(v);
  *total = __builtin_amdgcn_readlane(inc, 63);
  return inc - v;
}

}  // namespace moe
