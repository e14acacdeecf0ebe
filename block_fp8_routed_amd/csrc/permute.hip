// permute.hip — the token -> expert permutation kernels (permute_body), and
// the fused decode kernel that selects every token's experts and permutes in
// one workgroup (permute_wave).
#include "layer.hpp"
#include "permute.hpp"
#include "select.hpp"

namespace moe {

template <int W>
__global__ __launch_bounds__(64 * W) void permute_kernel(
    const int32_t* __restrict__ topk, int64_t T, int k, int E, int S,
    int32_t* __restrict__ offsets, int32_t* __restrict__ pair, int32_t* __restrict__ inv,
    int32_t* __restrict__ rtok, int32_t* __restrict__ meta, int4* __restrict__ gdesc,
    int32_t* __restrict__ tiles, int tile_rows) {
  extern __shared__ int32_t lds[];
  permute_body<W>(topk, T, k, E, S, offsets, pair, inv, rtok, meta, gdesc, tiles, tile_rows, lds);
}

// Decode sizes (T <= 16, E <= 512): workgroup t (one wavefront) selects token
// t's experts and gates (select_token) and writes them out. Selection is most
// of the kernel's work, so the tokens run on as many compute units. Each
// workgroup then publishes its result (release fence, then one atomic
// increment of *counter at device scope); the workgroup that brings the count
// to T is the last, and after an acquire fence it reads every token's
// selection back and builds the permutation alone (permute_wave). No
// workgroup ever waits for another. *counter must be zero at launch (the
// router kernel, launched just before on the same stream, zeroes it). Same
// results as topk_softmax + permute_kernel.
template <int NV>
__global__ __launch_bounds__(64) void select_permute_small(
    const float* __restrict__ plog, int slices, const float* __restrict__ bias, int64_t T, int k,
    int E, int S, int32_t* topk, float* __restrict__ gates, int32_t* counter,
    int32_t* __restrict__ offsets, int32_t* __restrict__ pair, int32_t* __restrict__ inv,
    int32_t* __restrict__ rtok, int32_t* __restrict__ meta, int4* __restrict__ gdesc,
    int32_t* __restrict__ tiles, int tile_rows) {
  __shared__ int32_t cnt[64 * kWaveExpertsPerLane];
  select_token<NV>(plog, slices, bias, T, blockIdx.x, E, k, topk, gates, nullptr, nullptr);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __builtin_amdgcn_wave_barrier();
  int done = 0;
  if (threadIdx.x == 0) done = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT);
  done = __builtin_amdgcn_readfirstlane(done);
  if (done != T - 1) return;  // uniform: not the last token
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  permute_wave(topk, T, k, E, S, offsets, pair, inv, rtok, meta, gdesc, tiles, tile_rows, cnt);
}

bool small_select_permute(const Dims& d) {
  return d.T <= kGemvMaxTokens && d.E <= 64 * kWaveExpertsPerLane;
}

hipError_t launch_select_permute_small(const Dims& d, const float* plog, const float* bias,
                                       const Work& w, int tile_rows, hipStream_t s) {
  const int ns = router_slices(d);
  const int nv = (d.E + 63) / 64;
  const unsigned grid = (unsigned)d.T;
#define MOE_SP(NV)                                                                          \
  select_permute_small<NV><<<grid, 64, 0, s>>>(plog, ns, bias, d.T, d.k, d.E, d.S, w.topk, \
                                               w.gates, w.meta + kMetaSelectCounter,       \
                                               w.offsets, w.pair, w.inv, w.rtok, w.meta,   \
                                               reinterpret_cast<int4*>(w.gdesc), w.tiles,  \
                                               tile_rows)
  if (nv <= 1)
    MOE_SP(1);
  else if (nv <= 2)
    MOE_SP(2);
  else if (nv <= 4)
    MOE_SP(4);
  else
    MOE_SP(8);
#undef MOE_SP
  return hipGetLastError();
}

hipError_t launch_permute(const Dims& d, const int32_t* topk, const Work& w, int tile_rows,
                          hipStream_t s) {
  if (d.E <= 512) {
    const size_t lds = (size_t)(16 * d.E + d.E + 64) * sizeof(int32_t);
    permute_kernel<16><<<1, 1024, lds, s>>>(topk, d.T, d.k, d.E, d.S, w.offsets, w.pair, w.inv,
                                            w.rtok, w.meta, reinterpret_cast<int4*>(w.gdesc),
                                            w.tiles, tile_rows);
  } else {
    const size_t lds = (size_t)(8 * d.E + d.E + 64) * sizeof(int32_t);
    permute_kernel<8><<<1, 512, lds, s>>>(topk, d.T, d.k, d.E, d.S, w.offsets, w.pair, w.inv,
                                          w.rtok, w.meta, reinterpret_cast<int4*>(w.gdesc),
                                          w.tiles, tile_rows);
  }
  return hipGetLastError();
}

}  // namespace moe
