// device.hpp — small device helpers shared by the kernels of libmoe_fp8.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Four E4M3FN bytes (little-endian in a dword) to fp32. gfx950's
// v_cvt_pk_f32_fp8 decodes the OCP E4M3FN encoding (bias 7, no infinities,
// 0x7F/0xFF NaN); the conversion is exact.
__device__ __forceinline__ void e4m3x4_to_f32(uint32_t w, float* o) {
  f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  o[0] = lo.x;
  o[1] = lo.y;
  o[2] = hi.x;
  o[3] = hi.y;
}

// bf16 halves of a dword to fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Sum over aligned groups of W lanes (W a power of two <= 64); every lane of
// the group ends with the group's sum. The order of additions is fixed, so
// the result is reproducible.
template <int W>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = W / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// 16-byte global load through the vector memory path.
__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// Lanes of a 64-wide wave laid over rows of K bytes, 16 bytes per lane per
// load. K >= 1024: the whole wave covers 1024 bytes of one row per load and a
// lane takes CH = K/1024 chunks. K < 1024: LPR = K/16 lanes share a row and a
// load covers RPL rows (RPL = 64/LPR when that divides, else 1 with idle
// lanes). RED is the width of the lane groups whose partial sums are added.
template <int K>
struct RowMap {
  static_assert(K % 16 == 0, "row length must be a multiple of 16 bytes");
  static_assert(K < 1024 || K % 1024 == 0, "rows of 1024+ bytes must be whole KiB");
  static constexpr int LPR = K >= 1024 ? 64 : K / 16;
  static constexpr int RPL = K >= 1024 ? 1 : (64 % LPR == 0 ? 64 / LPR : 1);
  static constexpr int CH = K >= 1024 ? K / 1024 : 1;
  static constexpr int RED = (K >= 1024 || 64 % LPR != 0) ? 64 : LPR;
  __device__ static bool active(int lane) { return lane < LPR * RPL; }
  __device__ static int row(int lane) { return RPL == 1 ? 0 : lane / LPR; }
  __device__ static int col(int lane, int c) {
    return K >= 1024 ? 16 * lane + 1024 * c : 16 * (lane % LPR);
  }
};

}  // namespace moe
