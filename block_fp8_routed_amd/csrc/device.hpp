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

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two E4M3FN bytes (bytes 2*HI and 2*HI+1 of a dword) to a bf16 pair. Every
// E4M3FN value is a bf16 value, and with a unit scale gfx950's
// v_cvt_scalef32_pk_bf16_fp8 converts exactly.
template <bool HI>
__device__ __forceinline__ bf16x2_t e4m3x2_to_bf16x2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, HI);
}

// c + a.lo * b.lo + a.hi * b.hi with bf16 inputs and an fp32 accumulator
// (v_dot2c_f32_bf16); b is a dword holding two bf16 values.
__device__ __forceinline__ float dot2_bf16(bf16x2_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(a, __builtin_bit_cast(bf16x2_t, b), c, false);
}

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// Two E4M3FN bytes to an fp16 pair (exact: every E4M3FN value is an fp16 value).
template <bool HI>
__device__ __forceinline__ f16x2_t e4m3x2_to_f16x2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w, 1.0f, HI);
}

// c + a.lo * b.lo + a.hi * b.hi with fp16 inputs and an fp32 accumulator
// (v_dot2c_f32_f16); b is a dword holding two fp16 values.
__device__ __forceinline__ float dot2_f16(f16x2_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(a, __builtin_bit_cast(f16x2_t, b), c, false);
}

// fp32 -> fp16 bits, round to nearest even (callers keep |v| below 2^15).
__device__ __forceinline__ uint16_t f32_to_f16(float v) {
  return __builtin_bit_cast(uint16_t, (_Float16)v);
}

// Scaled fp16 storage of the intermediates h and y. A row block of values
// whose largest magnitude is amax is stored as fp16(v * 2^-e) with one
// exponent byte e + 127 beside it, e = (binary exponent of amax) - 15, so the
// block's largest value lands in [2^14, 2^15): rounding cannot carry it past
// 2^15 < 65504, every value at least 2^-28 of amax keeps fp16's full 11-bit
// significand, and any finite fp32 range fits. e = 0 for an all-zero block;
// e is clamped to [-127, 127] (below -127 only blocks smaller than 2^-112
// lose range, and fp32 itself ends at 2^128).
constexpr int kF16ExpBias = 127;
__device__ __forceinline__ int f16_block_exponent(float amax) {
  if (!(amax > 0.f)) return 0;
  const int e = __builtin_amdgcn_frexp_expf(amax) - 15;  // amax = f 2^p, f in [0.5, 1)
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}
// value of one stored fp16 element under its block's exponent byte
__device__ __forceinline__ float f16_scaled_value(_Float16 v, uint32_t ebyte) {
  return __builtin_ldexpf((float)v, (int)ebyte - kF16ExpBias);
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

// ---- cross-lane reductions (DPP within 16-lane rows, readlane across rows) ----
// DPP controls: quad_perm [1,0,3,2] (xor 1), [2,3,0,1] (xor 2), row_half_mirror
// (lane i <-> 7-i in each 8) and row_mirror (i <-> 15-i in each 16). Applied in
// that order they leave every lane of a 16-lane row holding the row's total.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                               CTRL, 0xf, 0xf, true));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xf, 0xf, true);
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;

__device__ __forceinline__ float readlane_f(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// Sum over aligned groups of W lanes (W = 1, 2, 4, 8, 16 or 64); every lane
// of a group ends with the group's sum (for W = 64 the result is uniform).
// The order of additions is fixed, so results are reproducible.
template <int W>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(W == 1 || W == 2 || W == 4 || W == 8 || W == 16 || W == 64, "group width");
  if (W >= 2) v += dpp_f<kDppXor1>(v);
  if (W >= 4) v += dpp_f<kDppXor2>(v);
  if (W >= 8) v += dpp_f<kDppHalfMirror>(v);
  if (W >= 16) v += dpp_f<kDppMirror>(v);
  if (W == 64)
    v = (readlane_f(v, 0) + readlane_f(v, 16)) + (readlane_f(v, 32) + readlane_f(v, 48));
  return v;
}

// Sum over aligned segments of W lanes (W = 1, 2, 4, 8, 16, 32 or 64). The
// segment's last lane always holds the sum (for W <= 16 every lane of the
// segment does; W = 32 adds the even 16-lane row into the odd one with
// row_bcast:15; W = 64 is group_sum<64>). One call reduces every segment of
// the wavefront at once. Fixed order of additions.
constexpr int kDppRowBcast15 = 0x142;
template <int W>
__device__ __forceinline__ float seg_sum(float v) {
  static_assert(W == 1 || W == 2 || W == 4 || W == 8 || W == 16 || W == 32 || W == 64, "width");
  if (W == 64) return group_sum<64>(v);
  if (W >= 2) v += dpp_f<kDppXor1>(v);
  if (W >= 4) v += dpp_f<kDppXor2>(v);
  if (W >= 8) v += dpp_f<kDppHalfMirror>(v);
  if (W >= 16) v += dpp_f<kDppMirror>(v);
  if (W == 32)  // rows 1 and 3 receive lane 15 of rows 0 and 2; rows 0 and 2 keep v
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                               kDppRowBcast15, 0xA, 0xF, false));
  return v;
}

// Inclusive prefix sum over the 64 lanes of a wavefront, by DPP: row_shr 1,
// 2, 4, 8 inside each 16-lane row, then row_bcast:15 (rows 1 and 3 add the
// last lane of the row before) and row_bcast:31 (rows 2 and 3 add lane 31).
// Lanes whose DPP source is outside the row, and rows outside a row mask, add
// the zero passed as the instruction's old value.
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114,
              kDppRowShr8 = 0x118, kDppRowBcast31 = 0x143;
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr1, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr2, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr4, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr8, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowBcast15, 0xA, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowBcast31, 0xC, 0xF, false);
  return v;
}

// Wave-wide maximum of a 64-bit key, uniform on return: DPP exchanges inside
// 16-lane rows, then the row maxima are folded with row_bcast:15 / :31 into
// lane 63, which is read back. Rows outside a row mask compare against zero,
// so keys must be non-negative as unsigned (they are).
template <int CTRL, int ROWS>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t k) {
  const uint32_t lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)k, CTRL, ROWS, 0xF, false);
  const uint32_t hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(k >> 32), CTRL, ROWS, 0xF,
                                                  false);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t k) {
  uint64_t o;
  o = dpp_u64<kDppXor1, 0xF>(k);
  k = o > k ? o : k;
  o = dpp_u64<kDppXor2, 0xF>(k);
  k = o > k ? o : k;
  o = dpp_u64<kDppHalfMirror, 0xF>(k);
  k = o > k ? o : k;
  o = dpp_u64<kDppMirror, 0xF>(k);
  k = o > k ? o : k;
  o = dpp_u64<kDppRowBcast15, 0xA>(k);
  k = o > k ? o : k;
  o = dpp_u64<kDppRowBcast31, 0xC>(k);
  k = o > k ? o : k;
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)k, 63);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(k >> 32), 63);
  return ((uint64_t)hi << 32) | lo;
}

// Wave-wide maximum of a 32-bit unsigned key, uniform on return (the same
// DPP steps as wave_max_u64, one word wide). Keys must be non-negative as
// unsigned, as rows outside a row mask compare against zero.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t k) {
  k = max(k, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)k, kDppXor1, 0xF, 0xF, false));
  k = max(k, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)k, kDppXor2, 0xF, 0xF, false));
  k = max(k, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)k, kDppHalfMirror, 0xF, 0xF, false));
  k = max(k, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)k, kDppMirror, 0xF, 0xF, false));
  k = max(k, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)k, kDppRowBcast15, 0xA, 0xF, false));
  k = max(k, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)k, kDppRowBcast31, 0xC, 0xF, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)k, 63);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// 16-byte global load through the vector memory path.
__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// 16-byte non-temporal global load, for data read exactly once (expert
// weights streamed by the decode passes): it does not displace reused lines.
__device__ __forceinline__ uint4 ld16_nt(const void* p) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// 16-byte raw buffer load: base and range in a wave-uniform resource, a per-
// lane 32-bit offset and a uniform one (SGPR), so no per-lane 64-bit address
// arithmetic is needed; bytes past the range read as zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
// AUX is the instruction's cache-policy field (gfx950: bit 1 = nt, a
// non-temporal access for data read once).
template <int AUX = 0>
__device__ __forceinline__ uint4 buffer_ld16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, AUX);
  return make_uint4(v.x, v.y, v.z, v.w);
}
constexpr int kBufNonTemporal = 2;

// Loads and stores at the device's point of coherence (agent-scope relaxed
// atomics, sc1): data that one workgroup hands to another inside a kernel
// goes through these, so neither side needs a cache write-back or
// invalidation (the producer waits for its stores to complete before it
// signals; the consumer reads after it has seen the signal).
template <class T>
__device__ __forceinline__ T ld_coherent(const T* p) {
  return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <class T>
__device__ __forceinline__ void st_coherent(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint4 ld16_coherent(const void* p) {
  const uint64_t* q = reinterpret_cast<const uint64_t*>(p);
  const uint64_t a = ld_coherent(q), b = ld_coherent(q + 1);
  return make_uint4((uint32_t)a, (uint32_t)(a >> 32), (uint32_t)b, (uint32_t)(b >> 32));
}

// Workgroup barrier that orders LDS accesses only: global loads still in
// flight (streamed weights) stay in flight across it, where __syncthreads()
// would first wait for every outstanding load of the wavefront.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace moe
