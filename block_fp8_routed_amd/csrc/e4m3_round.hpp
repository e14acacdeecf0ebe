// e4m3_round.hpp — the E4M3 rounding and block-exponent rule of the FP8
// variant (activations and the SwiGLU output h), shared by the activation
// quantiser and the FP8 gate/up pass.
//
// Reading of this project (the pages describe E4M3 weights only): a block of
// 128 values gets the scale 2^e, e the smallest integer with max|v| <= 448 *
// 2^e (0 for an all-zero block, at least -127); each value becomes the
// nearest OCP E4M3FN value of v * 2^-e, ties to the even mantissa, sign kept.
#pragma once

#include "device.hpp"

namespace moe {

constexpr int kActBlock = 128;  // columns per activation scale block

// nearest E4M3FN byte to v, |v| <= 448 (ties to the even mantissa, sign kept)
__device__ __forceinline__ uint32_t e4m3_rne(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 31) << 7;
  const float a = fabsf(v);
  uint32_t code;
  if (a < 0x1p-6f) {
    // subnormal range: m * 2^-9 with m = 0 .. 8 (m = 8 is the smallest
    // normal, code 0x08)
    code = (uint32_t)__builtin_rintf(a * 512.0f);
  } else {
    int E = (int)((__float_as_uint(a) >> 23) & 0xff) - 127;  // a is a normal fp32
    const uint32_t r = (uint32_t)__builtin_rintf(__builtin_ldexpf(a, 3 - E));  // 8 .. 16
    const bool carry = r == 16;
    E += carry ? 1 : 0;
    code = ((uint32_t)(E + 7) << 3) | (carry ? 0u : r - 8);
  }
  return code | sign;
}

// smallest e >= -127 with amax <= 448 * 2^e; 0 for amax = 0
__device__ __forceinline__ int act_exponent(float amax) {
  if (amax == 0.0f) return 0;
  if (amax < 0x1p-119f) return -127;  // exponent field <= -120: the floor
  const uint32_t b = __float_as_uint(amax);
  const int E = (int)((b >> 23) & 0xff) - 127;  // amax = (1 + f) 2^E, f < 1
  // amax 2^-(E-8) = (1 + f) 256 <= 448 iff 1 + f <= 1.75 (mantissa bits 0x600000)
  return (b & 0x7fffff) <= 0x600000u ? E - 8 : E - 7;
}

// maximum over the 16 lanes of a DPP row, on every lane of the row
__device__ __forceinline__ uint32_t row16_max_u32(uint32_t k) {
  k = max(k, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)k, kDppXor1, 0xF, 0xF, false));
  k = max(k, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)k, kDppXor2, 0xF, 0xF, false));
  k = max(k, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)k, kDppHalfMirror, 0xF, 0xF, false));
  k = max(k, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)k, kDppMirror, 0xF, 0xF, false));
  return k;
}

}  // namespace moe
