// quant_act.hip — moe_quantize_act_e4m3: bf16 activations to E4M3 bytes with
// one power-of-two scale per token and block of 128 columns.
//
// This is the activation side of the variant that runs both operands of both
// expert contractions in E4M3 at prefill sizes. The pages describe E4M3
// weights only (colizig page, "What this project is trying to prove":
// natively block-FP8 checkpoints); the activation side is a reading of this
// project: a block's scale is 2^e with e the smallest integer such that the
// block's largest magnitude is at most 448 * 2^e (0 for an all-zero block,
// never below -127), and each value becomes the nearest E4M3FN value of
// x * 2^-e, an exact tie going to the even mantissa, the sign kept (negative
// values that round to zero give -0). Power-of-two scales are what gfx950's
// block-scaled FP8 matrix instructions take (E8M0), so the scale can ride in
// the instruction itself.
//
// x * 2^-e is exact in fp32 (a bf16 value times a power of two), except
// below 2^-126, where fp32 rounds; such values are far below half of
// E4M3's smallest subnormal (2^-10) and give a zero code either way, so
// each code is decided exactly as an exact-arithmetic rounding would.
//
// Sixteen lanes per block (a DPP row): lane L of a row takes columns 8L ..
// 8L + 7 with one 16-byte load, and the block's largest magnitude comes from
// a four-step DPP maximum within the row over the lanes' fp32 bit patterns
// (non-negative floats order as unsigned integers).
#include "device.hpp"
#include "e4m3_round.hpp"
#include "layer.hpp"

namespace moe {

// thread i of the grid takes 16-byte chunk i (columns 8 (i % 16) .. + 7 of
// block i / 16); chunks past the end repeat the last one and store nothing
__global__ __launch_bounds__(256) void quant_act_kernel(const uint4* __restrict__ x,
                                                       int64_t nblocks,
                                                       uint2* __restrict__ codes,
                                                       uint8_t* __restrict__ exps) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t n = nblocks * (kActBlock / 8);
  const uint4 w = x[i < n ? i : n - 1];
  const uint32_t d[4] = {w.x, w.y, w.z, w.w};
  float v[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[2 * j] = bf16_lo(d[j]);
    v[2 * j + 1] = bf16_hi(d[j]);
  }
  uint32_t m = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) m = max(m, __float_as_uint(fabsf(v[j])));
  const int e = act_exponent(__uint_as_float(row16_max_u32(m)));
  uint32_t c[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) c[j] = e4m3_rne(__builtin_ldexpf(v[j], -e));
  if (i >= n) return;
  codes[i] = make_uint2(c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24),
                        c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24));
  if ((i & 15) == 0) exps[i >> 4] = (uint8_t)(e + 127);
}

hipError_t launch_quant_act(const void* x, int64_t T, int H, uint8_t* codes, uint8_t* exps,
                            hipStream_t s) {
  const int64_t nb = T * (H / kActBlock);
  const int64_t chunks = nb * (kActBlock / 8);
  quant_act_kernel<<<(unsigned)((chunks + 255) / 256), 256, 0, s>>>(
      static_cast<const uint4*>(x), nb, reinterpret_cast<uint2*>(codes), exps);
  return hipGetLastError();
}

}  // namespace moe

extern "C" moe_status moe_quantize_act_e4m3(const void* x, int64_t tokens, int32_t hidden,
                                            uint8_t* codes, uint8_t* exps, void* stream) {
  if (!x || !codes || !exps) return MOE_ERR_NULL;
  if (tokens < 0 || hidden <= 0) return MOE_ERR_SHAPE;
  if (hidden % moe::kActBlock != 0) return MOE_ERR_UNSUPPORTED;
  if (tokens * (int64_t)(hidden / moe::kActBlock) >= ((int64_t)1 << 27))
    return MOE_ERR_UNSUPPORTED;  // the grid's x dimension counts 16-byte chunks / 256
  if (tokens == 0) return MOE_OK;
  return moe::launch_quant_act(x, tokens, hidden, codes, exps, static_cast<hipStream_t>(stream)) ==
                 hipSuccess
             ? MOE_OK
             : MOE_ERR_HIP;
}
