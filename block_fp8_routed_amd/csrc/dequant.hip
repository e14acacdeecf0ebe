// dequant.hip — moe_dequant_e4m3: expand a block-FP8 matrix to fp32.
//
// out[r][c] = dec(w[r][c]) * scales[r / B][c / B], the block-FP8 (E4M3)
// weight format of the colizig page ("Features", "Status"). It uses the same
// in-register decode (e4m3x4_to_f32) as the expert kernels, so checking it
// against a host decode checks the kernels' view of every code and of the
// scale grid. Each thread expands 16 consecutive bytes of one row.
#include "device.hpp"
#include "layer.hpp"

namespace moe {

__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ w,
                                                     const float* __restrict__ scales,
                                                     int64_t rows, int cols, int block,
                                                     float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // 16-byte chunk index
  const int per_row = cols / 16;
  if (i >= rows * per_row) return;
  const int64_t r = i / per_row;
  const int c = (int)(i - r * per_row) * 16;
  const uint4 q = ld16(w + r * cols + c);
  float d[16];
  e4m3x4_to_f32(q.x, d);
  e4m3x4_to_f32(q.y, d + 4);
  e4m3x4_to_f32(q.z, d + 8);
  e4m3x4_to_f32(q.w, d + 12);
  const float* srow = scales + (r / block) * (cols / block);
  float* o = out + r * cols + c;
#pragma unroll
  for (int j = 0; j < 16; ++j) o[j] = d[j] * srow[(c + j) / block];
}

}  // namespace moe

extern "C" moe_status moe_dequant_e4m3(const uint8_t* w, const float* scales, int64_t rows,
                                       int32_t cols, int32_t block, float* out, void* stream) {
  if (!w || !scales || !out) return MOE_ERR_NULL;
  if (rows < 0 || cols <= 0 || block <= 0 || rows % block != 0 || cols % block != 0)
    return MOE_ERR_SHAPE;
  if (cols % 16 != 0) return MOE_ERR_UNSUPPORTED;
  if (rows == 0) return MOE_OK;
  const int64_t chunks = rows * (cols / 16);
  const dim3 grid((unsigned)((chunks + 255) / 256));
  moe::dequant_kernel<<<grid, 256, 0, static_cast<hipStream_t>(stream)>>>(w, scales, rows, cols,
                                                                          block, out);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}
