// quant.hip -- per-32-block int8 activation quantiser.
//
// gfx90a report §6.1: activations are quantised online to INT8 per 32
// elements; §7.1 item 7: native HIP INT8 quantisation.  Rule (the pages
// print none; this is the library's documented reading): d = amax/127 with
// IEEE fp32 division, q = clamp(rint(x/d), -127, 127), ties to even; an
// all-zero block gives d = 0, q = 0.
//
// Memory-bound: 4 lanes per block, 8 elements (two 16-byte loads) per lane,
// so a wave reads 2 KiB contiguous per instruction pair and writes one
// 8-byte code word per lane.
#include "common.h"

namespace moe {

__global__ __launch_bounds__(256) void quant_q8_kernel(const float* __restrict__ x, int64_t ld_x,
                                                       int rows, int cols, int8_t* __restrict__ q,
                                                       int64_t ld_q, float* __restrict__ s,
                                                       int64_t ld_s) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int per_row = cols / 8;
  const int64_t total = (int64_t)rows * per_row;
  // groups of 4 lanes (one block) are either all valid or all invalid
  const bool valid = i < total;
  const int r = valid ? (int)(i / per_row) : 0;
  const int c8 = valid ? (int)(i % per_row) : 0;
  float v[8];
  if (valid) {
    const float4 a = *(const float4*)(x + (int64_t)r * ld_x + (int64_t)c8 * 8);
    const float4 b = *(const float4*)(x + (int64_t)r * ld_x + (int64_t)c8 * 8 + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = 0.f;
  }
  float m = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) m = fmaxf(m, fabsf(v[k]));
  m = fmaxf(m, __shfl_xor(m, 1, 64));
  m = fmaxf(m, __shfl_xor(m, 2, 64));
  const float d = m / 127.0f;
  uint32_t w0 = 0, w1 = 0;
  if (d != 0.f) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float qf = fminf(fmaxf(rintf(v[k] / d), -127.f), 127.f);
      const uint32_t byte = (uint32_t)((int32_t)qf) & 0xFFu;
      if (k < 4) w0 |= byte << (8 * k);
      else w1 |= byte << (8 * (k - 4));
    }
  }
  if (valid) {
    u32x2 packed = {w0, w1};
    *(u32x2*)(q + (int64_t)r * ld_q + (int64_t)c8 * 8) = packed;
    if ((c8 & 3) == 0) s[(int64_t)r * ld_s + c8 / 4] = d;
  }
}

}  // namespace moe

using namespace moe;

extern "C" int moe_quant_act_q8(const float* x, int64_t ld_x, int rows, int cols, int8_t* q,
                                int64_t ld_q, float* scales, int64_t ld_s, void* stream) {
  if (rows < 0 || cols < 0) return MOE_ERR_INVALID_ARG;
  if (cols % kBlock) return MOE_ERR_SHAPE;
  if (rows == 0 || cols == 0) return MOE_OK;
  if (!x || !q || !scales) return MOE_ERR_INVALID_ARG;
  if (ld_x < cols || ld_q < cols || ld_s < cols / kBlock) return MOE_ERR_STRIDE;
  if (!aligned(x, 16) || ld_x % 4 || !aligned(q, 8) || ld_q % 8 || !aligned(scales, 4))
    return MOE_ERR_ALIGNMENT;
  if (!device_is_gfx950()) return MOE_ERR_UNSUPPORTED_ARCH;
  const int64_t threads = (int64_t)rows * (cols / 8);
  hipLaunchKernelGGL(quant_q8_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                     (hipStream_t)stream, x, ld_x, rows, cols, q, ld_q, scales, ld_s);
  return launch_status();
}
