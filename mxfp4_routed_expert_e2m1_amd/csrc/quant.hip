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
  quant_q8_thread((int64_t)blockIdx.x * blockDim.x + threadIdx.x, x, ld_x, rows, cols, q, ld_q, s,
                  ld_s);
}

int quant_args_check(const float* x, int64_t ld_x, int rows, int cols, const int8_t* q,
                     int64_t ld_q, const float* scales, int64_t ld_s) {
  if (rows < 0 || cols < 0) return MOE_ERR_INVALID_ARG;
  if (cols % kBlock) return MOE_ERR_SHAPE;
  if (rows == 0 || cols == 0) return MOE_OK;
  if (!x || !q || !scales) return MOE_ERR_INVALID_ARG;
  if (ld_x < cols || ld_q < cols || ld_s < cols / kBlock) return MOE_ERR_STRIDE;
  if (!aligned(x, 16) || ld_x % 4 || !aligned(q, 8) || ld_q % 8 || !aligned(scales, 4))
    return MOE_ERR_ALIGNMENT;
  return MOE_OK;
}

}  // namespace moe

using namespace moe;

extern "C" int moe_quant_act_q8(const float* x, int64_t ld_x, int rows, int cols, int8_t* q,
                                int64_t ld_q, float* scales, int64_t ld_s, void* stream) {
  const int rc = quant_args_check(x, ld_x, rows, cols, q, ld_q, scales, ld_s);
  if (rc != MOE_OK) return rc;
  if (rows == 0 || cols == 0) return MOE_OK;
  if (!device_is_gfx950()) return MOE_ERR_UNSUPPORTED_ARCH;
  const int64_t threads = (int64_t)rows * (cols / 8);
  hipLaunchKernelGGL(quant_q8_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                     (hipStream_t)stream, x, ld_x, rows, cols, q, ld_q, scales, ld_s);
  return launch_status();
}
