// pack.hip -- canonical MXFP4 <-> packed device layout (see common.h).
//
// A one-time load transformation: the gfx90a report (§5.2) applies its W2
// output permutation to raw weights and scales once at load, with no decode
// hot-path cost, and (§5.3) warns that shuffled scales must be consumed
// through the matching address map.  Here the map is fixed by PackedDims and
// both directions are bit-exact inverses.
#include "common.h"

namespace moe {

// One thread per packed nibble dword: (pr, slot, lane = 16 j + r, g) -> bytes
// 4g..4g+3 of row r's block j of the chunk.
__global__ void pack_nibbles_kernel(const uint8_t* __restrict__ codes, int64_t ld_codes,
                                    int n_out, int d_in, int interleave, int64_t n_words,
                                    uint32_t* __restrict__ dst) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_words) return;
  const int64_t kcn = d_in / kChunkK;
  const int g = (int)(i & 3);
  const int lane = (int)((i >> 2) & 63);
  const int64_t tile = i >> 8;  // pr * KC + storage slot
  const int kc = slot_chunk((int)(tile % kcn), (int)kcn);
  const int pr = (int)(tile / kcn);
  const int row = packed_group_src_row(pr, n_out, interleave) + (lane & 15);
  const int64_t byte = ((int64_t)kc * kChunkK + (lane >> 4) * kBlock) / 2 + 4 * g;
  dst[i] = *(const uint32_t*)(codes + (int64_t)row * ld_codes + byte);
}

__global__ void unpack_nibbles_kernel(const uint32_t* __restrict__ src, int n_out, int d_in,
                                      int interleave, int64_t n_words,
                                      uint8_t* __restrict__ codes, int64_t ld_codes) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_words) return;
  const int64_t kcn = d_in / kChunkK;
  const int g = (int)(i & 3);
  const int lane = (int)((i >> 2) & 63);
  const int64_t tile = i >> 8;
  const int kc = slot_chunk((int)(tile % kcn), (int)kcn);
  const int pr = (int)(tile / kcn);
  const int row = packed_group_src_row(pr, n_out, interleave) + (lane & 15);
  const int64_t byte = ((int64_t)kc * kChunkK + (lane >> 4) * kBlock) / 2 + 4 * g;
  *(uint32_t*)(codes + (int64_t)row * ld_codes + byte) = src[i];
}

// One thread per packed scale byte: (pr, s, r, b).
__global__ void pack_scales_kernel(const uint8_t* __restrict__ scales, int64_t ld_scales,
                                   int n_out, int d_in, int interleave, int64_t n_bytes,
                                   uint8_t* __restrict__ dst) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_bytes) return;
  const int64_t scn = (d_in / kBlock + kSuperBlocks - 1) / kSuperBlocks;
  const int b = (int)(i & 15);
  const int r = (int)((i >> 4) & 15);
  const int64_t t = i >> 8;
  const int s = (int)(t % scn);
  const int pr = (int)(t / scn);
  const int blk = s * kSuperBlocks + b;
  const int row = packed_group_src_row(pr, n_out, interleave) + r;
  dst[i] = (blk < d_in / kBlock) ? scales[(int64_t)row * ld_scales + blk] : (uint8_t)0;
}

__global__ void unpack_scales_kernel(const uint8_t* __restrict__ src, int n_out, int d_in,
                                     int interleave, int64_t n_bytes,
                                     uint8_t* __restrict__ scales, int64_t ld_scales) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_bytes) return;
  const int64_t scn = (d_in / kBlock + kSuperBlocks - 1) / kSuperBlocks;
  const int b = (int)(i & 15);
  const int r = (int)((i >> 4) & 15);
  const int64_t t = i >> 8;
  const int s = (int)(t % scn);
  const int pr = (int)(t / scn);
  const int blk = s * kSuperBlocks + b;
  const int row = packed_group_src_row(pr, n_out, interleave) + r;
  if (blk < d_in / kBlock) scales[(int64_t)row * ld_scales + blk] = src[i];
}

static int check_matrix(int n_out, int d_in, int interleave) {
  if (n_out <= 0 || d_in <= 0) return MOE_ERR_SHAPE;
  if (n_out % kRowsPerGroup || d_in % kChunkK) return MOE_ERR_SHAPE;
  if (interleave != 0 && interleave != 1) return MOE_ERR_INVALID_ARG;
  if (interleave && (n_out % (2 * kRowsPerGroup))) return MOE_ERR_SHAPE;
  return MOE_OK;
}

}  // namespace moe

using namespace moe;

extern "C" size_t moe_packed_bytes(int n_out, int d_in) {
  if (check_matrix(n_out, d_in, 0) != MOE_OK) return 0;
  return (size_t)PackedDims(n_out, d_in).total();
}

extern "C" int moe_pack_mxfp4(const uint8_t* codes, int64_t ld_codes, const uint8_t* scales,
                              int64_t ld_scales, int n_out, int d_in, int gate_up_interleave,
                              void* dst, size_t dst_bytes, void* stream) {
  if (!codes || !scales || !dst) return MOE_ERR_INVALID_ARG;
  int rc = check_matrix(n_out, d_in, gate_up_interleave);
  if (rc != MOE_OK) return rc;
  if (ld_codes < d_in / 2 || ld_scales < d_in / kBlock) return MOE_ERR_STRIDE;
  if (!aligned(codes, 4) || ld_codes % 4 || !aligned(dst, 256)) return MOE_ERR_ALIGNMENT;
  const PackedDims pd(n_out, d_in);
  if (dst_bytes < (size_t)pd.total()) return MOE_ERR_WORKSPACE;
  if (!device_is_gfx950()) return MOE_ERR_UNSUPPORTED_ARCH;
  hipStream_t s = (hipStream_t)stream;
  const int64_t n_words = pd.nib_bytes / 4;
  hipLaunchKernelGGL(pack_nibbles_kernel, dim3((unsigned)((n_words + 255) / 256)), dim3(256), 0,
                     s, codes, ld_codes, n_out, d_in, gate_up_interleave, n_words,
                     (uint32_t*)dst);
  hipLaunchKernelGGL(pack_scales_kernel, dim3((unsigned)((pd.scale_bytes + 255) / 256)),
                     dim3(256), 0, s, scales, ld_scales, n_out, d_in, gate_up_interleave,
                     pd.scale_bytes, (uint8_t*)dst + pd.nib_bytes);
  return launch_status();
}

extern "C" int moe_unpack_mxfp4(const void* src, int n_out, int d_in, int gate_up_interleave,
                                uint8_t* codes, int64_t ld_codes, uint8_t* scales,
                                int64_t ld_scales, void* stream) {
  if (!codes || !scales || !src) return MOE_ERR_INVALID_ARG;
  int rc = check_matrix(n_out, d_in, gate_up_interleave);
  if (rc != MOE_OK) return rc;
  if (ld_codes < d_in / 2 || ld_scales < d_in / kBlock) return MOE_ERR_STRIDE;
  if (!aligned(codes, 4) || ld_codes % 4 || !aligned(src, 256)) return MOE_ERR_ALIGNMENT;
  if (!device_is_gfx950()) return MOE_ERR_UNSUPPORTED_ARCH;
  const PackedDims pd(n_out, d_in);
  hipStream_t s = (hipStream_t)stream;
  const int64_t n_words = pd.nib_bytes / 4;
  hipLaunchKernelGGL(unpack_nibbles_kernel, dim3((unsigned)((n_words + 255) / 256)), dim3(256),
                     0, s, (const uint32_t*)src, n_out, d_in, gate_up_interleave, n_words, codes,
                     ld_codes);
  hipLaunchKernelGGL(unpack_scales_kernel, dim3((unsigned)((pd.scale_bytes + 255) / 256)),
                     dim3(256), 0, s, (const uint8_t*)src + pd.nib_bytes, n_out, d_in,
                     gate_up_interleave, pd.scale_bytes, scales, ld_scales);
  return launch_status();
}
