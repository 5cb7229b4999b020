// router.hip -- router projection: the BF16 hidden state times BF16 router
// weights into fp32 logits (gfx90a report Fig. 1, "Router Top-6"; its Table 4
// lists the router GEMM among the steps tried as BF16 CK instances and as a
// simple LDS BF16 MFMA kernel).
//
// A product of two BF16 values is exact in fp32, so a logit depends only on
// the order of its additions, and that order is fixed (the exact-rows
// contract of the Strix Halo report): 64 partial sums, partial l folding the
// elements k = 512 j + 8 l + i (j ascending, then i = 0..7) with fused
// multiply-adds from zero, then the butterfly p[l] += p[l ^ m] for
// m = 32, 16, 8, 4, 2, 1.  Partial l is lane l of one wave, so a logit has
// the same bits whatever the number of rows or their tiling.
//
// Work split, decode rows (router_kernel): a workgroup of 4 waves takes RT
// rows, whose x it stages once in LDS (the BF16 values held as fp32, at most
// 8192 elements), and 4 experts, one per wave, a lane holding its NJ 16-byte
// pieces of the expert's weight row: 64 workgroups per row tile read the
// 2 MiB of weights of 256 experts once, every row in flight while x is staged.
#include "common.h"

namespace moe {

struct RouterArgs {
  const float* x;
  int64_t ld_x;
  const uint16_t* w;
  int64_t ld_w;
  float* logits;
  int64_t ld_l;
  int rows, d_model, n_experts;
};

// staged x per workgroup, in elements: decode tiles as fp32 (32 KiB, one
// batch of loads per thread), many-row tiles as BF16 (64 KiB)
constexpr int kDecodeXMax = 8192;
constexpr int kTileXMax = 32768;
constexpr int kStageBatch = 8;        // float4 loads a thread has in flight while staging

__device__ inline void bf16x8_unpack(const u32x4 v, float (&f)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(v[i] << 16);
    f[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
  }
}

template <int NJ>
__device__ inline void router_load_row(const RouterArgs& a, int e, int lane, u32x4 (&wv)[NJ]) {
  const uint16_t* row = a.w + (int64_t)e * a.ld_w;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int k = 512 * j + 8 * lane;
    wv[j] = k < a.d_model ? *(const u32x4*)(row + k) : u32x4{0u, 0u, 0u, 0u};
  }
}

// Decode rows: RT rows per workgroup (x staged in LDS, the BF16 values held
// as fp32), one expert per wave, NJ 512-wide pieces of d_model per lane; the
// expert's whole weight row is in flight while x is staged.
template <int RT, int NJ>
__global__ __launch_bounds__(256) void router_kernel(RouterArgs a) {
  extern __shared__ __align__(16) float xs[];  // [RT][d_model]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int D = a.d_model;
  const int t0 = blockIdx.y * RT;
  const int e = blockIdx.x * 4 + wave;

  u32x4 wv[NJ];
  if (e < a.n_experts) router_load_row<NJ>(a, e, lane, wv);

  // x rows t0 .. t0+RT rounded to BF16 (nearest, ties to even), kStageBatch
  // loads in flight per thread; rows past the end are zeros, never written
  const int q4 = D / 4, total = RT * q4;
  for (int base = tid; base < total; base += 256 * kStageBatch) {
    f32x4 v[kStageBatch];
#pragma unroll
    for (int u = 0; u < kStageBatch; ++u) {
      const int idx = base + 256 * u;
      const int t = idx / q4, c = idx - t * q4;
      v[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (idx < total && t0 + t < a.rows)
        v[u] = *(const f32x4*)(a.x + (int64_t)(t0 + t) * a.ld_x + 4 * c);
    }
#pragma unroll
    for (int u = 0; u < kStageBatch; ++u) {
      const int idx = base + 256 * u;
      if (idx < total)
        *(f32x4*)(xs + 4 * idx) = f32x4{round_bf16(v[u][0]), round_bf16(v[u][1]),
                                        round_bf16(v[u][2]), round_bf16(v[u][3])};
    }
  }
  __syncthreads();
  if (e >= a.n_experts) return;  // past the only barrier

  float acc[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) acc[t] = 0.f;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int k = 512 * j + 8 * lane;
    if (k < D) {
      float wf[8];
      bf16x8_unpack(wv[j], wf);
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const f32x4 x0 = *(const f32x4*)(xs + t * D + k);
        const f32x4 x1 = *(const f32x4*)(xs + t * D + k + 4);
        const float xf[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[t] = fmaf(xf[i], wf[i], acc[t]);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) acc[t] = acc[t] + __shfl_xor(acc[t], m, 64);
  if (lane == 0) {
#pragma unroll
    for (int t = 0; t < RT; ++t)
      if (t0 + t < a.rows) a.logits[(int64_t)(t0 + t) * a.ld_l + e] = acc[t];
  }
}

// Many rows: the same sums, organised for reuse.  A workgroup of 8 waves
// stages RT rows of x as BF16 in LDS and gives each wave 16 experts, 4 at a
// time; the wave
// walks d_model one 512-wide piece at a time (a lane's 8 elements of it), so
// one read of a row's piece feeds 4 experts and one weight piece feeds RT
// rows.  Weight pieces are loaded two pieces ahead.  A lane still folds its
// elements in ascending order, so the bits are those of router_kernel.
constexpr int kTileExperts = 4;   // experts folded together by a wave
constexpr int kTileNe = 16;       // experts per wave
constexpr int kTileWaves = 8;     // waves per workgroup (128 experts share a staged x tile)

template <int RT, int NJ>
__global__ __launch_bounds__(kTileWaves * 64, 2) void router_tile_kernel(RouterArgs a) {
  extern __shared__ __align__(16) uint16_t xb[];  // [RT][d_model] BF16
  constexpr int EB = kTileExperts;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int D = a.d_model;
  const int t0 = blockIdx.y * RT;
  const int e0 = (blockIdx.x * kTileWaves + wave) * kTileNe;
  const int e_end = min(e0 + kTileNe, a.n_experts);

  // weight piece j of experts e .. e+EB (rows past the end re-read the last)
  auto load_piece = [&](int e, int j, u32x4 (&w)[EB]) {
    const int k = 512 * j + 8 * lane;
#pragma unroll
    for (int b = 0; b < EB; ++b) {
      const uint16_t* row = a.w + (int64_t)min(e + b, a.n_experts - 1) * a.ld_w;
      w[b] = k < D ? *(const u32x4*)(row + k) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  // the (group, piece) sequence this wave walks, as one counter
  const int n_groups = e0 < e_end ? (e_end - e0 + EB - 1) / EB : 0;
  const int n_steps = n_groups * NJ;
  u32x4 w0[EB], w1[EB], w2[EB];
  if (n_steps > 0) load_piece(e0, 0, w0);
  if (n_steps > 1) load_piece(e0 + EB * (1 / NJ), 1 % NJ, w1);

  const int q4 = D / 4, total = RT * q4;
  for (int base = tid; base < total; base += kTileWaves * 64 * kStageBatch) {
    f32x4 v[kStageBatch];
#pragma unroll
    for (int u = 0; u < kStageBatch; ++u) {
      const int idx = base + kTileWaves * 64 * u;
      const int t = idx / q4, c = idx - t * q4;
      v[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (idx < total && t0 + t < a.rows)
        v[u] = *(const f32x4*)(a.x + (int64_t)(t0 + t) * a.ld_x + 4 * c);
    }
#pragma unroll
    for (int u = 0; u < kStageBatch; ++u) {
      const int idx = base + kTileWaves * 64 * u;
      if (idx < total) {
        const uint32_t b0 = __float_as_uint(round_bf16(v[u][0])) >> 16;
        const uint32_t b1 = __float_as_uint(round_bf16(v[u][1])) & 0xFFFF0000u;
        const uint32_t b2 = __float_as_uint(round_bf16(v[u][2])) >> 16;
        const uint32_t b3 = __float_as_uint(round_bf16(v[u][3])) & 0xFFFF0000u;
        *(u32x2*)(xb + 4 * idx) = u32x2{b0 | b1, b2 | b3};
      }
    }
  }
  __syncthreads();

  float acc[EB][RT];
  for (int st = 0; st < n_steps; ++st) {
    const int g = st / NJ, j = st - g * NJ;
    const int e = e0 + EB * g;
    if (j == 0) {
#pragma unroll
      for (int b = 0; b < EB; ++b)
#pragma unroll
        for (int t = 0; t < RT; ++t) acc[b][t] = 0.f;
    }
    if (st + 2 < n_steps) {
      const int g2 = (st + 2) / NJ;
      load_piece(e0 + EB * g2, (st + 2) - g2 * NJ, w2);
    }
    const int k = 512 * j + 8 * lane;
    if (k < D) {
      float wf[EB][8];
#pragma unroll
      for (int b = 0; b < EB; ++b) bf16x8_unpack(w0[b], wf[b]);
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        float xf[8];
        bf16x8_unpack(*(const u32x4*)(xb + t * D + k), xf);
#pragma unroll
        for (int b = 0; b < EB; ++b)
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[b][t] = fmaf(xf[i], wf[b][i], acc[b][t]);
      }
    }
    if (j == NJ - 1) {
#pragma unroll
      for (int b = 0; b < EB; ++b)
#pragma unroll
        for (int t = 0; t < RT; ++t)
#pragma unroll
          for (int m = 32; m >= 1; m >>= 1)
            acc[b][t] = acc[b][t] + __shfl_xor(acc[b][t], m, 64);
      if (lane == 0) {
#pragma unroll
        for (int b = 0; b < EB; ++b)
#pragma unroll
          for (int t = 0; t < RT; ++t)
            if (t0 + t < a.rows && e + b < e_end)
              a.logits[(int64_t)(t0 + t) * a.ld_l + e + b] = acc[b][t];
      }
    }
#pragma unroll
    for (int b = 0; b < EB; ++b) {
      w0[b] = w1[b];
      w1[b] = w2[b];
    }
  }
}

int router_args_check(const float* x, int64_t ld_x, int rows, int d_model, const void* w_router,
                      int64_t ld_w, int n_experts, const float* logits, int64_t ld_l) {
  if (rows < 0) return MOE_ERR_INVALID_ARG;
  if (d_model <= 0 || d_model % 32 || d_model > 8192) return MOE_ERR_SHAPE;
  if (n_experts < 1 || n_experts > 4096) return MOE_ERR_SHAPE;
  if (ld_x < d_model || ld_w < d_model || ld_l < n_experts) return MOE_ERR_STRIDE;
  if (rows == 0) return MOE_OK;  // nothing is read or written
  if (!x || !w_router || !logits) return MOE_ERR_INVALID_ARG;
  if (!aligned(x, 16) || ld_x % 4 || !aligned(w_router, 16) || ld_w % 8 || !aligned(logits, 4))
    return MOE_ERR_ALIGNMENT;
  return MOE_OK;
}

template <int RT>
static void launch_router_rt(const RouterArgs& a, dim3 grid, size_t lds, hipStream_t s) {
  const int nj = (a.d_model + 511) / 512;
  if (nj <= 1)
    hipLaunchKernelGGL((router_kernel<RT, 1>), grid, dim3(256), lds, s, a);
  else if (nj <= 2)
    hipLaunchKernelGGL((router_kernel<RT, 2>), grid, dim3(256), lds, s, a);
  else if (nj <= 4)
    hipLaunchKernelGGL((router_kernel<RT, 4>), grid, dim3(256), lds, s, a);
  else if (nj <= 8)
    hipLaunchKernelGGL((router_kernel<RT, 8>), grid, dim3(256), lds, s, a);
  else
    hipLaunchKernelGGL((router_kernel<RT, 16>), grid, dim3(256), lds, s, a);
}

template <int RT>
static void launch_router_tile(const RouterArgs& a, dim3 grid, size_t lds, hipStream_t s) {
  const int nj = (a.d_model + 511) / 512;
  if (nj <= 1)
    hipLaunchKernelGGL((router_tile_kernel<RT, 1>), grid, dim3(kTileWaves * 64), lds, s, a);
  else if (nj <= 2)
    hipLaunchKernelGGL((router_tile_kernel<RT, 2>), grid, dim3(kTileWaves * 64), lds, s, a);
  else if (nj <= 4)
    hipLaunchKernelGGL((router_tile_kernel<RT, 4>), grid, dim3(kTileWaves * 64), lds, s, a);
  else if (nj <= 8)
    hipLaunchKernelGGL((router_tile_kernel<RT, 8>), grid, dim3(kTileWaves * 64), lds, s, a);
  else
    hipLaunchKernelGGL((router_tile_kernel<RT, 16>), grid, dim3(kTileWaves * 64), lds, s, a);
}

// Enqueues the projection; arguments already checked by router_args_check.
// MOE_ERR_SHAPE, with nothing enqueued, past 65535 row tiles.  Decode rows
// (router_kernel): tiles of at most 8192 elements of x, one batch of loads
// per thread, every weight row of a wave loaded at once.  More rows
// (router_tile_kernel): 8-row tiles (BF16 x, at most 64 KiB), 8 waves and
// 128 experts per workgroup.
int launch_router(const float* x, int64_t ld_x, int rows, int d_model, const void* w_router,
                  int64_t ld_w, int n_experts, float* logits, int64_t ld_l, hipStream_t s) {
  if (rows == 0) return MOE_OK;
  const bool decode = rows <= MOE_MAX_DECODE_ROWS;
  int rt = decode ? (rows <= 1 ? 1 : rows <= 2 ? 2 : rows <= 4 ? 4 : 8) : 8;
  const int cap = decode ? kDecodeXMax : kTileXMax;
  while (rt > 1 && rt * d_model > cap) rt >>= 1;
  const RouterArgs a{x, ld_x, (const uint16_t*)w_router, ld_w, logits, ld_l, rows, d_model,
                     n_experts};
  const int64_t gy = ((int64_t)rows + rt - 1) / rt;
  if (gy > 65535) return MOE_ERR_SHAPE;
  const int per_wg = decode ? 4 : kTileWaves * kTileNe;  // experts per workgroup
  const dim3 grid((n_experts + per_wg - 1) / per_wg, (unsigned)gy);
  if (!decode) {
    const size_t lds = (size_t)rt * d_model * sizeof(uint16_t);
    switch (rt) {
      case 1: launch_router_tile<1>(a, grid, lds, s); break;
      case 2: launch_router_tile<2>(a, grid, lds, s); break;
      case 4: launch_router_tile<4>(a, grid, lds, s); break;
      default: launch_router_tile<8>(a, grid, lds, s); break;
    }
  } else {
    const size_t lds = (size_t)rt * d_model * sizeof(float);
    switch (rt) {
      case 1: launch_router_rt<1>(a, grid, lds, s); break;
      case 2: launch_router_rt<2>(a, grid, lds, s); break;
      case 4: launch_router_rt<4>(a, grid, lds, s); break;
      default: launch_router_rt<8>(a, grid, lds, s); break;
    }
  }
  return launch_status();
}

}  // namespace moe

using namespace moe;

extern "C" int moe_router_logits(const float* x, int64_t ld_x, int rows, int d_model,
                                 const void* w_router, int64_t ld_w, int n_experts, float* logits,
                                 int64_t ld_l, void* stream) {
  int rc = router_args_check(x, ld_x, rows, d_model, w_router, ld_w, n_experts, logits, ld_l);
  if (rc != MOE_OK || rows == 0) return rc;
  if (!device_is_gfx950()) return MOE_ERR_UNSUPPORTED_ARCH;
  return launch_router(x, ld_x, rows, d_model, w_router, ld_w, n_experts, logits, ld_l,
                       (hipStream_t)stream);
}
