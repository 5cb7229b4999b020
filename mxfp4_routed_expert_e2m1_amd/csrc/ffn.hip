// ffn.hip -- block-scaled MXFP4 x int8 projections on the gfx950 matrix core,
// and the routed-expert FFN built from them.
//
// One projection kernel family serves the k-row matvec and both FFN passes:
//   * A workgroup owns RGW packed 16-row groups of one weight matrix and one
//     "tile" of up to 16 token columns that share the weight pass (each
//     weight byte is read once for all resident rows: Strix record, "The
//     exact-rows contract"; weight reuse across 2..16 columns: lucebox PR,
//     "Tune small HIP batches").
//   * Its W waves split the K dimension; each wave streams its K chunks of
//     all RGW row groups as contiguous 1 KiB bursts, turns every dword of 8
//     E2M1 codes into the bf16 A fragment with one FP4 converter instruction
//     per byte (the power-of-two E8M0 scale folded in exactly), and runs one
//     16x16x32 bf16 matrix-core op per 32-element block with a zero
//     accumulator.  The result is the exact block dot times 2^(u-128)
//     (gfx90a report §6.1: integer block dot, then activation and E8M0
//     scaling); the activation scale is applied with one fp32 FMA per block.
//   * Partial sums of the W waves meet in LDS and are added in wave order
//     (fixed, no atomics), then the epilogue runs: plain store (matvec,
//     down projection partials) or SwiGLU + group-32 int8 requant of the
//     intermediate (gate/up), as in the gfx90a report §8.2.
// The combine adds the per-slot fp32 partials in slot order, shared expert
// last (gfx90a report §8.2 and Table 4: fp32 partials, fixed reduction).
#include <algorithm>
#include <atomic>

#include "ffn_internal.h"

namespace moe {

enum Pass : int { PASS_MATVEC = 0, PASS_GATEUP = 1, PASS_DOWN = 2 };

constexpr int kMaxPrefillRows = 1 << 22;

// One wave's share of a projection: RGW row groups x K chunks [kc0, kc0 + n),
// accumulated into acc.  KPW > 0: exactly KPW chunks, every weight load issued
// up front (kc0 % 4 == 0 when KPW == 4, so one 16-byte load per row group
// holds the scales of all its blocks); KPW == 0: runtime chunk count with a
// one-chunk prefetch.  B/activation-scale loads run one chunk ahead.
template <int PASS, int RGW, int KPW>
__device__ inline void wave_project(const ProjArgs& p, const uint8_t* blob, int pr0, int kc0,
                                    int n_kc, int brow, f32x4 (&acc)[RGW]) {
  const int lane = lane_id();
  const int g8 = 8 * (lane >> 4);
  const u32x4* nib = (const u32x4*)blob;
  const uint8_t* scl = blob + p.nib_bytes;

  auto load_b = [&](int kc, u32x4* b, f32x4& d) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t k = (int64_t)kc * kChunkK + j * kBlock + g8;
      if (PASS == PASS_DOWN) {
        b[j] = *(const u32x4*)((const uint16_t*)p.b + (int64_t)brow * p.ld_b + k);
      } else {
        const u32x2 v = *(const u32x2*)((const int8_t*)p.b + (int64_t)brow * p.ld_b + k);
        b[j] = u32x4{v[0], v[1], 0u, 0u};
      }
    }
    d = *(const f32x4*)(p.bs + (int64_t)brow * p.ld_bs + (int64_t)kc * 4);
  };
  auto compute = [&](const u32x4* a_tile, const uint32_t* s, const u32x4* b, f32x4 d) {
    u32x4 a[RGW];
#pragma unroll
    for (int g = 0; g < RGW; ++g) a[g] = tile_to_bf16_frags(a_tile[g]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf16x8 bb;
      if (PASS == PASS_DOWN) bb = __builtin_bit_cast(bf16x8, b[j]);
      else bb = i8x8_to_bf16x8(u32x2{b[j][0], b[j][1]});
#pragma unroll
      for (int g = 0; g < RGW; ++g) {
        const float sc = e8m0_to_f32((s[g] >> (8 * j)) & 0xFFu);
        const f32x4 r = mfma_block(fp4x8_to_bf16x8(a[g][j], sc), bb);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[g][i] = fmaf(r[i], d[j], acc[g][i]);
      }
    }
  };

  if constexpr (KPW > 0) {
    u32x4 a[KPW][RGW];
#pragma unroll
    for (int kk = 0; kk < KPW; ++kk)
#pragma unroll
      for (int g = 0; g < RGW; ++g)
        a[kk][g] = nib[((int64_t)(pr0 + g) * p.kc_total + chunk_slot(kc0 + kk, p.kc_total)) * 64 + lane];
    uint32_t s[KPW][RGW];
    if constexpr (KPW == 4) {
#pragma unroll
      for (int g = 0; g < RGW; ++g) {
        const u32x4 sv = *(const u32x4*)(scl + (((int64_t)(pr0 + g) * p.sc_total + (kc0 >> 2)) * 16 +
                                                (lane & 15)) * 16);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) s[kk][g] = sv[kk];
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < KPW; ++kk)
#pragma unroll
        for (int g = 0; g < RGW; ++g) {
          const int kc = kc0 + kk;
          s[kk][g] = *(const uint32_t*)(scl + (((int64_t)(pr0 + g) * p.sc_total + (kc >> 2)) * 16 +
                                               (lane & 15)) * 16 + (kc & 3) * 4);
        }
    }
    u32x4 b[2][4];
    f32x4 d[2];
    load_b(kc0, b[0], d[0]);
#pragma unroll
    for (int kk = 0; kk < KPW; ++kk) {
      if (kk + 1 < KPW) load_b(kc0 + kk + 1, b[(kk + 1) & 1], d[(kk + 1) & 1]);
      compute(a[kk], s[kk], b[kk & 1], d[kk & 1]);
    }
  } else {
    u32x4 a_cur[RGW], a_nxt[RGW], b_cur[4], b_nxt[4];
    uint32_t s_cur[RGW], s_nxt[RGW];
    f32x4 d_cur, d_nxt;
    auto load_a = [&](int kc, u32x4* a, uint32_t* s) {
#pragma unroll
      for (int g = 0; g < RGW; ++g) {
        a[g] = nib[((int64_t)(pr0 + g) * p.kc_total + chunk_slot(kc, p.kc_total)) * 64 + lane];
        s[g] = *(const uint32_t*)(scl + (((int64_t)(pr0 + g) * p.sc_total + (kc >> 2)) * 16 +
                                         (lane & 15)) * 16 + (kc & 3) * 4);
      }
    };
    if (n_kc > 0) {
      load_a(kc0, a_cur, s_cur);
      load_b(kc0, b_cur, d_cur);
    }
    for (int kc = kc0; kc < kc0 + n_kc; ++kc) {
      if (kc + 1 < kc0 + n_kc) {
        load_a(kc + 1, a_nxt, s_nxt);
        load_b(kc + 1, b_nxt, d_nxt);
      }
      compute(a_cur, s_cur, b_cur, d_cur);
#pragma unroll
      for (int g = 0; g < RGW; ++g) {
        a_cur[g] = a_nxt[g];
        s_cur[g] = s_nxt[g];
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) b_cur[j] = b_nxt[j];
      d_cur = d_nxt;
    }
  }
}

// 4 waves per SIMD (<= 128 VGPRs) keeps two 8-wave workgroups resident per CU.
template <int PASS, int W, int RGW, int KPW>
__global__ __launch_bounds__(W * 64, 4) void proj_kernel(ProjArgs p) {
  static_assert(PASS != PASS_GATEUP || RGW == 4, "gate/up needs 2 gate/up pairs = 32 features");
  __shared__ float red[W][RGW * 4][64];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int n_rb = p.rg_total / RGW;
  const int rb = blockIdx.x % n_rb;
  const int tile_idx = blockIdx.x / n_rb;

  Tile t;
  int n_tiles = 1;
  if (PASS == PASS_MATVEC) {
    t.expert = 0;
    t.start = 0;
    t.count = p.rows;
  } else {
    t = find_tile(p.offsets, p.n_experts, p.has_shared, p.rows, tile_idx, &n_tiles);
  }
  if (t.expert < 0) return;  // the same for every wave of the workgroup
  const bool shared = (PASS != PASS_MATVEC) && t.expert == p.n_experts;
  const uint8_t* blob = (PASS == PASS_MATVEC) ? p.w
                        : shared             ? p.w_shared
                                             : p.w + (int64_t)t.expert * p.w_stride;
  const int n_tok_assign = p.rows * p.top_k;

  // B row of this lane's column (columns past the tile repeat column 0)
  const int col = lane & 15;
  const int ccol = col < t.count ? col : 0;
  int brow;
  if (PASS == PASS_MATVEC) brow = ccol;
  else if (PASS == PASS_GATEUP) brow = shared ? t.start + ccol : p.sorted[t.start + ccol] / p.top_k;
  else brow = shared ? n_tok_assign + t.start + ccol : t.start + ccol;

  const int pr0 = rb * RGW;
  f32x4 acc[RGW];
#pragma unroll
  for (int g = 0; g < RGW; ++g) acc[g] = f32x4{0.f, 0.f, 0.f, 0.f};
  if constexpr (KPW > 0) {
    wave_project<PASS, RGW, KPW>(p, blob, pr0, wave * KPW, KPW, brow, acc);
  } else {
    const int kc0 = wave * p.kc_total / W;
    const int kc1 = (wave + 1) * p.kc_total / W;
    wave_project<PASS, RGW, 0>(p, blob, pr0, kc0, kc1 - kc0, brow, acc);
  }

  // cross-wave reduction, fixed wave order
#pragma unroll
  for (int g = 0; g < RGW; ++g)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][g * 4 + i][lane] = acc[g][i];
  __syncthreads();
  for (int e = threadIdx.x; e < RGW * 4 * 64; e += W * 64) {
    float v = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < W; ++w2) v += red[w2][e >> 6][e & 63];
    red[0][e >> 6][e & 63] = v;
  }
  __syncthreads();

  if (PASS != PASS_GATEUP) {
    for (int e = threadIdx.x; e < RGW * 4 * 64; e += W * 64) {
      const int gi = e >> 6, l = e & 63;
      const int n = l & 15;
      if (n >= t.count) continue;
      const int row = (pr0 + (gi >> 2)) * 16 + 4 * (l >> 4) + (gi & 3);
      int orow;
      if (PASS == PASS_MATVEC) orow = n;
      else orow = shared ? n_tok_assign + t.start + n : p.sorted[t.start + n];
      p.y[(int64_t)orow * p.ld_y + row] = red[0][gi][l];
    }
  } else {
    // SwiGLU + requant of 32 features x up to 16 columns; a group of 32
    // consecutive threads holds one column, so its amax is a 32-lane reduce.
    const int f0 = rb * 32;
    for (int pidx = threadIdx.x; pidx < 16 * 32; pidx += W * 64) {
      const int n = pidx >> 5, f = pidx & 31;
      const int gsel = 2 * (f >> 4);  // packed group of the gate value
      const int l = 16 * ((f & 15) >> 2) + n;
      const float gv = red[0][gsel * 4 + (f & 3)][l];
      const float uv = red[0][(gsel + 1) * 4 + (f & 3)][l];
      const float hv = mid_round(swiglu(gv, uv), p.bf16_mid);
      const float d = max32(fabsf(hv)) / 127.0f;
      const float qf = q8_code(hv, d);
      if (n < t.count) {
        const int64_t hrow = shared ? n_tok_assign + t.start + n : t.start + n;
        p.h[hrow * p.ld_h + f0 + f] = (uint16_t)(__float_as_uint(qf) >> 16);
        if (f == 0) p.hs[hrow * p.ld_hs + (f0 >> 5)] = d;
      }
    }
  }
}

// y[t] = sum_i w[t][i] * P[t*k+i] (slots with ids < 0 skipped) + P[shared t]
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ P,
                                                      const int32_t* __restrict__ ids,
                                                      const float* __restrict__ w, int rows,
                                                      int top_k, int has_shared, int d_model,
                                                      float* __restrict__ y, int64_t ld_y) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int per_row = d_model / 4;
  if (i >= (int64_t)rows * per_row) return;
  const int t = (int)(i / per_row);
  const int c = (int)(i % per_row) * 4;
  // y = fma over the slots in slot order from 0, then + the shared expert's
  // partial: the one order every decode path uses (exact rows)
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < top_k; ++s) {
    const int64_t a = (int64_t)t * top_k + s;
    if (ids[a] < 0) continue;
    const float wa = w[a];
    const f32x4 pa = *(const f32x4*)(P + a * d_model + c);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = fmaf(wa, pa[i], acc[i]);
  }
  if (has_shared) acc += *(const f32x4*)(P + ((int64_t)rows * top_k + t) * d_model + c);
  *(f32x4*)(y + (int64_t)t * ld_y + c) = acc;
}

// dots[t][n][b]: one wave per (row group, K chunk); same unpack + matrix-core
// functions as the projections with the weight scale forced to 1.
__global__ __launch_bounds__(64) void block_dots_kernel(const uint8_t* __restrict__ blob,
                                                        int n_out, int d_in,
                                                        const int8_t* __restrict__ q,
                                                        int64_t ld_q, int rows,
                                                        int32_t* __restrict__ dots) {
  const PackedDims pd(n_out, d_in);
  const int kc = blockIdx.x % pd.kc;
  const int pr = blockIdx.x / pd.kc;
  const int lane = threadIdx.x;
  const int col = lane & 15;
  const int brow = col < rows ? col : 0;
  const u32x4 a = tile_to_bf16_frags(
      ((const u32x4*)blob)[((int64_t)pr * pd.kc + chunk_slot(kc, (int)pd.kc)) * 64 + lane]);
  const int nb = d_in / kBlock;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const u32x2 v = *(const u32x2*)(q + (int64_t)brow * ld_q + (int64_t)kc * kChunkK + j * kBlock +
                                    8 * (lane >> 4));
    const f32x4 r = mfma_block(fp4x8_to_bf16x8(a[j], 1.0f), i8x8_to_bf16x8(v));
    if (col < rows) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = pr * 16 + 4 * (lane >> 4) + i;
        dots[((int64_t)col * n_out + row) * nb + kc * 4 + j] = (int32_t)(r[i] * 2.0f);
      }
    }
  }
}

// ------------------------------------------------------------------ host
// K split: KPW = 4 chunks per wave when K/128 is 8, 16 or 32 (W = 2..8 waves),
// otherwise a runtime split over W = min(8, K/128) waves.
template <int PASS, int RGW>
static void launch_proj(const ProjArgs& a, int tiles, hipStream_t s) {
  const unsigned grid = (unsigned)((int64_t)tiles * (a.rg_total / RGW));
  switch (a.kc_total) {
    case 32:
      hipLaunchKernelGGL((proj_kernel<PASS, 8, RGW, 4>), dim3(grid), dim3(512), 0, s, a);
      return;
    case 16:
      hipLaunchKernelGGL((proj_kernel<PASS, 4, RGW, 4>), dim3(grid), dim3(256), 0, s, a);
      return;
    case 8:
      hipLaunchKernelGGL((proj_kernel<PASS, 2, RGW, 4>), dim3(grid), dim3(128), 0, s, a);
      return;
    default:
      break;
  }
  if (a.kc_total >= 8)
    hipLaunchKernelGGL((proj_kernel<PASS, 8, RGW, 0>), dim3(grid), dim3(512), 0, s, a);
  else if (a.kc_total >= 4)
    hipLaunchKernelGGL((proj_kernel<PASS, 4, RGW, 0>), dim3(grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((proj_kernel<PASS, 2, RGW, 0>), dim3(grid), dim3(128), 0, s, a);
}

static int check_layer(const moe_layer_t* L) {
  if (!L) return MOE_ERR_INVALID_ARG;
  if (L->d_model <= 0 || L->d_ff <= 0 || L->d_model % kChunkK || L->d_ff % kChunkK)
    return MOE_ERR_SHAPE;
  if (L->n_experts < 1 || L->n_experts > 512) return MOE_ERR_SHAPE;
  if (L->top_k < 1 || L->top_k > L->n_experts || L->top_k > MOE_MAX_TOP_K) return MOE_ERR_SHAPE;
  if (L->has_shared != 0 && L->has_shared != 1) return MOE_ERR_INVALID_ARG;
  if (!L->gate_up || !L->down) return MOE_ERR_INVALID_ARG;
  if (L->flags & ~MOE_LAYER_BF16_INTERMEDIATE) return MOE_ERR_INVALID_ARG;
  if (L->has_shared && (!L->shared_gate_up || !L->shared_down)) return MOE_ERR_INVALID_ARG;
  const int64_t gu = PackedDims(2 * L->d_ff, L->d_model).total();
  const int64_t dn = PackedDims(L->d_model, L->d_ff).total();
  if (L->n_experts > 1 && (L->gate_up_stride < gu || L->down_stride < dn)) return MOE_ERR_STRIDE;
  if (L->gate_up_stride % 256 || L->down_stride % 256) return MOE_ERR_ALIGNMENT;
  if (!aligned(L->gate_up, 256) || !aligned(L->down, 256)) return MOE_ERR_ALIGNMENT;
  if (L->has_shared && (!aligned(L->shared_gate_up, 256) || !aligned(L->shared_down, 256)))
    return MOE_ERR_ALIGNMENT;
  if (L->router) {
    if (L->d_model > 8192) return MOE_ERR_SHAPE;
    if (L->router_ld < L->d_model) return MOE_ERR_STRIDE;
    if (!aligned(L->router, 16) || L->router_ld % 8) return MOE_ERR_ALIGNMENT;
  }
  return MOE_OK;
}

static int check_acts(const int8_t* q, int64_t ld_q, const float* qs, int64_t ld_qs, int cols,
                      float* y, int64_t ld_y, int ycols) {
  if (!q || !qs || !y) return MOE_ERR_INVALID_ARG;
  if (ld_q < cols || ld_qs < cols / kBlock || ld_y < ycols) return MOE_ERR_STRIDE;
  if (!aligned(q, 8) || ld_q % 8 || !aligned(qs, 16) || ld_qs % 4 || !aligned(y, 16) ||
      ld_y % 4)
    return MOE_ERR_ALIGNMENT;
  return MOE_OK;
}

void launch_combine(const float* P, const int32_t* ids, const float* w, int rows, int top_k,
                    int has_shared, int d_model, float* y, int64_t ld_y, hipStream_t s) {
  const int64_t threads = (int64_t)rows * (d_model / 4);
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, P,
                     ids, w, rows, top_k, has_shared, d_model, y, ld_y);
}

// Arguments of the gate/up projection of one call (workspace regions
// included).
static ProjArgs gateup_args(const moe_layer_t* L, const int8_t* q, int64_t ld_q, const float* qs,
                            int64_t ld_qs, int rows, const int32_t* offsets,
                            const int32_t* sorted, void* ws) {
  const WsLayout lay = ws_layout(L, rows);
  uint8_t* base = (uint8_t*)ws;
  const PackedDims pd(2 * L->d_ff, L->d_model);
  ProjArgs g{};
  g.offsets = offsets;
  g.sorted = sorted;
  g.n_experts = L->n_experts;
  g.top_k = L->top_k;
  g.has_shared = L->has_shared;
  g.rows = rows;
  g.w = (const uint8_t*)L->gate_up;
  g.w_stride = L->gate_up_stride;
  g.w_shared = (const uint8_t*)L->shared_gate_up;
  g.nib_bytes = pd.nib_bytes;
  g.rg_total = (int)pd.rg;
  g.kc_total = (int)pd.kc;
  g.sc_total = (int)pd.sc;
  g.b = q;
  g.ld_b = ld_q;
  g.bs = qs;
  g.ld_bs = ld_qs;
  g.h = (uint16_t*)(base + lay.hidden);
  g.hs = (float*)(base + lay.hidden_scales);
  g.ld_h = L->d_ff;
  g.ld_hs = L->d_ff / kBlock;
  g.bf16_mid = (L->flags & MOE_LAYER_BF16_INTERMEDIATE) != 0;
  return g;
}

static int ffn_run(const moe_layer_t* L, bool decode, int stages, const int8_t* q,
                   int64_t ld_q, const float* qs, int64_t ld_qs, int rows, const int32_t* ids,
                   const float* w, const int32_t* offsets, const int32_t* sorted, float* y,
                   int64_t ld_y, void* ws, hipStream_t s) {
  const WsLayout lay = ws_layout(L, rows);
  uint8_t* base = (uint8_t*)ws;
  const int A = rows * L->top_k;
  const int tiles = std::min(L->n_experts, A) + (A + 15) / 16 +
                    (L->has_shared ? (rows + 15) / 16 : 0);

  ProjArgs a{};
  a.offsets = offsets;
  a.sorted = sorted;
  a.n_experts = L->n_experts;
  a.top_k = L->top_k;
  a.has_shared = L->has_shared;
  a.rows = rows;

  // gate/up + SwiGLU + requant
  if (stages & MOE_STAGE_GATE_UP) {
    const ProjArgs g = gateup_args(L, q, ld_q, qs, ld_qs, rows, offsets, sorted, ws);
    if (decode && stream_supported(g.kc_total, g.rg_total)) launch_stream(STREAM_GATEUP, g, tiles, s);
    else launch_proj<PASS_GATEUP, 4>(g, tiles, s);
  }
  // down projection -> per-slot partials -> fixed-order combine into y
  if ((stages & MOE_STAGE_DOWN) && decode && down_rows_supported(L, rows)) {
    const int rc = down_rows_run(L, rows, ids, w, offsets, sorted,
                                 (const uint16_t*)(base + lay.hidden),
                                 (const float*)(base + lay.hidden_scales), y, ld_y, s);
    if (rc != MOE_OK) return rc;
  } else if (stages & MOE_STAGE_DOWN) {
    const PackedDims pd(L->d_model, L->d_ff);
    ProjArgs d = a;
    d.w = (const uint8_t*)L->down;
    d.w_stride = L->down_stride;
    d.w_shared = (const uint8_t*)L->shared_down;
    d.nib_bytes = pd.nib_bytes;
    d.rg_total = (int)pd.rg;
    d.kc_total = (int)pd.kc;
    d.sc_total = (int)pd.sc;
    d.b = base + lay.hidden;
    d.ld_b = L->d_ff;
    d.bs = (const float*)(base + lay.hidden_scales);
    d.ld_bs = L->d_ff / kBlock;
    d.y = (float*)(base + lay.partials);
    d.ld_y = L->d_model;
    if (decode && stream_supported(d.kc_total, d.rg_total)) launch_stream(STREAM_DOWN, d, tiles, s);
    else launch_proj<PASS_DOWN, 4>(d, tiles, s);
    launch_combine((const float*)(base + lay.partials), ids, w, rows, L->top_k, L->has_shared,
                   L->d_model, y, ld_y, s);
  }
  return launch_status();
}

static int ffn_entry(const moe_layer_t* L, bool decode, int stages, const int8_t* q,
                     int64_t ld_q, const float* qs, int64_t ld_qs, int rows, const int32_t* ids,
                     const float* w, const int32_t* offsets, const int32_t* sorted, float* y,
                     int64_t ld_y, void* ws, size_t ws_bytes, void* stream) {
  const int max_rows = decode ? MOE_MAX_DECODE_ROWS : kMaxPrefillRows;
  if ((stages & MOE_STAGE_ALL) == 0 || (stages & ~(MOE_STAGE_ALL | MOE_STAGE_REUSE_ACTS)))
    return MOE_ERR_INVALID_ARG;
  if ((stages & MOE_STAGE_REUSE_ACTS) && (decode || !(stages & MOE_STAGE_GATE_UP)))
    return MOE_ERR_INVALID_ARG;
  int rc = check_layer(L);
  if (rc != MOE_OK) return rc;
  if (rows < 1 || rows > max_rows) return MOE_ERR_SHAPE;
  if ((int64_t)rows * (L->top_k + 1) > (1 << 24)) return MOE_ERR_SHAPE;
  if (!ids || !w || !offsets || !sorted || !ws) return MOE_ERR_INVALID_ARG;
  rc = check_acts(q, ld_q, qs, ld_qs, L->d_model, y, ld_y, L->d_model);
  if (rc != MOE_OK) return rc;
  if (!aligned(ws, 256)) return MOE_ERR_ALIGNMENT;
  if (ws_bytes < ws_layout(L, rows).total) return MOE_ERR_WORKSPACE;
  if (!device_is_gfx950()) return MOE_ERR_UNSUPPORTED_ARCH;
  // the prefill GEMM works in 256-row weight blocks; other shapes use the tiles
  if (!decode && L->d_model % 256 == 0 && (2 * L->d_ff) % 256 == 0)
    return prefill_run(L, stages, q, ld_q, qs, ld_qs, rows, ids, w, offsets, sorted, y, ld_y, ws,
                       (hipStream_t)stream);
  return ffn_run(L, decode, stages, q, ld_q, qs, ld_qs, rows, ids, w, offsets, sorted, y, ld_y,
                 ws, (hipStream_t)stream);
}

}  // namespace moe

using namespace moe;

extern "C" size_t moe_ffn_workspace_bytes(const moe_layer_t* L, int rows) {
  if (check_layer(L) != MOE_OK || rows < 0) return 0;
  return ws_layout(L, rows).total;
}

extern "C" int moe_ffn_workspace_layout(const moe_layer_t* L, int rows, size_t* off_hidden,
                                        size_t* off_hidden_scales, size_t* off_partials) {
  const int rc = check_layer(L);
  if (rc != MOE_OK) return rc;
  if (rows < 0) return MOE_ERR_INVALID_ARG;
  const WsLayout w = ws_layout(L, rows);
  if (off_hidden) *off_hidden = w.hidden;
  if (off_hidden_scales) *off_hidden_scales = w.hidden_scales;
  if (off_partials) *off_partials = w.partials;
  return MOE_OK;
}

extern "C" int moe_ffn_decode(const moe_layer_t* L, const int8_t* q, int64_t ld_q,
                              const float* qs, int64_t ld_qs, int rows, const int32_t* ids,
                              const float* w, const int32_t* offsets, const int32_t* sorted,
                              float* y, int64_t ld_y, void* ws, size_t ws_bytes, void* stream) {
  return ffn_entry(L, true, MOE_STAGE_ALL, q, ld_q, qs, ld_qs, rows, ids, w, offsets, sorted, y,
                   ld_y, ws, ws_bytes, stream);
}

extern "C" int moe_decode_prep(const float* x, int64_t ld_x, int cols, int8_t* q, int64_t ld_q,
                               float* scales, int64_t ld_s, const float* logits, int64_t ld_l,
                               int rows, int n_experts, int top_k, int32_t* ids, float* w,
                               int32_t* counts, int32_t* offsets, int32_t* sorted, void* stream);

// Checks of a decode step from the layer input that do not involve the
// workspace or the device (MOE_OK or the first error).
static int step_args_check(const moe_layer_t* L, const float* x, int64_t ld_x,
                           const float* logits, int64_t ld_l, int rows, const int8_t* q,
                           int64_t ld_q, const float* qs, int64_t ld_qs, const int32_t* ids,
                           const float* w, const int32_t* counts, const int32_t* offsets,
                           const int32_t* sorted, float* y, int64_t ld_y) {
  int rc = check_layer(L);
  if (rc != MOE_OK) return rc;
  if (rows < 1 || rows > MOE_MAX_DECODE_ROWS) return MOE_ERR_SHAPE;
  rc = quant_args_check(x, ld_x, rows, L->d_model, q, ld_q, qs, ld_qs);
  if (rc != MOE_OK) return rc;
  rc = route_args_check(logits, ld_l, rows, L->n_experts, L->top_k, ids, w, counts, offsets,
                        sorted);
  if (rc != MOE_OK) return rc;
  if (L->router) {
    rc = router_args_check(x, ld_x, rows, L->d_model, L->router, L->router_ld, L->n_experts,
                           logits, ld_l);
    if (rc != MOE_OK) return rc;
  }
  return check_acts(q, ld_q, qs, ld_qs, L->d_model, y, ld_y, L->d_model);
}

// The launches of a validated decode step (ws: a workspace of at least
// ws_layout(L, rows).total bytes).
static int step_launch(const moe_layer_t* L, int stages, const float* x, int64_t ld_x,
                       float* logits, int64_t ld_l, int rows, int8_t* q, int64_t ld_q, float* qs,
                       int64_t ld_qs, int32_t* ids, float* w, int32_t* counts, int32_t* offsets,
                       int32_t* sorted, float* y, int64_t ld_y, void* ws, void* stream) {
  int rc = MOE_OK;
  hipStream_t s = (hipStream_t)stream;
  if (L->router && (stages & MOE_STAGE_GATE_UP)) {
    // the router projection writes the logits the routing below reads
    rc = launch_router(x, ld_x, rows, L->d_model, L->router, L->router_ld, L->n_experts, logits,
                       ld_l, s);
    if (rc != MOE_OK) return rc;
  }
  const ProjArgs g = gateup_args(L, q, ld_q, qs, ld_qs, rows, offsets, sorted, ws);
  if (rows == 1 && stream_supported(g.kc_total, g.rg_total)) {
    // one launch quantises, routes and runs gate/up; then the down stage
    if (stages & MOE_STAGE_GATE_UP) {
      StepIn in{x, logits, q, qs, ids, w, counts, offsets, sorted};
      if ((stages & MOE_STAGE_DOWN) && down_rows_supported(L, rows)) {
        const PackedDims pd(L->d_model, L->d_ff);
        in.dn = (const uint8_t*)L->down;
        in.dn_stride = L->down_stride;
        in.dn_shared = (const uint8_t*)L->shared_down;
        in.dn_nib_bytes = pd.nib_bytes;
        in.dn_kc = (int)pd.kc;
        in.dn_sc = (int)pd.sc;
        in.dn_rg = (int)pd.rg;
      }
      launch_stream_step1(g, in, s);
    }
    if (!(stages & MOE_STAGE_DOWN)) return launch_status();
    return ffn_run(L, true, MOE_STAGE_DOWN, q, ld_q, qs, ld_qs, rows, ids, w, offsets, sorted, y,
                   ld_y, ws, s);
  }
  if (stages & MOE_STAGE_GATE_UP) {
    rc = moe_decode_prep(x, ld_x, L->d_model, q, ld_q, qs, ld_qs, logits, ld_l, rows,
                         L->n_experts, L->top_k, ids, w, counts, offsets, sorted, stream);
    if (rc != MOE_OK) return rc;
  }
  return ffn_run(L, true, stages, q, ld_q, qs, ld_qs, rows, ids, w, offsets, sorted, y, ld_y, ws,
                 s);
}

extern "C" int moe_ffn_decode_step_stages(const moe_layer_t* L, int stages, const float* x,
                                          int64_t ld_x, float* logits, int64_t ld_l,
                                          int rows, int8_t* q, int64_t ld_q, float* qs,
                                          int64_t ld_qs, int32_t* ids, float* w, int32_t* counts,
                                          int32_t* offsets, int32_t* sorted, float* y,
                                          int64_t ld_y, void* ws, size_t ws_bytes, void* stream) {
  if (stages <= 0 || stages > MOE_STAGE_ALL) return MOE_ERR_INVALID_ARG;
  const int rc = step_args_check(L, x, ld_x, logits, ld_l, rows, q, ld_q, qs, ld_qs, ids, w,
                                 counts, offsets, sorted, y, ld_y);
  if (rc != MOE_OK) return rc;
  if (!ws) return MOE_ERR_INVALID_ARG;
  if (!aligned(ws, 256)) return MOE_ERR_ALIGNMENT;
  if (ws_bytes < ws_layout(L, rows).total) return MOE_ERR_WORKSPACE;
  if (!device_is_gfx950()) return MOE_ERR_UNSUPPORTED_ARCH;
  return step_launch(L, stages, x, ld_x, logits, ld_l, rows, q, ld_q, qs, ld_qs, ids, w, counts,
                     offsets, sorted, y, ld_y, ws, stream);
}

extern "C" int moe_ffn_decode_step(const moe_layer_t* L, const float* x, int64_t ld_x,
                                   float* logits, int64_t ld_l, int rows, int8_t* q,
                                   int64_t ld_q, float* qs, int64_t ld_qs, int32_t* ids, float* w,
                                   int32_t* counts, int32_t* offsets, int32_t* sorted, float* y,
                                   int64_t ld_y, void* ws, size_t ws_bytes, void* stream) {
  return moe_ffn_decode_step_stages(L, MOE_STAGE_ALL, x, ld_x, logits, ld_l, rows, q, ld_q, qs,
                                    ld_qs, ids, w, counts, offsets, sorted, y, ld_y, ws, ws_bytes,
                                    stream);
}

// ------------------------------------------------- allocation-free entry
// Scratch memory of moe_ffn_decode_step_noalloc: the workspace of one decode
// step lives in this file-scope device array instead of a caller buffer.
// Every GPU holds its own copy at its own address until the process ends; in
// host code the array's name is not a device address, so the address is
// taken once per device (with that device current) and kept in g_scratch.
constexpr size_t kScratchBytes = size_t(8) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
static std::atomic<uintptr_t> g_scratch[64];  // device ordinal -> scratch address

static int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return MOE_ERR_HIP;
  uintptr_t p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == 0) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
      return MOE_ERR_HIP;
    p = (uintptr_t)ptr;
    g_scratch[dev].store(p, std::memory_order_release);  // racing first calls store the same
  }
  *out = (void*)p;
  return MOE_OK;
}

extern "C" int moe_ffn_decode_step_noalloc(const moe_layer_t* L, const float* x, int64_t ld_x,
                                           float* logits, int64_t ld_l, int rows, int8_t* q,
                                           int64_t ld_q, float* qs, int64_t ld_qs, int32_t* ids,
                                           float* w, int32_t* counts, int32_t* offsets,
                                           int32_t* sorted, float* y, int64_t ld_y,
                                           void* stream) {
  // the checks of moe_ffn_decode_step, the scratch size in place of the
  // workspace's, all before anything is enqueued
  int rc = step_args_check(L, x, ld_x, logits, ld_l, rows, q, ld_q, qs, ld_qs, ids, w, counts,
                           offsets, sorted, y, ld_y);
  if (rc != MOE_OK) return rc;
  if (ws_layout(L, rows).total > kScratchBytes) return MOE_ERR_WORKSPACE;
  if (!device_is_gfx950()) return MOE_ERR_UNSUPPORTED_ARCH;
  void* ws = nullptr;
  rc = scratch_address(&ws);
  if (rc != MOE_OK) return rc;
  return step_launch(L, MOE_STAGE_ALL, x, ld_x, logits, ld_l, rows, q, ld_q, qs, ld_qs, ids, w,
                     counts, offsets, sorted, y, ld_y, ws, stream);
}

extern "C" int moe_matvec_mxfp4(const void* w_packed, int n_out, int d_in, const int8_t* q,
                                int64_t ld_q, const float* qs, int64_t ld_qs, int rows, float* y,
                                int64_t ld_y, void* stream) {
  if (!w_packed) return MOE_ERR_INVALID_ARG;
  if (n_out <= 0 || d_in <= 0 || n_out % kRowsPerGroup || d_in % kChunkK) return MOE_ERR_SHAPE;
  if (rows < 1 || rows > MOE_MAX_DECODE_ROWS) return MOE_ERR_SHAPE;
  int rc = check_acts(q, ld_q, qs, ld_qs, d_in, y, ld_y, n_out);
  if (rc != MOE_OK) return rc;
  if (!aligned(w_packed, 256)) return MOE_ERR_ALIGNMENT;
  if (!device_is_gfx950()) return MOE_ERR_UNSUPPORTED_ARCH;
  const PackedDims pd(n_out, d_in);
  ProjArgs a{};
  a.w = (const uint8_t*)w_packed;
  a.nib_bytes = pd.nib_bytes;
  a.rg_total = (int)pd.rg;
  a.kc_total = (int)pd.kc;
  a.sc_total = (int)pd.sc;
  a.rows = rows;
  a.top_k = 1;
  a.b = q;
  a.ld_b = ld_q;
  a.bs = qs;
  a.ld_bs = ld_qs;
  a.y = y;
  a.ld_y = ld_y;
  hipStream_t s = (hipStream_t)stream;
  if (stream_supported(a.kc_total, a.rg_total)) launch_stream(STREAM_MATVEC, a, 1, s);
  else if (pd.rg % 2 == 0) launch_proj<PASS_MATVEC, 2>(a, 1, s);
  else launch_proj<PASS_MATVEC, 1>(a, 1, s);
  return launch_status();
}

extern "C" int moe_debug_block_dots(const void* w_packed, int n_out, int d_in, const int8_t* q,
                                    int64_t ld_q, int rows, int32_t* dots, void* stream) {
  if (!w_packed || !q || !dots) return MOE_ERR_INVALID_ARG;
  if (n_out <= 0 || d_in <= 0 || n_out % kRowsPerGroup || d_in % kChunkK) return MOE_ERR_SHAPE;
  if (rows < 1 || rows > MOE_MAX_DECODE_ROWS) return MOE_ERR_SHAPE;
  if (ld_q < d_in) return MOE_ERR_STRIDE;
  if (!aligned(q, 8) || ld_q % 8 || !aligned(w_packed, 256) || !aligned(dots, 4))
    return MOE_ERR_ALIGNMENT;
  if (!device_is_gfx950()) return MOE_ERR_UNSUPPORTED_ARCH;
  const PackedDims pd(n_out, d_in);
  hipLaunchKernelGGL(block_dots_kernel, dim3((unsigned)(pd.rg * pd.kc)), dim3(64), 0,
                     (hipStream_t)stream, (const uint8_t*)w_packed, n_out, d_in, q, ld_q, rows,
                     dots);
  return launch_status();
}

// Prefill runs the grouped matrix-core GEMM (prefill.hip).
extern "C" int moe_ffn_prefill(const moe_layer_t* L, const int8_t* q, int64_t ld_q,
                               const float* qs, int64_t ld_qs, int rows, const int32_t* ids,
                               const float* w, const int32_t* offsets, const int32_t* sorted,
                               float* y, int64_t ld_y, void* ws, size_t ws_bytes, void* stream) {
  return ffn_entry(L, false, MOE_STAGE_ALL, q, ld_q, qs, ld_qs, rows, ids, w, offsets, sorted,
                   y, ld_y, ws, ws_bytes, stream);
}

extern "C" int moe_ffn_stages(const moe_layer_t* L, int prefill, int stage_mask,
                              const int8_t* q, int64_t ld_q, const float* qs, int64_t ld_qs,
                              int rows, const int32_t* ids, const float* w,
                              const int32_t* offsets, const int32_t* sorted, float* y,
                              int64_t ld_y, void* ws, size_t ws_bytes, void* stream) {
  if (prefill != 0 && prefill != 1) return MOE_ERR_INVALID_ARG;
  return ffn_entry(L, prefill == 0, stage_mask, q, ld_q, qs, ld_qs, rows, ids, w, offsets,
                   sorted, y, ld_y, ws, ws_bytes, stream);
}
