// prefill.hip -- grouped matrix-core GEMM for prefill chunks.
//
// The gfx90a report (§7.1) moves prefill from a per-assignment dot path to
// INT8 MFMA routed gate and down kernels with FP4 unpack reused across rows,
// and (§7.1 item 8) sorts assignments into per-expert row blocks so an expert
// with ~48 rows scans its packed weights once.  Here a workgroup owns one
// tile of up to 128 token rows of one expert (rows grouped by
// moe_route_group) and 256 weight rows, so each expert's weights are streamed
// once per 128 tokens.  The contraction runs on the bf16 matrix core with the
// same exact per-block scheme as decode (E2M1 x E8M0 folded into bf16 by the
// FP4 converter, int8 codes exact in bf16, one 16x16x32 op per 32-element
// block, fp32 FMA with the activation scale).
//
//   * A prep kernel gathers every hidden row's activation codes once into
//     bf16 rows in tile order (so a tile's token rows are contiguous).
//   * A workgroup owns 128 token rows x 256 weight rows; 16 waves = 4 row
//     quarters x 4 token parts (token groups interleaved for balance); wave
//     tile = 4 row groups x up to 2 token groups, the live count being a
//     template parameter so the inner loop is branch-free.  32-row tiles
//     take 8 waves (4 row quarters x 2 token parts, one token group each).
//   * Weights, scales, token fragments and activation scales stream through
//     a 3-stage LDS ring filled by direct global->LDS loads (no registers),
//     each piece in the lane order its reader uses.
//   * Block ids are remapped so the workgroups that share a token tile run on
//     the same XCD and share its L2.
//   * Gate/up epilogue: SwiGLU + group-32 requant in registers (a wave holds
//     gate and up of the same 32 features); down epilogue: fp32 partials.
#include "ffn_internal.h"

namespace moe {

// Token rows per tile: 128 (8 groups of 16), or 32 when experts hold few rows
// each: a short tile's stage takes half the LDS, so two workgroups share a
// CU and one streams while the other starts (finds its tile, waits for its
// first chunk).  Measured on MI355X, 512-token step: 0.783 vs 0.920 ms.
constexpr int kBMFull = 128;
constexpr int kBMShort = 32;
constexpr int kBNGroups = 16;     // 16-row weight groups per workgroup (256 rows)
// Waves per workgroup: 4 row quarters x TH token parts.  128-row tiles take
// 16 waves (each 2 of the 8 token groups; 4 waves per SIMD hide the MFMA and
// load latencies), 32-row tiles 8 (each 1 of 2).  Waves 0-7 issue the ring's
// loads.
template <int BM> constexpr int gemm_waves() { return BM == kBMFull ? 16 : 8; }
template <int BM> constexpr int gemm_th() { return gemm_waves<BM>() / 4; }
// LDS ring depth (prefetch distance: stages - 1 chunks); 3 x 25.5 KB lets
// two short-tile workgroups share a CU (a 5-deep ring for one workgroup
// measured 0.921 ms)
template <int BM> constexpr int ring_stages() { return 3; }
constexpr int kLoadsPerChunk = 8; // direct-to-LDS loads per wave per K chunk

enum GemmPass : int { GEMM_GATEUP = 0, GEMM_DOWN = 1 };

struct GemmArgs {
  const uint8_t* w;
  int64_t w_stride;
  const uint8_t* w_shared;
  int64_t nib_bytes;
  int rg_total, kc_total, sc_total;
  const int32_t* offsets;
  const int32_t* sorted;
  int n_experts, top_k, has_shared, rows;
  const uint16_t* xb;  // B rows (bf16 codes), tile order
  int64_t ld_xb;
  const float* xs;
  int64_t ld_xs;
  int n_items;  // tiles bound x weight-row blocks
  uint16_t* h;  // gate/up outputs
  float* hs;
  int64_t ld_h, ld_hs;
  float* y;  // down partials
  int64_t ld_y;
  int bf16_mid;  // gate/up: round the intermediate to bf16 before its requant
};

// One LDS stage = one 128-element K chunk of the workgroup's operands, each
// piece in the lane order its consumer reads (conflict-free ds_read_b128):
template <int BM>
struct Stage {
  u32x4 a[kBNGroups][64];        // weight fragments, [row group][lane]      16 KiB
  uint32_t s[kBNGroups][16];     // E8M0 bytes of the chunk's 4 blocks, per row 1 KiB
  u32x4 b[BM / 16][4][64];       // token fragments, [token group][block][lane] BM/4 KiB
  float d[BM / 16][4][16];       // activation scales, [token group][block][token]
};

// vmcnt <= n (n < 64), no wait on the other counters (gfx9 encoding: vmcnt
// bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
#define WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(0xF70 | ((n) & 15) | (((n) >> 4) << 14))

// Workgroup barrier for the LDS ring.  __syncthreads() (and any LDS fence)
// would wait for every outstanding direct-to-LDS load (vmcnt(0)) and collapse
// the prefetch to one chunk.  Instead each wave first waits for its own loads
// of the chunk about to be consumed (WAIT_VMCNT; loads complete in issue
// order), then all waves meet at s_barrier; every LDS read of the previous
// chunk has returned (its data was consumed) before a wave reaches it.  The
// empty asm statements keep the compiler from moving memory accesses across.
__device__ inline void ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One thread per 8 activations of a hidden row: q[token] -> bf16 row p.
__global__ __launch_bounds__(256) void gather_act_kernel(
    const int8_t* __restrict__ q, int64_t ld_q, const float* __restrict__ qs, int64_t ld_qs,
    const int32_t* __restrict__ sorted, const int32_t* __restrict__ offsets, int n_experts,
    int rows, int top_k, int has_shared, int d_model, uint16_t* __restrict__ xb, int64_t ld_xb,
    float* __restrict__ xs, int64_t ld_xs) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int per_row = d_model / 8;
  const int A = rows * top_k;
  const int64_t n_rows = (int64_t)A + (has_shared ? rows : 0);
  if (i >= n_rows * per_row) return;
  const int p = (int)(i / per_row);
  const int c = (int)(i % per_row);
  int token;
  if (p < A) {
    if (p >= offsets[n_experts]) return;  // sentinel-only tail: no hidden row
    token = sorted[p] / top_k;
  } else {
    token = p - A;
  }
  const u32x2 v = *(const u32x2*)(q + (int64_t)token * ld_q + (int64_t)c * 8);
  *(bf16x8*)(xb + (int64_t)p * ld_xb + (int64_t)c * 8) = i8x8_to_bf16x8(v);
  if ((c & 3) == 0) xs[(int64_t)p * ld_xs + c / 4] = qs[(int64_t)token * ld_qs + c / 4];
}

// Everything a workgroup knows about its item once the tile is found.
struct GemmCtx {
  const u32x4* nib;
  const uint8_t* scl;
  int prb;       // first packed row group of the workgroup
  int64_t row0;  // first B row (hidden row) of the tile
  Tile t;
  bool shared;
  int A;
};

// Issue wave `wave`'s share of K chunk kc into `S`: 2 weight tiles, 1 scale
// load, and -- when its token group is live -- 4 token fragments + 1 scale load.
template <int BM>
__device__ inline void gemm_issue(const GemmArgs& p, const GemmCtx& c, Stage<BM>& S, int kc,
                                  int wave, int lane, bool b_live) {
  const int n = lane & 15, g4 = lane >> 4, rq = wave & 3;
  if (wave >= 8) return;  // waves 8-15 (16-wave workgroups) issue nothing
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int rg = 2 * wave + i;
    load_to_lds(c.nib + ((int64_t)(c.prb + rg) * p.kc_total + chunk_slot(kc, p.kc_total)) * 64 + lane,
                &S.a[rg][0], 16);
  }
  {
    const int rg = 4 * rq + g4;
    load_to_lds(c.scl + (((int64_t)(c.prb + rg) * p.sc_total + (kc >> 2)) * 16 + n) * 16 + (kc & 3) * 4,
                &S.s[4 * rq][0], 4);
  }
  if (b_live) {
    const int r = min(wave * 16 + n, c.t.count - 1);
    const uint16_t* src = p.xb + (c.row0 + r) * p.ld_xb + (int64_t)kc * kChunkK + 8 * g4;
#pragma unroll
    for (int j = 0; j < 4; ++j) load_to_lds(src + j * kBlock, &S.b[wave][j][0], 16);
    load_to_lds(p.xs + (c.row0 + r) * p.ld_xs + (int64_t)kc * 4 + g4, &S.d[wave][0][0], 4);
  }
}

// K loop + epilogue of one wave owning row groups prb+4*rq .. +3 and token
// groups th, th+TH, .. (NQ of them live).  Branch-free inner loop.
template <int PASS, int NQ, int BM>
__device__ __forceinline__ void gemm_body(const GemmArgs& p, const GemmCtx& c, Stage<BM>* ring) {
  constexpr int NST = ring_stages<BM>();
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int n = lane & 15, g4 = lane >> 4;
  constexpr int TH = gemm_th<BM>();
  const int rq = wave & 3, th = wave >> 2;
  const int nnt = (c.t.count + 15) >> 4;
  const bool b_live = wave < nnt;  // this wave stages token group `wave` (< 8)

  f32x4 acc[4][NQ > 0 ? NQ : 1];
#pragma unroll
  for (int g = 0; g < 4; ++g)
#pragma unroll
    for (int q4 = 0; q4 < NQ; ++q4) acc[g][q4] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int KC = p.kc_total;
  // chunks 0 .. NST-2 go out first; chunk kc + NST - 1 after chunk kc lands
#pragma unroll
  for (int k0 = 0; k0 < NST - 1; ++k0)
    if (k0 < KC) gemm_issue(p, c, ring[k0], k0, wave, lane, b_live);
  for (int kc = 0; kc < KC; ++kc) {
    // chunk kc has landed when no more than the loads of the chunks issued
    // after it are outstanding (loads complete in issue order)
    static_assert(NST - 2 <= 3 && 3 * kLoadsPerChunk < 64, "vmcnt range");
    switch (min(NST - 2, KC - 1 - kc)) {
      case 0: WAIT_VMCNT(0); break;
      case 1: if (b_live) WAIT_VMCNT(kLoadsPerChunk); else WAIT_VMCNT(3); break;
      case 2: if (b_live) WAIT_VMCNT(2 * kLoadsPerChunk); else WAIT_VMCNT(6); break;
      default: if (b_live) WAIT_VMCNT(3 * kLoadsPerChunk); else WAIT_VMCNT(9); break;
    }
    ring_barrier();  // every wave's loads of chunk kc have landed; chunk kc-1 is consumed
    if (kc + NST - 1 < KC)
      gemm_issue(p, c, ring[(kc + NST - 1) % NST], kc + NST - 1, wave, lane, b_live);
    if constexpr (NQ > 0) {
      const Stage<BM>& S = ring[kc % NST];
      float dxv[NQ][4];
#pragma unroll
      for (int q4 = 0; q4 < NQ; ++q4)
#pragma unroll
        for (int j = 0; j < 4; ++j) dxv[q4][j] = S.d[th + TH * q4][j][n];
      uint32_t sw[4];
      u32x4 aw[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        sw[g] = S.s[4 * rq + g][n];
        aw[g] = S.a[4 * rq + g][lane];
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x8 bfr[NQ];
#pragma unroll
        for (int q4 = 0; q4 < NQ; ++q4)
          bfr[q4] = __builtin_bit_cast(bf16x8, S.b[th + TH * q4][j][lane]);
        f32x4 r[4][NQ];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const bf16x8 af = fp4x8_to_bf16x8(aw[g][j], e8m0_to_f32((sw[g] >> (8 * j)) & 0xFFu));
#pragma unroll
          for (int q4 = 0; q4 < NQ; ++q4) r[g][q4] = mfma_block(af, bfr[q4]);
        }
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int q4 = 0; q4 < NQ; ++q4)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[g][q4][i] = fmaf(r[g][q4][i], dxv[q4][j], acc[g][q4][i]);
      }
    }
  }

  if constexpr (NQ > 0) {
    const int pr0 = c.prb + 4 * rq;
    if (PASS == GEMM_GATEUP) {
      // rows pr0..pr0+3 = (gate j, up j, gate j+1, up j+1): 32 features from f0
      const int f0 = pr0 * 8;
#pragma unroll
      for (int q4 = 0; q4 < NQ; ++q4) {
        const int nt = th + TH * q4;
        float hv[8];
        float m = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float g0 = acc[0][q4][i], u0 = acc[1][q4][i];
          const float g1 = acc[2][q4][i], u1 = acc[3][q4][i];
          hv[i] = mid_round(swiglu(g0, u0), p.bf16_mid);
          hv[4 + i] = mid_round(swiglu(g1, u1), p.bf16_mid);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(hv[i]));
        m = fmaxf(m, __shfl_xor(m, 16, 64));
        m = fmaxf(m, __shfl_xor(m, 32, 64));
        const float d = m / 127.0f;
        const int col = nt * 16 + n;
        if (col < c.t.count) {
          uint32_t packed[4];
#pragma unroll
          for (int i = 0; i < 8; i += 2) {
            const float q0 = q8_code(hv[i], d);
            const float q1 = q8_code(hv[i + 1], d);
            packed[i / 2] = (__float_as_uint(q0) >> 16) | (__float_as_uint(q1) & 0xFFFF0000u);
          }
          uint16_t* hrow = p.h + (c.row0 + col) * p.ld_h;
          *(u32x2*)(hrow + f0 + 4 * g4) = u32x2{packed[0], packed[1]};
          *(u32x2*)(hrow + f0 + 16 + 4 * g4) = u32x2{packed[2], packed[3]};
          if (g4 == 0) p.hs[(c.row0 + col) * p.ld_hs + (f0 >> 5)] = d;
        }
      }
    } else {
#pragma unroll
      for (int q4 = 0; q4 < NQ; ++q4) {
        const int col = (th + TH * q4) * 16 + n;
        if (col >= c.t.count) continue;
        const int64_t orow = c.shared ? (int64_t)c.A + c.t.start + col : p.sorted[c.t.start + col];
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *(f32x4*)(p.y + orow * p.ld_y + (pr0 + g) * 16 + 4 * g4) = acc[g][q4];
      }
    }
  }
}

template <int PASS, int BM>
__global__ __launch_bounds__(gemm_waves<BM>() * 64, 1) void gemm_kernel(GemmArgs p) {
  __shared__ Stage<BM> ring[ring_stages<BM>()];

  // Block b runs on XCD b % 8 (round-robin dispatch).  XCD x walks tiles
  // x, x+8, x+16, ... and all weight-row blocks of a tile back to back, so the
  // workgroups sharing a token tile share that XCD's L2, and the live tiles
  // (the low ids) spread over all eight XCDs.
  const int n_nb = p.rg_total / kBNGroups;
  const int xcd = (int)(blockIdx.x % 8), slot = (int)(blockIdx.x / 8);
  const int tile_idx = (slot / n_nb) * 8 + xcd;
  const int nb = slot % n_nb;
  if (tile_idx * n_nb >= p.n_items) return;
  int n_tiles;
  GemmCtx c;
  c.t = find_tile<BM>(p.offsets, p.n_experts, p.has_shared, p.rows, tile_idx, &n_tiles);
  if (c.t.expert < 0) return;
  c.shared = c.t.expert == p.n_experts;
  const uint8_t* blob = c.shared ? p.w_shared : p.w + (int64_t)c.t.expert * p.w_stride;
  c.nib = (const u32x4*)blob;
  c.scl = blob + p.nib_bytes;
  c.prb = nb * kBNGroups;
  c.A = p.rows * p.top_k;
  c.row0 = c.shared ? (int64_t)c.A + c.t.start : c.t.start;

  // live token groups of this wave's part: th, th+TH, ... below nnt
  constexpr int TH = gemm_th<BM>();
  const int nnt = (c.t.count + 15) >> 4;
  const int th = (threadIdx.x >> 6) >> 2;
  const int nq = min(BM / 16 / TH, max(0, (nnt - th + TH - 1) / TH));
  if constexpr (BM == kBMShort) {
    if (nq == 1) gemm_body<PASS, 1, BM>(p, c, ring);  // wave-uniform
    else gemm_body<PASS, 0, BM>(p, c, ring);
  } else {
    switch (nq) {  // wave-uniform
      case 2: gemm_body<PASS, 2, BM>(p, c, ring); break;
      case 1: gemm_body<PASS, 1, BM>(p, c, ring); break;
      default: gemm_body<PASS, 0, BM>(p, c, ring); break;
    }
  }
}

int prefill_run(const moe_layer_t* L, int stages, const int8_t* q, int64_t ld_q,
                const float* qs, int64_t ld_qs, int rows, const int32_t* ids, const float* w,
                const int32_t* offsets, const int32_t* sorted, float* y, int64_t ld_y, void* ws,
                hipStream_t s) {
  const WsLayout lay = ws_layout(L, rows);
  uint8_t* base = (uint8_t*)ws;
  const int A = rows * L->top_k;
  const int n_h = A + (L->has_shared ? rows : 0);
  // short tiles when experts average at most 16 rows (then more than 32 in
  // one expert is rare, and a second tile is the only cost)
  const bool short_tiles = (int64_t)A <= 16LL * L->n_experts;
  const int BM = short_tiles ? kBMShort : kBMFull;
  const int tiles = std::min(L->n_experts, A) + A / BM + 1 +
                    (L->has_shared ? (rows + BM - 1) / BM : 0);

  GemmArgs a{};
  a.offsets = offsets;
  a.sorted = sorted;
  a.n_experts = L->n_experts;
  a.top_k = L->top_k;
  a.has_shared = L->has_shared;
  a.rows = rows;

  if (stages & MOE_STAGE_GATE_UP) {
    uint16_t* xb = (uint16_t*)(base + lay.act);
    float* xs = (float*)(base + lay.act_scales);
    const int64_t threads = (int64_t)n_h * (L->d_model / 8);
    hipLaunchKernelGGL(gather_act_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                       s, q, ld_q, qs, ld_qs, sorted, offsets, L->n_experts, rows, L->top_k,
                       L->has_shared, L->d_model, xb, (int64_t)L->d_model, xs,
                       (int64_t)(L->d_model / kBlock));
    const PackedDims pd(2 * L->d_ff, L->d_model);
    GemmArgs g = a;
    g.w = (const uint8_t*)L->gate_up;
    g.w_stride = L->gate_up_stride;
    g.w_shared = (const uint8_t*)L->shared_gate_up;
    g.nib_bytes = pd.nib_bytes;
    g.rg_total = (int)pd.rg;
    g.kc_total = (int)pd.kc;
    g.sc_total = (int)pd.sc;
    g.xb = xb;
    g.ld_xb = L->d_model;
    g.xs = xs;
    g.ld_xs = L->d_model / kBlock;
    g.h = (uint16_t*)(base + lay.hidden);
    g.hs = (float*)(base + lay.hidden_scales);
    g.ld_h = L->d_ff;
    g.ld_hs = L->d_ff / kBlock;
    g.bf16_mid = (L->flags & MOE_LAYER_BF16_INTERMEDIATE) != 0;
    g.n_items = tiles * (g.rg_total / kBNGroups);
    const unsigned grid = (unsigned)((tiles + 7) / 8 * 8 * (g.rg_total / kBNGroups));
    if (short_tiles)
      hipLaunchKernelGGL((gemm_kernel<GEMM_GATEUP, kBMShort>), dim3(grid), dim3(gemm_waves<kBMShort>() * 64), 0, s, g);
    else
      hipLaunchKernelGGL((gemm_kernel<GEMM_GATEUP, kBMFull>), dim3(grid), dim3(gemm_waves<kBMFull>() * 64), 0, s, g);
  }
  if (stages & MOE_STAGE_DOWN) {
    const PackedDims pd(L->d_model, L->d_ff);
    GemmArgs d = a;
    d.w = (const uint8_t*)L->down;
    d.w_stride = L->down_stride;
    d.w_shared = (const uint8_t*)L->shared_down;
    d.nib_bytes = pd.nib_bytes;
    d.rg_total = (int)pd.rg;
    d.kc_total = (int)pd.kc;
    d.sc_total = (int)pd.sc;
    d.xb = (const uint16_t*)(base + lay.hidden);
    d.ld_xb = L->d_ff;
    d.xs = (const float*)(base + lay.hidden_scales);
    d.ld_xs = L->d_ff / kBlock;
    d.y = (float*)(base + lay.partials);
    d.ld_y = L->d_model;
    d.n_items = tiles * (d.rg_total / kBNGroups);
    const unsigned grid = (unsigned)((tiles + 7) / 8 * 8 * (d.rg_total / kBNGroups));
    if (short_tiles)
      hipLaunchKernelGGL((gemm_kernel<GEMM_DOWN, kBMShort>), dim3(grid), dim3(gemm_waves<kBMShort>() * 64), 0, s, d);
    else
      hipLaunchKernelGGL((gemm_kernel<GEMM_DOWN, kBMFull>), dim3(grid), dim3(gemm_waves<kBMFull>() * 64), 0, s, d);
    launch_combine((const float*)(base + lay.partials), ids, w, rows, L->top_k, L->has_shared,
                   L->d_model, y, ld_y, s);
  }
  return launch_status();
}

}  // namespace moe
