// prefill.hip -- grouped GEMM for prefill chunks on gfx950's scaled FP4
// matrix core.
//
// The gfx90a report (§7.1) moves prefill from a per-assignment dot path to
// INT8 MFMA routed gate and down kernels with FP4 unpack reused across rows,
// and (§7.1 item 8) sorts assignments into per-expert row blocks so an expert
// with ~48 rows scans its packed weights once.  Here a workgroup owns one
// tile of up to 128 token rows of one expert (rows grouped by
// moe_route_group) and 256 weight rows, so each expert's weights stream once
// per 128 tokens.  The contraction is exact on the matrix core without any
// unpacking of the weights:
//
//   * gfx950's scaled 16x16x128 FP4 instruction takes the packed E2M1 codes
//     as they are and applies one E8M0 byte per row and 32-element K slot
//     (picked from a register by the instruction's byte select), so the
//     weights go from LDS to the matrix core untouched.
//   * An int8 activation block has no exact FP4 form, but its code q in
//     [-127, 127] splits into balanced base-4 digits, q = d0 + 4 d1 + 16 d2 +
//     64 d3 with every d in {-2..2}, each an exact E2M1 value.  The four
//     digit planes of one 32-element block fill the instruction's four K
//     slots, with B scales 2^0, 2^2, 2^4, 2^6, against the same weight block
//     in every slot: one instruction gives the exact integer block dot times
//     2^(u-127) (every product and partial sum is a multiple of half an E2M1
//     step below 2^15 of them, exact in fp32) -- the same fp32 value as the
//     decode kernels' bf16 route.  The activation scale follows with one fp32
//     FMA per output and block.
//   * The sums run as in every decode kernel: runs of 16 blocks (4 chunks),
//     each folded from zero in block order, added in order -- so a prefill
//     row has the bits of the same row decoded alone (exact rows).
//
// Data movement:
//   * A prep kernel turns each token's int8 codes into digit planes once
//     (2 bytes per code); the gate/up GEMM reads the planes of its tile's
//     tokens through the sorted assignment list.  Its epilogue (SwiGLU +
//     group-32 requant) writes the hidden codes as digit planes too, in tile
//     order, which the down GEMM reads directly.
//   * Weights, scales, digit planes and activation scales stream through a
//     3-stage LDS ring filled by direct global->LDS loads (no registers).
//   * 16 waves (128-row tiles; 8 for 32-row tiles): 4 row quarters (4 row
//     groups each) x 4 token parts (token groups tp, tp+4), a 64 x 32 output
//     block per wave.
//   * Block ids are remapped so the workgroups that share a token tile run on
//     the same XCD and share its L2.
#include "ffn_internal.h"

namespace moe {

// Token rows per tile: 128 (8 groups of 16), or 32 when experts hold few rows
// each: a short tile's stage takes half the LDS, so two workgroups share a
// CU and one streams while the other starts (finds its tile, waits for its
// first chunk).
constexpr int kBMFull = 128;
constexpr int kBMShort = 32;
constexpr int kBNGroups = 16;  // 16-row weight groups per workgroup (256 rows)
constexpr int kRing = 3;       // LDS stages (chunks in flight ahead: kRing - 1)
constexpr int kRunChunks = 4;  // chunks per exact-rows run (16 blocks)
// Waves per workgroup: 4 row quarters x TH token parts, 4 waves per SIMD
// (<= 128 VGPRs each) so latencies of one wave hide behind the others.
// 128-row tiles: 16 waves, each 4 row groups x 2 of the 8 token groups;
// 32-row tiles: 8 waves, each 4 row groups x 1 of the 2 (two workgroups
// share a CU).
template <int BM> constexpr int gemm_waves() { return 8; }
template <int BM> constexpr int gemm_th() { return gemm_waves<BM>() / 4; }

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
  const uint8_t* xp;  // B digit planes: tokens (gate/up) or hidden rows (down)
  int64_t ld_xp;      // bytes per row of planes (2 * K)
  const float* xs;    // B scales: qs (gate/up) or hidden scales (down)
  int64_t ld_xs;
  int n_items;  // tiles bound x weight-row blocks
  uint8_t* h;   // gate/up: hidden digit planes
  float* hs;
  int64_t ld_h, ld_hs;  // bytes per hidden row, floats per hidden-scale row
  float* y;             // down partials
  int64_t ld_y;
  int bf16_mid;  // gate/up: round the intermediate to bf16 before its requant
};

// One LDS stage = one 128-element K chunk of the workgroup's operands, each
// piece in the order its reader uses:
template <int BM>
struct Stage {
  static constexpr int NTG = BM / 16;              // token groups
  static constexpr int NTD = NTG < 4 ? 4 : NTG;    // scale rows, whole loads of 4 groups
  u32x4 a[kBNGroups][64];  // packed tiles, lane 16 j + r: row r's block j   16 KiB
  uint32_t s[kBNGroups][16];  // E8M0 bytes of the chunk's 4 blocks, per row  1 KiB
  u32x4 b[NTG][4][64];     // digit planes, [token group][block][16 s + col]  BM/4 KiB
  f32x4 d[NTD][16];        // activation scales of the chunk's 4 blocks, per column
};

// vmcnt <= n (n < 64), no wait on the other counters (gfx9 encoding: vmcnt
// bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
#define WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(0xF70 | ((n) & 15) | (((n) >> 4) << 14))
__device__ inline void wait_vmcnt(int n) {  // n wave-uniform, 0..15
  switch (n) {
    case 0: WAIT_VMCNT(0); break;
    case 1: WAIT_VMCNT(1); break;
    case 2: WAIT_VMCNT(2); break;
    case 3: WAIT_VMCNT(3); break;
    case 4: WAIT_VMCNT(4); break;
    case 5: WAIT_VMCNT(5); break;
    case 6: WAIT_VMCNT(6); break;
    case 7: WAIT_VMCNT(7); break;
    case 8: WAIT_VMCNT(8); break;
    case 9: WAIT_VMCNT(9); break;
    case 10: WAIT_VMCNT(10); break;
    case 11: WAIT_VMCNT(11); break;
    case 12: WAIT_VMCNT(12); break;
    case 13: WAIT_VMCNT(13); break;
    case 14: WAIT_VMCNT(14); break;
    default: WAIT_VMCNT(15); break;
  }
}

// Workgroup barrier for the LDS ring.  __syncthreads() (and any LDS fence)
// would wait for every outstanding direct-to-LDS load (vmcnt(0)) and collapse
// the prefetch to one chunk.  Instead each wave first waits for its own loads
// of the chunk about to be consumed (loads complete in issue order), then
// all waves meet at s_barrier; every LDS read of the previous chunk has
// returned (its data was consumed) before a wave reaches it.  The empty asm
// statements keep the compiler from moving memory accesses across.
__device__ inline void ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Direct buffer -> LDS load: lane l writes `bytes` (4 or 16) at lds_base + l *
// bytes from the resource at voff (per lane) + soff (uniform).  A resource
// in scalar registers and one 32-bit lane offset cost fewer vector registers
// than a 64-bit address per lane.
__device__ inline void buf_to_lds(__amdgpu_buffer_rsrc_t r, void* lds_base, int bytes,
                                  uint32_t voff, uint32_t soff) {
  if (bytes == 16)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)lds_base, 16, voff, soff, 0, 0);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)lds_base, 4, voff, soff, 0, 0);
}

// ------------------------------------------------------------ digit planes
// E2M1 code of a digit in {-2..2}: sign bit 3, |d| = 1 -> 0b010, 2 -> 0b100.
__device__ inline uint32_t digit_code(int d) {
  return (d < 0 ? 8u : 0u) | ((uint32_t)(d < 0 ? -d : d) << 1);
}
// The four balanced base-4 digits of q in [-127, 127] as E2M1 codes:
// d_s = ((x + 2) mod 4) - 2, x <- (x - d_s) / 4, the last digit what is left.
__device__ inline void q8_digit_codes(int q, uint32_t (&c)[4]) {
  int x = q;
#pragma unroll
  for (int s = 0; s < 3; ++s) {
    const int dg = ((x + 2) & 3) - 2;
    c[s] = digit_code(dg);
    x = (x - dg) >> 2;
  }
  c[3] = digit_code(x);
}

// One thread per 8 codes of a token row: plane s of block b holds the 32
// digit-s codes of the block (16 bytes, element 2i in the low nibble of byte
// i); a row is [K/32 blocks][4 planes][16 B].  Threads 4b..4b+3 of a row
// write the 64 bytes of block b.
__global__ __launch_bounds__(256) void prep_digits_kernel(const int8_t* __restrict__ q,
                                                          int64_t ld_q, int rows, int d_model,
                                                          uint8_t* __restrict__ xp,
                                                          int64_t ld_xp) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int per_row = d_model / 8;
  if (i >= (int64_t)rows * per_row) return;
  const int t = (int)(i / per_row);
  const int c8 = (int)(i % per_row);  // 8-element group: block c8 / 4, quarter c8 % 4
  const u32x2 v = *(const u32x2*)(q + (int64_t)t * ld_q + (int64_t)c8 * 8);
  uint32_t plane[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int code = (int)(int8_t)((v[e >> 2] >> (8 * (e & 3))) & 0xFFu);
    uint32_t c[4];
    q8_digit_codes(code, c);
#pragma unroll
    for (int s = 0; s < 4; ++s) plane[s] |= c[s] << (4 * e);
  }
  uint8_t* dst = xp + (int64_t)t * ld_xp + (int64_t)(c8 >> 2) * 64 + (c8 & 3) * 4;
#pragma unroll
  for (int s = 0; s < 4; ++s) *(uint32_t*)(dst + 16 * s) = plane[s];
}

// ------------------------------------------------------------------- GEMM
// Everything a workgroup knows about its item once the tile is found.
struct GemmCtx {
  __amdgpu_buffer_rsrc_t blob;  // the expert's packed matrix (tiles, then E8M0 bytes)
  int prb;       // first packed row group of the workgroup
  int64_t row0;  // first hidden row of the tile (A + start for the shared expert)
  Tile t;
  bool shared;
  int A;
  int b_row;  // B / scale row of this lane's B loads (token or hidden row)
  int d_row;  // B / scale row of this lane's scale loads
};

// B row of tile row r (clamped into the tile): the token for gate/up (through
// the sorted list for routed experts), the hidden row for down.
template <int PASS>
__device__ inline int gemm_brow(const GemmArgs& p, const GemmCtx& c, int r) {
  r = min(r, c.t.count - 1);
  if (PASS == GEMM_DOWN) return (int)c.row0 + r;
  return c.shared ? c.t.start + r : p.sorted[c.t.start + r] / p.top_k;
}

// The loads of one K chunk, spread over the waves: the 16 weight tiles
// (16 / W per wave), the B digit-plane loads (one per token group and block:
// NTG * 4 / W per wave, all of them in token group (wave * that) / 4), the
// E8M0 bytes (waves 0-3, 4 row groups each) and the activation scales (waves
// 4 .. 4 + NTD/4 - 1, 4 token groups each).
template <int BM> constexpr int gemm_a_per_wave() { return kBNGroups / gemm_waves<BM>(); }
template <int BM> constexpr int gemm_b_per_wave() { return Stage<BM>::NTG * 4 / gemm_waves<BM>(); }
template <int BM> __device__ inline int gemm_b_tg(int wave) { return wave * gemm_b_per_wave<BM>() / 4; }

template <int BM>
__device__ inline int gemm_loads_per_chunk(int wave, bool b_live) {
  constexpr int NTD = Stage<BM>::NTD;
  int n = gemm_a_per_wave<BM>() + (wave < 4 ? 1 : 0) + (wave >= 4 && wave < 4 + NTD / 4 ? 1 : 0);
  if (b_live) n += gemm_b_per_wave<BM>();
  return n;
}

template <int PASS, int BM>
__device__ inline void gemm_issue(const GemmArgs& p, const GemmCtx& c, Stage<BM>& S, int kc,
                                  int wave, int lane, bool b_live) {
  const int n = lane & 15, g4 = lane >> 4;
  constexpr int AW = gemm_a_per_wave<BM>(), BW = gemm_b_per_wave<BM>();
  const uint32_t slot = (uint32_t)chunk_slot(kc, p.kc_total);
#pragma unroll
  for (int i = 0; i < AW; ++i) {
    const int rg = AW * wave + i;
    buf_to_lds(c.blob, &S.a[rg][0], 16, (uint32_t)lane * 16u,
               ((uint32_t)(c.prb + rg) * (uint32_t)p.kc_total + slot) * 1024u);
  }
  if (wave < 4) {  // E8M0 bytes of row groups 4 wave .. 4 wave + 3
    buf_to_lds(c.blob, &S.s[4 * wave][0], 4,
               (uint32_t)g4 * (uint32_t)p.sc_total * 256u + (uint32_t)n * 16u,
               (uint32_t)p.nib_bytes +
                   ((uint32_t)(c.prb + 4 * wave) * (uint32_t)p.sc_total + (uint32_t)(kc >> 2)) * 256u +
                   (uint32_t)(kc & 3) * 4u);
  } else if (wave < 4 + Stage<BM>::NTD / 4) {  // scales of token groups 4 q .. 4 q + 3
    const int qd = wave - 4;
    load_to_lds(p.xs + (int64_t)c.d_row * p.ld_xs + (int64_t)kc * 4, &S.d[4 * qd][0], 16);
  }
  if (b_live) {
    const uint8_t* src = p.xp + (int64_t)c.b_row * p.ld_xp + (int64_t)kc * 256 + 16 * g4;
#pragma unroll
    for (int i = 0; i < BW; ++i) {
      const int li = BW * wave + i, tg = li >> 2, j = li & 3;
      load_to_lds(src + 64 * j, &S.b[tg][j][0], 16);
    }
  }
}

// K loop + epilogue of one wave owning row groups prb+4*rq .. +3 and token
// groups tp, tp+TH, .. (NQ of them live).  Branch-free inner loop.
template <int PASS, int NQ, int BM>
__device__ __forceinline__ void gemm_body(const GemmArgs& p, const GemmCtx& c, Stage<BM>* ring) {
  const int tid = threadIdx.x;
  const int wave = uniform(tid >> 6), lane = tid & 63;
  const int n = lane & 15, g4 = lane >> 4;
  constexpr int TH = gemm_th<BM>();
  const int rq = wave & 3, tp = wave >> 2;
  const int nnt = (c.t.count + 15) >> 4;
  // token group this wave stages
  const bool b_live = gemm_b_tg<BM>(wave) < nnt;
  const int per_chunk = gemm_loads_per_chunk<BM>(wave, b_live);
  // B scale of K slot g4 (digit plane g4 carries weight 4^g4)
  const int sb = 127 + 2 * g4;

  f32x4 acc[4][NQ > 0 ? NQ : 1];
#pragma unroll
  for (int g = 0; g < 4; ++g)
#pragma unroll
    for (int q4 = 0; q4 < NQ; ++q4) acc[g][q4] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int KC = p.kc_total;
  // chunks 0 .. kRing-2 go out first; chunk kc + kRing - 1 after chunk kc lands
#pragma unroll
  for (int k0 = 0; k0 < kRing - 1; ++k0)
    if (k0 < KC) gemm_issue<PASS, BM>(p, c, ring[k0], k0, wave, lane, b_live);
  int kc = 0;
  // runs of kRunChunks chunks, each summed from zero and added in order
  for (int kr = 0; kr < KC; kr += kRunChunks) {
    f32x4 run[4][NQ > 0 ? NQ : 1];
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int q4 = 0; q4 < NQ; ++q4) run[g][q4] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int kend = min(kr + kRunChunks, KC);
    for (; kc < kend; ++kc) {
      // chunk kc has landed when no more than the loads of the chunks issued
      // after it are outstanding (loads complete in issue order)
      wait_vmcnt(min(kRing - 2, KC - 1 - kc) * per_chunk);
      ring_barrier();  // every wave's loads of chunk kc have landed; chunk kc-1 is consumed
      if (kc + kRing - 1 < KC)
        gemm_issue<PASS, BM>(p, c, ring[(kc + kRing - 1) % kRing], kc + kRing - 1, wave, lane,
                             b_live);
      if constexpr (NQ > 0) {
        const Stage<BM>& S = ring[kc % kRing];
        const float* sd = (const float*)&S.d[0][0];  // [token group][column][block]
        uint32_t sw[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) sw[g] = S.s[4 * rq + g][n];
        // operands of block j: A[g] (row n's block j of row group g, the same
        // 16 bytes in all four K slots), B[q4] (digit planes), D[q4] (scale)
        u32x4 A[2][4], B[2][NQ];
        float D[2][NQ];
        auto load = [&](int j, int slot) {
#pragma unroll
          for (int q4 = 0; q4 < NQ; ++q4) {
            B[slot][q4] = S.b[tp + TH * q4][j][lane];
            D[slot][q4] = sd[((tp + TH * q4) * 16 + n) * 4 + j];
          }
#pragma unroll
          for (int g = 0; g < 4; ++g) A[slot][g] = S.a[4 * rq + g][16 * j + n];
        };
        load(0, 0);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int cur = j & 1;
          if (j + 1 < 4) load(j + 1, cur ^ 1);  // next block's reads go out first
          // row group g's products, then the scaling of row group g-1's:
          // every FMA reads a result one row group old, never a fresh one
          f32x4 R[2][NQ];
#pragma unroll
          for (int g = 0; g <= 4; ++g) {
            if (g < 4) {
              const v8i32 av = {(int)A[cur][g][0], (int)A[cur][g][1], (int)A[cur][g][2],
                                (int)A[cur][g][3], 0, 0, 0, 0};
#pragma unroll
              for (int q4 = 0; q4 < NQ; ++q4) {
                const v8i32 bv = {(int)B[cur][q4][0], (int)B[cur][q4][1], (int)B[cur][q4][2],
                                  (int)B[cur][q4][3], 0, 0, 0, 0};
                R[g & 1][q4] = mfma_fp4_block(av, bv, j, (int)sw[g], sb);
              }
            }
            if (g > 0) {
#pragma unroll
              for (int q4 = 0; q4 < NQ; ++q4)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                  run[g - 1][q4][i] = fmaf(R[(g - 1) & 1][q4][i], D[cur][q4], run[g - 1][q4][i]);
            }
          }
        }
      }
    }
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int q4 = 0; q4 < NQ; ++q4) acc[g][q4] += run[g][q4];
  }

  if constexpr (NQ > 0) {
    const int pr0 = c.prb + 4 * rq;
    if (PASS == GEMM_GATEUP) {
      // rows pr0..pr0+3 = (gate j, up j, gate j+1, up j+1): 32 features from
      // f0; this lane holds features f0 + 4 g4 + i and f0 + 16 + 4 g4 + i
      const int f0 = pr0 * 8;
#pragma unroll
      for (int q4 = 0; q4 < NQ; ++q4) {
        const int nt = tp + TH * q4;
        float hv[8];
        float m = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          hv[i] = mid_round(swiglu(acc[0][q4][i], acc[1][q4][i]), p.bf16_mid);
          hv[4 + i] = mid_round(swiglu(acc[2][q4][i], acc[3][q4][i]), p.bf16_mid);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(hv[i]));
        m = fmaxf(m, __shfl_xor(m, 16, 64));
        m = fmaxf(m, __shfl_xor(m, 32, 64));
        const float d = m / 127.0f;
        const int col = nt * 16 + n;
        if (col < c.t.count) {
          // the 4 digit planes of this lane's 8 codes: elements 4 g4 .. +3
          // (bytes 2 g4, 2 g4 + 1) and 16 + 4 g4 .. +3 (bytes 8 + 2 g4, ..)
          uint32_t half[2][4] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            uint32_t cd[4];
            q8_digit_codes((int)q8_code(hv[e], d), cd);
#pragma unroll
            for (int s = 0; s < 4; ++s) half[e >> 2][s] |= cd[s] << (4 * (e & 3));
          }
          uint8_t* hrow = p.h + (c.row0 + col) * p.ld_h + (int64_t)(f0 >> 5) * 64 + 2 * g4;
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            *(uint16_t*)(hrow + 16 * s) = (uint16_t)half[0][s];
            *(uint16_t*)(hrow + 16 * s + 8) = (uint16_t)half[1][s];
          }
          if (g4 == 0) p.hs[(c.row0 + col) * p.ld_hs + (f0 >> 5)] = d;
        }
      }
    } else {
#pragma unroll
      for (int q4 = 0; q4 < NQ; ++q4) {
        const int col = (tp + TH * q4) * 16 + n;
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
__global__ __launch_bounds__(gemm_waves<BM>() * 64, BM == kBMFull ? 2 : 4) void gemm_kernel(GemmArgs p) {
  __shared__ Stage<BM> ring[kRing];

  // Block b runs on XCD b % 8 (round-robin dispatch).  XCD x walks tiles
  // x, x+8, x+16, ... and all weight-row blocks of a tile back to back, so the
  // workgroups sharing a token tile share that XCD's L2, and the live tiles
  // (the low ids) spread over all eight XCDs.
  const int n_nb = p.rg_total / kBNGroups;
  const int xcd = (int)(blockIdx.x % 8), slot = (int)(blockIdx.x / 8);
  const int tile_idx = (slot / n_nb) * 8 + xcd;
  const int nb = slot % n_nb;
  if (tile_idx * n_nb >= p.n_items) return;
  // The shared expert's tiles (all full but the last) take the low ids, so
  // the longest items start first and the short routed tiles fill the tail.
  TileMap<BM> m;
  m.load(p.offsets, p.n_experts, p.has_shared, p.rows);
  GemmCtx c;
  c.t = m.lookup(p.n_experts, p.rows,
                 tile_idx < m.shared_tiles ? m.routed + tile_idx : tile_idx - m.shared_tiles);
  c.t.expert = uniform(c.t.expert);
  c.t.start = uniform(c.t.start);
  c.t.count = uniform(c.t.count);
  if (c.t.expert < 0) return;
  c.shared = c.t.expert == p.n_experts;
  const int64_t eoff = c.shared ? 0 : uniform((int64_t)c.t.expert * p.w_stride);
  const uint8_t* blob = (c.shared ? p.w_shared : p.w) + eoff;
  c.blob = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(blob), (short)0,
      (int)(p.nib_bytes + (int64_t)p.rg_total * p.sc_total * 256), 0x00020000);
  c.prb = nb * kBNGroups;
  c.A = p.rows * p.top_k;
  c.row0 = c.shared ? (int64_t)c.A + c.t.start : c.t.start;
  const int wave = uniform((int)(threadIdx.x >> 6)), lane = (int)(threadIdx.x & 63);
  // the rows behind this lane's B load (the wave's token group, column
  // lane % 16) and scale load (token group 4 (wave - 4) + lane / 16)
  c.b_row = gemm_brow<PASS>(p, c, 16 * gemm_b_tg<BM>(wave) + (lane & 15));
  c.d_row = gemm_brow<PASS>(p, c, 16 * (4 * max(wave - 4, 0) + (lane >> 4)) + (lane & 15));

  // live token groups of this wave's part: tp, tp+TH, ... below nnt
  constexpr int TH = gemm_th<BM>();
  const int nnt = (c.t.count + 15) >> 4;
  const int tp = wave >> 2;
  const int nq = min(BM / 16 / TH, max(0, (nnt - tp + TH - 1) / TH));
  if constexpr (BM == kBMFull) {
    switch (nq) {  // wave-uniform
      case 4: gemm_body<PASS, 4, BM>(p, c, ring); break;
      case 3: gemm_body<PASS, 3, BM>(p, c, ring); break;
      case 2: gemm_body<PASS, 2, BM>(p, c, ring); break;
      case 1: gemm_body<PASS, 1, BM>(p, c, ring); break;
      default: gemm_body<PASS, 0, BM>(p, c, ring); break;
    }
  } else {
    if (nq == 1) gemm_body<PASS, 1, BM>(p, c, ring);
    else gemm_body<PASS, 0, BM>(p, c, ring);
  }
}

int prefill_run(const moe_layer_t* L, int stages, const int8_t* q, int64_t ld_q,
                const float* qs, int64_t ld_qs, int rows, const int32_t* ids, const float* w,
                const int32_t* offsets, const int32_t* sorted, float* y, int64_t ld_y, void* ws,
                hipStream_t s) {
  const WsLayout lay = ws_layout(L, rows);
  uint8_t* base = (uint8_t*)ws;
  const int A = rows * L->top_k;
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
  a.h = base + lay.hidden;
  a.hs = (float*)(base + lay.hidden_scales);
  a.ld_h = 2 * (int64_t)L->d_ff;
  a.ld_hs = L->d_ff / kBlock;

  auto launch = [&](int pass, GemmArgs& g) {
    g.n_items = tiles * (g.rg_total / kBNGroups);
    const unsigned grid = (unsigned)((tiles + 7) / 8 * 8 * (g.rg_total / kBNGroups));
    const dim3 block(gemm_waves<kBMFull>() * 64), block_s(gemm_waves<kBMShort>() * 64);
    if (pass == GEMM_GATEUP) {
      if (short_tiles) hipLaunchKernelGGL((gemm_kernel<GEMM_GATEUP, kBMShort>), dim3(grid), block_s, 0, s, g);
      else hipLaunchKernelGGL((gemm_kernel<GEMM_GATEUP, kBMFull>), dim3(grid), block, 0, s, g);
    } else {
      if (short_tiles) hipLaunchKernelGGL((gemm_kernel<GEMM_DOWN, kBMShort>), dim3(grid), block_s, 0, s, g);
      else hipLaunchKernelGGL((gemm_kernel<GEMM_DOWN, kBMFull>), dim3(grid), block, 0, s, g);
    }
  };

  if (stages & MOE_STAGE_GATE_UP) {
    uint8_t* xp = base + lay.act;
    const int64_t ld_xp = 2 * (int64_t)L->d_model;
    if (!(stages & MOE_STAGE_REUSE_ACTS)) {
      const int64_t threads = (int64_t)rows * (L->d_model / 8);
      hipLaunchKernelGGL(prep_digits_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256),
                         0, s, q, ld_q, rows, L->d_model, xp, ld_xp);
    }
    const PackedDims pd(2 * L->d_ff, L->d_model);
    GemmArgs g = a;
    g.w = (const uint8_t*)L->gate_up;
    g.w_stride = L->gate_up_stride;
    g.w_shared = (const uint8_t*)L->shared_gate_up;
    g.nib_bytes = pd.nib_bytes;
    g.rg_total = (int)pd.rg;
    g.kc_total = (int)pd.kc;
    g.sc_total = (int)pd.sc;
    g.xp = xp;
    g.ld_xp = ld_xp;
    g.xs = qs;
    g.ld_xs = ld_qs;
    g.bf16_mid = (L->flags & MOE_LAYER_BF16_INTERMEDIATE) != 0;
    launch(GEMM_GATEUP, g);
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
    d.xp = a.h;
    d.ld_xp = a.ld_h;
    d.xs = a.hs;
    d.ld_xs = a.ld_hs;
    d.y = (float*)(base + lay.partials);
    d.ld_y = L->d_model;
    launch(GEMM_DOWN, d);
    launch_combine((const float*)(base + lay.partials), ids, w, rows, L->top_k, L->has_shared,
                   L->d_model, y, ld_y, s);
  }
  return launch_status();
}

}  // namespace moe
