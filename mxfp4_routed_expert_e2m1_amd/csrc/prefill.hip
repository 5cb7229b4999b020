// prefill.hip -- grouped GEMM for prefill chunks on gfx950's scaled matrix
// core.
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
//   * gfx950's scaled 32x32x64 instruction takes the packed E2M1 weight codes
//     as they are and applies one E8M0 byte per row and 32-element K slot
//     (picked from a register by the instruction's byte select), so the
//     weights go from LDS to the matrix core untouched.
//   * An int8 activation block has no exact 4-bit form, but its code q in
//     [-127, 127] splits into two balanced base-16 digits, q = d0 + 16 d1
//     with d0 in [-8, 7] and d1 in [-8, 8], and every integer in [-8, 8] is
//     an exact E3M2 (6-bit) value.  The two digit planes of one 32-element
//     block fill the instruction's two K slots, with B scales 2^0 and 2^4,
//     against the same weight block in both: one instruction gives the exact
//     integer block dot times 2^(u-127) for a 32 x 32 output tile (every
//     product and partial sum is a multiple of half an E2M1 step below 2^16
//     of them, exact in fp32) -- the same fp32 value as the decode kernels'
//     bf16 route.  The activation scale follows with one fp32 FMA per output
//     and block.
//   * The sums run as in every decode kernel: runs of 16 blocks (4 chunks),
//     each folded from zero in block order, added in order -- so a prefill
//     row has the bits of the same row decoded alone (exact rows).
//
// Data movement:
//   * A prep kernel turns each token's int8 codes into digit planes once
//     (1.5 bytes per code); the gate/up GEMM reads the planes of its tile's
//     tokens through the sorted assignment list.  Its epilogue (SwiGLU +
//     group-32 requant) writes the hidden codes as digit planes too, in tile
//     order, which the down GEMM reads directly.
//   * Weights, scales, digit planes and activation scales stream through a
//     3-stage LDS ring filled by direct global->LDS loads (no registers).
//   * Waves: 4 row parts (64 weight rows, two 32-row tiles) x 2 token parts
//     (128-row tiles: token tiles tp, tp+2 of 32 tokens; 8 waves), or x 1
//     (32-row tiles: 4 waves, two workgroups per CU) -- a 64 x 64 output
//     block per wave at most.
//   * Block ids are remapped so the workgroups that share a token tile run on
//     the same XCD and share its L2.
#include "ffn_internal.h"

namespace moe {

// Token rows per tile: 128 (4 tiles of 32 tokens), or 32 when experts hold
// few rows each: a short tile's stage takes less LDS, so two workgroups share
// a CU and one streams while the other starts (finds its tile, waits for its
// first chunk).
constexpr int kBMFull = 128;
constexpr int kBMShort = 32;
constexpr int kBNGroups = 16;  // 16-row weight groups per workgroup (256 rows)
constexpr int kRing = 3;       // LDS stages (chunks in flight ahead: kRing - 1)
constexpr int kRunChunks = 4;  // chunks per exact-rows run (16 blocks)
constexpr int kMaxTileExperts = 512;  // TileMap's limit (8 experts per lane)
constexpr int kDigitBlock = 48;   // bytes of one 32-code block as two E3M2 digit planes
constexpr int kDigitChunk = 4 * kDigitBlock;  // one 128-element K chunk
// Waves per workgroup: 4 row parts x TP token parts, two waves per SIMD.
template <int BM> constexpr int gemm_waves() { return BM == kBMFull ? 8 : 4; }
template <int BM> constexpr int gemm_tp() { return gemm_waves<BM>() / 4; }
// 32-token tiles per wave
template <int BM> constexpr int gemm_qt() { return BM / 32 / gemm_tp<BM>(); }

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
  int64_t ld_xp;      // bytes per row of planes (>= 1.5 K)
  const float* xs;    // B scales: qs (gate/up) or hidden scales (down)
  int64_t ld_xs;
  u32x4 xp_rsrc, xs_rsrc;  // buffer resources over the rows of xp and xs
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
//   b: per 16-token group, the 16-byte pieces of the chunk's digit planes,
//   [piece][token]; block j of a token is pieces 3j (plane 0, bytes 0-15),
//   3j+1 (plane 1, bytes 0-15) and 3j+2 (bytes 16-23 of plane 0, then of
//   plane 1) -- the token's 192 bytes of the chunk in order.
template <int BM>
struct Stage {
  static constexpr int NTG = BM / 16;              // token groups
  static constexpr int NTD = NTG < 4 ? 4 : NTG;    // scale rows, whole loads of 4 groups
  u32x4 a[kBNGroups][64];  // packed tiles, lane 16 j + r: row r's block j   16 KiB
  uint32_t s[kBNGroups][16];  // E8M0 bytes of the chunk's 4 blocks, per row  1 KiB
  u32x4 b[NTG][12][16];    // digit planes (see above)                       3 BM/16 KiB
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

// Direct global -> LDS loads (no registers): lane l writes 16 (or 4) bytes
// at lds_base + 16 l (4 l).  They are written as asm so that the compiler
// does not see them as LDS stores: it cannot tell the ring's stages apart,
// and would wait for every load in flight (the prefetched chunks too)
// before the first LDS read of each chunk.  The ring orders them itself: a
// stage is read only after each wave's vmcnt wait for its own loads of it
// and a barrier, and refilled only after the barrier that follows its last
// reads.  M0 carries the LDS address (one wait state before the load); no
// other code in these kernels uses M0.
__device__ inline uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)(lds_ptr)p; }
// from the buffer resource r (scalar registers) at voff (per lane) + soff
// (uniform): a resource and a 32-bit lane offset cost fewer vector registers
// than a 64-bit address per lane
__device__ inline void buf_to_lds16(u32x4 r, const void* lds_base, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(lds_addr(lds_base)), "v"(voff), "s"(r), "s"(soff) : "memory", "m0");
}
__device__ inline void buf_to_lds4(u32x4 r, const void* lds_base, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :: "s"(lds_addr(lds_base)), "v"(voff), "s"(r), "s"(soff) : "memory", "m0");
}
// from a per-lane global address
__device__ inline void glb_to_lds16(const void* src, const void* lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(lds_addr(lds_base)), "v"(src) : "memory", "m0");
}

// ------------------------------------------------------------ digit planes
// E3M2 code (sign bit 5, 3 exponent bits with bias 3, 2 mantissa bits) of an
// integer d in [-8, 8]: the magnitude codes of 0..8 are 7-bit fields of one
// constant.
__device__ inline uint32_t bf6_digit(int d) {
  constexpr uint64_t kMag = (0x0CULL << 7) | (0x10ULL << 14) | (0x12ULL << 21) |
                            (0x14ULL << 28) | (0x15ULL << 35) | (0x16ULL << 42) |
                            (0x17ULL << 49) | (0x18ULL << 56);
  const int a = d < 0 ? -d : d;
  return (d < 0 ? 0x20u : 0u) | (uint32_t)((kMag >> (7 * a)) & 0x7Fu);
}
// The two balanced base-16 digits of q in [-128, 127] as E3M2 codes:
// d0 = ((q + 8) mod 16) - 8 in [-8, 7], d1 = (q - d0) / 16 in [-8, 8].
__device__ inline void q8_bf6_digits(int q, uint32_t& c0, uint32_t& c1) {
  const int d0 = ((q + 8) & 15) - 8;
  c0 = bf6_digit(d0);
  c1 = bf6_digit((q - d0) >> 4);
}
// 24-bit run of 4 codes (element i at bits 6i)
__device__ inline uint32_t bf6_run4(const uint32_t (&c)[4]) {
  return c[0] | (c[1] << 6) | (c[2] << 12) | (c[3] << 18);
}
// One plane of 32 codes as 6 dwords from its eight 4-code runs (run m at bit
// 24 m).
__device__ inline void bf6_plane(const uint32_t (&t)[8], uint32_t (&w)[6]) {
  w[0] = t[0] | (t[1] << 24);
  w[1] = (t[1] >> 8) | (t[2] << 16);
  w[2] = (t[2] >> 16) | (t[3] << 8);
  w[3] = t[4] | (t[5] << 24);
  w[4] = (t[5] >> 8) | (t[6] << 16);
  w[5] = (t[6] >> 16) | (t[7] << 8);
}
// A block's 48 bytes from its two planes: plane 0 bytes 0-15, plane 1 bytes
// 0-15, plane 0 bytes 16-23, plane 1 bytes 16-23.
__device__ inline void bf6_store_block(uint8_t* dst, const uint32_t (&p0)[6],
                                       const uint32_t (&p1)[6]) {
  *(u32x4*)dst = u32x4{p0[0], p0[1], p0[2], p0[3]};
  *(u32x4*)(dst + 16) = u32x4{p1[0], p1[1], p1[2], p1[3]};
  *(u32x4*)(dst + 32) = u32x4{p0[4], p0[5], p1[4], p1[5]};
}

// One thread per 32-code block of a token row: reads the block's int8 codes
// and writes its 48 bytes of digit planes; a row is [K/32 blocks][48 B].
__global__ __launch_bounds__(256) void prep_digits_kernel(const int8_t* __restrict__ q,
                                                          int64_t ld_q, int rows, int d_model,
                                                          uint8_t* __restrict__ xp,
                                                          int64_t ld_xp) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int per_row = d_model / 32;
  if (i >= (int64_t)rows * per_row) return;
  const int t = (int)(i / per_row);
  const int b = (int)(i % per_row);
  const u32x2* src = (const u32x2*)(q + (int64_t)t * ld_q + (int64_t)b * 32);
  uint32_t r0[8], r1[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const u32x2 v = src[k];
#pragma unroll
    for (int hw = 0; hw < 2; ++hw) {
      uint32_t c0[4], c1[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) q8_bf6_digits((int)(int8_t)((v[hw] >> (8 * e)) & 0xFFu), c0[e], c1[e]);
      r0[2 * k + hw] = bf6_run4(c0);
      r1[2 * k + hw] = bf6_run4(c1);
    }
  }
  uint32_t p0[6], p1[6];
  bf6_plane(r0, p0);
  bf6_plane(r1, p1);
  bf6_store_block(xp + (int64_t)t * ld_xp + (int64_t)b * kDigitBlock, p0, p1);
}

// ------------------------------------------------------------------- GEMM
// Everything a workgroup knows about its item once the tile is found.
struct GemmCtx {
  u32x4 blob;  // buffer resource of the expert's packed matrix (tiles, then E8M0 bytes)
  int prb;       // first packed row group of the workgroup
  int64_t row0;  // first hidden row of the tile (A + start for the shared expert)
  Tile t;
  bool shared;
  int A;
  uint32_t b_off;  // byte offset in xp of this lane's B loads' row (+ its 16-byte piece)
  uint32_t d_off;  // byte offset in xs of this lane's scale loads' row
};

// B row of tile row r (clamped into the tile): the token for gate/up (through
// the sorted list for routed experts), the hidden row for down.  In two
// steps, so that a persistent workgroup can load the next item's entries
// early and use them late: gemm_brow_raw reads (the sorted list's
// assignment for a routed gate/up tile, else the row itself), gemm_brow_fin
// turns that into the row.
template <int PASS>
__device__ inline int gemm_brow_raw(const GemmArgs& p, const GemmCtx& c, int r) {
  r = min(r, c.t.count - 1);
  if (PASS == GEMM_DOWN) return (int)c.row0 + r;
  return c.shared ? c.t.start + r : p.sorted[c.t.start + r];
}
template <int PASS>
__device__ inline int gemm_brow_fin(const GemmArgs& p, bool shared, int raw) {
  return (PASS == GEMM_DOWN || shared) ? raw : raw / p.top_k;
}

// The loads of one K chunk, spread over the waves: the 16 weight tiles
// (16 / W per wave), the B digit-plane loads (three per token group, each 4
// pieces x 16 tokens; wave w takes loads [w NB / W, (w + 1) NB / W), all in
// one token group), the E8M0 bytes (waves 0-3, 4 row groups each) and the
// activation scales (the last NTD/4 waves, 4 token groups each).
template <int BM> constexpr int gemm_a_per_wave() { return kBNGroups / gemm_waves<BM>(); }
template <int BM> constexpr int gemm_b_loads() { return Stage<BM>::NTG * 3; }
template <int BM> constexpr int gemm_b_max() {
  return (gemm_b_loads<BM>() + gemm_waves<BM>() - 1) / gemm_waves<BM>();
}
template <int BM> __device__ inline int gemm_b_first(int wave) {
  return wave * gemm_b_loads<BM>() / gemm_waves<BM>();
}
template <int BM> __device__ inline int gemm_b_count(int wave) {
  return gemm_b_first<BM>(wave + 1) - gemm_b_first<BM>(wave);
}
template <int BM> __device__ inline int gemm_b_tg(int wave) { return gemm_b_first<BM>(wave) / 3; }
// index of the scale load of this wave (4 token groups from 4 * it), or -1
template <int BM> __device__ inline int gemm_d_wave(int wave) {
  constexpr int W = gemm_waves<BM>(), ND = Stage<BM>::NTD / 4;
  return wave >= W - ND ? wave - (W - ND) : -1;
}

template <int BM>
__device__ inline int gemm_loads_per_chunk(int wave, bool b_live) {
  int n = gemm_a_per_wave<BM>() + (wave < 4 ? 1 : 0) + (gemm_d_wave<BM>(wave) >= 0 ? 1 : 0);
  if (b_live) n += gemm_b_count<BM>(wave);
  return n;
}

template <int PASS, int BM>
__device__ inline void gemm_issue(const GemmArgs& p, const GemmCtx& c, Stage<BM>& S, int kc,
                                  int wave, int lane, bool b_live) {
  const int n = lane & 15, g4 = lane >> 4;
  constexpr int AW = gemm_a_per_wave<BM>();
  const uint32_t slot = (uint32_t)chunk_slot(kc, p.kc_total);
#pragma unroll
  for (int i = 0; i < AW; ++i) {
    const int rg = AW * wave + i;
    buf_to_lds16(c.blob, &S.a[rg][0], (uint32_t)lane * 16u,
               ((uint32_t)(c.prb + rg) * (uint32_t)p.kc_total + slot) * 1024u);
  }
  if (wave < 4) {  // E8M0 bytes of row groups 4 wave .. 4 wave + 3
    buf_to_lds4(c.blob, &S.s[4 * wave][0],
               (uint32_t)g4 * (uint32_t)p.sc_total * 256u + (uint32_t)n * 16u,
               (uint32_t)p.nib_bytes +
                   ((uint32_t)(c.prb + 4 * wave) * (uint32_t)p.sc_total + (uint32_t)(kc >> 2)) * 256u +
                   (uint32_t)(kc & 3) * 4u);
  }
  const int qd = gemm_d_wave<BM>(wave);
  if (qd >= 0)  // scales of token groups 4 qd .. 4 qd + 3
    buf_to_lds16(p.xs_rsrc, &S.d[4 * qd][0], c.d_off, (uint32_t)kc * 16u);
  if (b_live) {
    // load li: token group li / 3, pieces 4 (li % 3) .. + 3 of its 16 tokens
    // (lane: piece 4 (li % 3) + lane / 16 of token lane % 16)
    const int b0 = gemm_b_first<BM>(wave), nb = gemm_b_count<BM>(wave);
#pragma unroll
    for (int i = 0; i < gemm_b_max<BM>(); ++i) {
      if (i < nb) {
        const int li = b0 + i, tg = li / 3, part = li % 3;
        buf_to_lds16(p.xp_rsrc, &S.b[tg][4 * part][0], c.b_off,
                     (uint32_t)kc * (uint32_t)kDigitChunk + 64u * (uint32_t)part);
      }
    }
  }
}

// K loop + epilogue of one wave: row tiles rt = 0, 1 (16-row groups
// pr0 + 2 rt for rows 0-15 of the tile and pr0 + 2 rt + 1 for rows 16-31,
// pr0 = prb + 4 rp) and its NQ live 32-token tiles tp, tp + TP.  Lane l
// works on row / token l % 32 of a tile: 16-row group (or token group)
// 2 x + hi, column n, hi = (l / 16) % 2; its K slot h = l / 32 carries digit
// plane h.  Branch-free inner loop.
template <int PASS, int BM> __device__ inline bool gemm_b_live(const GemmCtx& c, int wave) {
  return gemm_b_tg<BM>(wave) < ((c.t.count + 15) >> 4);  // this wave stages a live token group
}

// The first kRing-1 chunks of an item (the rest go out as the K loop runs).
template <int PASS, int BM>
__device__ inline void gemm_issue_first(const GemmArgs& p, const GemmCtx& c, Stage<BM>* ring) {
  const int wave = uniform((int)(threadIdx.x >> 6)), lane = (int)(threadIdx.x & 63);
  const bool b_live = gemm_b_live<PASS, BM>(c, wave);
#pragma unroll
  for (int k0 = 0; k0 < kRing - 1; ++k0)
    if (k0 < p.kc_total) gemm_issue<PASS, BM>(p, c, ring[k0], k0, wave, lane, b_live);
}

// Item c, whose first chunks are already out; between() runs between the K
// loop and the epilogue (a persistent workgroup sends its next item's first
// chunks there, after a barrier -- the ring is free once every wave is past
// its last chunk -- so they land while this item's epilogue runs).
template <int PASS, int NQ, int BM, typename Between>
__device__ __forceinline__ void gemm_body(const GemmArgs& p, const GemmCtx& c, Stage<BM>* ring,
                                          Between between) {
  const int tid = threadIdx.x;
  const int wave = uniform(tid >> 6), lane = tid & 63;
  const int n = lane & 15, hi = (lane >> 4) & 1, h = lane >> 5;
  constexpr int TP = gemm_tp<BM>();
  constexpr int NQ1 = NQ > 0 ? NQ : 1;
  constexpr int NT = 2 * NQ;  // tiles per block
  const int rp = wave & 3, tp = wave >> 2;
  auto tile_of = [&](int q) { return tp + TP * q; };  // token tile of slot q
  const bool b_live = gemm_b_live<PASS, BM>(c, wave);
  const int per_chunk = gemm_loads_per_chunk<BM>(wave, b_live);
  // B scale of K slot h (digit plane h carries weight 16^h)
  const int sb = 127 + 4 * h;

  f32x16 acc[2][NQ1];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int q = 0; q < NQ1; ++q) acc[rt][q] = f32x16{};

  const int KC = p.kc_total;
  // chunk kc + kRing - 1 goes out after chunk kc lands
  int kc = 0;
  // runs of kRunChunks chunks, each summed from zero and added in order
  for (int kr = 0; kr < KC; kr += kRunChunks) {
    f32x16 run[2][NQ1];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int q = 0; q < NQ1; ++q) run[rt][q] = f32x16{};
    const int kend = min(kr + kRunChunks, KC);
    for (; kc < kend; ++kc) {
      // chunk kc has landed when no more than the loads of the chunks issued
      // after it are outstanding (loads complete in issue order)
      wait_vmcnt(min(kRing - 2, KC - 1 - kc) * per_chunk);
      ring_barrier();  // every wave's loads of chunk kc have landed; chunk kc-1 is consumed
      if (kc + kRing - 1 < KC)
        gemm_issue<PASS, BM>(p, c, ring[(kc + kRing - 1) % kRing], kc + kRing - 1, wave, lane,
                             b_live);
      if constexpr (NT > 0) {
        const Stage<BM>& S = ring[kc % kRing];
        const float* sd = (const float*)&S.d[0][0];  // [token group][column][block]
        uint32_t sw[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) sw[rt] = S.s[4 * rp + 2 * rt + hi][n];
        // the token's activation scales of the chunk's 4 blocks, one 16-byte
        // read per token tile (4-byte reads of single blocks would put the
        // two 16-token groups of a tile on the same LDS banks)
        f32x4 D[NQ1];
#pragma unroll
        for (int q = 0; q < NQ; ++q) D[q] = *(const f32x4*)&sd[((2 * tile_of(q) + hi) * 16 + n) * 4];
        // operands of block j: A[rt] (this lane's row, block j: the same 16
        // bytes in both K slots), BL/BH[q] (digit plane h of its token: bytes
        // 0-15, 16-23)
        u32x4 A[2][2], BL[2][NQ1];
        u32x2 BH[2][NQ1];
        auto load = [&](int j, int slot) {
#pragma unroll
          for (int q = 0; q < NQ; ++q) {
            const int tg = 2 * tile_of(q) + hi;
            BL[slot][q] = S.b[tg][3 * j + h][n];
            BH[slot][q] = ((const u32x2*)&S.b[tg][3 * j + 2][n])[h];
          }
#pragma unroll
          for (int rt = 0; rt < 2; ++rt) A[slot][rt] = S.a[4 * rp + 2 * rt + hi][16 * j + n];
        };
        load(0, 0);
        // the chunk's 4 x NT tile-blocks in order, u = NT j + t (tile t =
        // (row tile t / NQ, token tile t % NQ)): tile-block u's instruction,
        // then the scaling of tile-block u-1's value, so every FMA reads a
        // result one instruction old.  Block j+1's operands are read right
        // after block j's first instruction, into the slot of block j-1
        // (whose instructions are all out): a block's reads have a whole
        // block to land, and the wait before its first instruction covers no
        // later reads.
        f32x16 R[2];
#pragma unroll
        for (int u = 0; u <= 4 * NT; ++u) {
          // the steps stay in this order (the scheduler would sink the
          // reads next to their use and wait for them there)
          __builtin_amdgcn_sched_barrier(0);
          float dprev = 0.f;
          if (u > 0) dprev = D[((u - 1) % NT) % NQ1][(u - 1) / NT];
          if (u < 4 * NT) {
            const int j = u / NT, t = u % NT, cur = j & 1;
            const int rt = t / NQ1, q = t % NQ1;
            const u32x4 a4 = A[cur][rt], bl = BL[cur][q];
            const u32x2 bh = BH[cur][q];
            const v8i32 av = {(int)a4[0], (int)a4[1], (int)a4[2], (int)a4[3], 0, 0, 0, 0};
            const v8i32 bv = {(int)bl[0], (int)bl[1], (int)bl[2], (int)bl[3],
                              (int)bh[0], (int)bh[1], 0, 0};
            R[u & 1] = mfma_fp4_bf6_block(av, bv, j, (int)sw[rt], sb);
          }
          // the scaling below reads the previous instruction's result: kept
          // after this instruction, so the matrix core's latency is hidden
          __builtin_amdgcn_sched_barrier(0);
          if (u < 4 * NT && u % NT == 0 && u / NT + 1 < 4) load(u / NT + 1, (u / NT + 1) & 1);
          if (u > 0) {
            const int t = (u - 1) % NT;
            const int rt = t / NQ1, q = t % NQ1;
#pragma unroll
            for (int i = 0; i < 16; ++i)
              run[rt][q][i] = fmaf(R[(u - 1) & 1][i], dprev, run[rt][q][i]);
          }
        }
      }
    }
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int q = 0; q < NQ1; ++q) acc[rt][q] += run[rt][q];
  }
  between();  // (a persistent workgroup sends its next item's first chunks here)

  if constexpr (NT > 0) {
    const int pr0 = c.prb + 4 * rp;
    if (PASS == GEMM_GATEUP) {
      // row tile rt = (gate, up) of hidden features f0 + 16 rt .. + 15; a
      // lane holds features f0 + 16 rt + 8 a + 4 h + b (element 4 a + b of
      // the gate rows, 8 + 4 a + b of the up rows), lane l ^ 32 the other 16
      // of the 32 that share one requant scale.  Element e sits in 4-code
      // run e / 4 = 2 (2 rt + a) + h of its plane; a lane builds its runs of
      // both planes and writes plane h, taking the other runs of plane h
      // from lane l ^ 32.
      const int f0 = pr0 * 8;
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        float hv[2][8];
        float m = 0.f;
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            hv[rt][i] = mid_round(swiglu(acc[rt][q][i], acc[rt][q][8 + i]), p.bf16_mid);
            m = fmaxf(m, fabsf(hv[rt][i]));
          }
        m = fmaxf(m, __shfl_xor(m, 32, 64));
        const float d = m / 127.0f;
        // runs 2 k + h (k = 2 rt + a) of both planes
        uint32_t r0[4], r1[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          uint32_t c0[4], c1[4];
#pragma unroll
          for (int b = 0; b < 4; ++b)
            q8_bf6_digits((int)q8_code(hv[k >> 1][4 * (k & 1) + b], d), c0[b], c1[b]);
          r0[k] = bf6_run4(c0);
          r1[k] = bf6_run4(c1);
        }
        uint32_t t8[8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t own = h ? r1[k] : r0[k];
          const uint32_t got = (uint32_t)__shfl_xor((int)(h ? r0[k] : r1[k]), 32, 64);
          t8[2 * k] = h ? got : own;
          t8[2 * k + 1] = h ? own : got;
        }
        uint32_t w6[6];
        bf6_plane(t8, w6);
        const int col = 32 * tile_of(q) + 16 * hi + n;
        if (col < c.t.count) {
          uint8_t* hrow = p.h + (c.row0 + col) * p.ld_h + (int64_t)(f0 >> 5) * kDigitBlock;
          *(u32x4*)(hrow + 16 * h) = u32x4{w6[0], w6[1], w6[2], w6[3]};
          *(u32x2*)(hrow + 32 + 8 * h) = u32x2{w6[4], w6[5]};
          if (h == 0) p.hs[(c.row0 + col) * p.ld_hs + (f0 >> 5)] = d;
        }
      }
    } else {
      // rows pr0 * 16 + 32 rt + 8 a + 4 h + b: element 4 a + b of row tile rt
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const int col = 32 * tile_of(q) + 16 * hi + n;
        if (col >= c.t.count) continue;
        const int64_t orow = c.shared ? (int64_t)c.A + c.t.start + col : p.sorted[c.t.start + col];
        float* yr = p.y + orow * p.ld_y + (int64_t)pr0 * 16 + 4 * h;
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
          for (int a = 0; a < 4; ++a)
            *(f32x4*)(yr + 32 * rt + 8 * a) = f32x4{acc[rt][q][4 * a], acc[rt][q][4 * a + 1],
                                                    acc[rt][q][4 * a + 2], acc[rt][q][4 * a + 3]};
      }
    }
  }
}

// B / scale rows of this lane for an item with tile t: the token (gate/up,
// through the sorted list for routed experts) or hidden row (down) behind
// its B loads (the wave's token group, column lane % 16) and its scale load
// (token group 4 qd + lane / 16).  These are the item's only loads before
// its first chunk.
template <int PASS, int BM>
__device__ inline void gemm_rows(const GemmArgs& p, Tile t, int& raw_b, int& raw_d) {
  GemmCtx c;
  c.t = t;
  c.shared = t.expert == p.n_experts;
  c.row0 = c.shared ? (int64_t)p.rows * p.top_k + t.start : t.start;
  const int wave = uniform((int)(threadIdx.x >> 6));
  // (the lane index passes an empty asm, so the rows below are derived from
  // it afresh for each item: held across the K loop, the derived values were
  // spilled, and the reload's wait also waited for the chunks in flight)
  int lane = (int)(threadIdx.x & 63);
  asm volatile("" : "+v"(lane));
  raw_b = gemm_brow_raw<PASS>(p, c, 16 * gemm_b_tg<BM>(wave) + (lane & 15));
  raw_d = gemm_brow_raw<PASS>(p, c, 16 * (4 * max(gemm_d_wave<BM>(wave), 0) + (lane >> 4)) +
                                        (lane & 15));
}

// Everything about item (tile t, weight-row block nb) that the K loop and
// the epilogue need, given its rows.
template <int PASS, int BM>
__device__ inline GemmCtx gemm_ctx_rows(const GemmArgs& p, Tile t, int nb, int raw_b, int raw_d) {
  GemmCtx c;
  c.t.expert = uniform(t.expert);
  c.t.start = uniform(t.start);
  c.t.count = uniform(t.count);
  c.shared = c.t.expert == p.n_experts;
  const int64_t eoff = c.shared ? 0 : uniform((int64_t)c.t.expert * p.w_stride);
  const uint8_t* blob = (c.shared ? p.w_shared : p.w) + eoff;
  // base address (48 bits, stride 0), size in bytes (reads past it return
  // zero), raw dword access
  const uint64_t ba = (uint64_t)(uintptr_t)blob;
  c.blob = u32x4{(uint32_t)ba, (uint32_t)(ba >> 32) & 0xFFFFu,
                 (uint32_t)(p.nib_bytes + (int64_t)p.rg_total * p.sc_total * 256), 0x00020000u};
  c.prb = nb * kBNGroups;
  c.A = p.rows * p.top_k;
  c.row0 = c.shared ? (int64_t)c.A + c.t.start : c.t.start;
  const int lane = (int)(threadIdx.x & 63);
  c.b_off = (uint32_t)gemm_brow_fin<PASS>(p, c.shared, raw_b) * (uint32_t)p.ld_xp +
            16u * (uint32_t)(lane >> 4);
  c.d_off = (uint32_t)gemm_brow_fin<PASS>(p, c.shared, raw_d) * (uint32_t)p.ld_xs * 4u;
  return c;
}

template <int PASS, int BM>
__device__ inline GemmCtx gemm_ctx(const GemmArgs& p, Tile t, int nb) {
  int raw_b, raw_d;
  gemm_rows<PASS, BM>(p, t, raw_b, raw_d);
  return gemm_ctx_rows<PASS, BM>(p, t, nb, raw_b, raw_d);
}

// One item with the K loop's instantiation for this wave's live token tiles
// (tp, tp + TP, ... below the tile's 32-token tiles).
template <int PASS, int BM, typename Between>
__device__ inline void gemm_item(const GemmArgs& p, const GemmCtx& c, Stage<BM>* ring,
                                 Between between) {
  constexpr int TP = gemm_tp<BM>();
  const int n32 = (c.t.count + 31) >> 5;
  const int tp = uniform((int)(threadIdx.x >> 6)) >> 2;
  const int nq = min(gemm_qt<BM>(), max(0, (n32 - tp + TP - 1) / TP));
  if constexpr (gemm_qt<BM>() == 2) {
    switch (nq) {  // wave-uniform
      case 2: gemm_body<PASS, 2, BM>(p, c, ring, between); break;
      case 1: gemm_body<PASS, 1, BM>(p, c, ring, between); break;
      default: gemm_body<PASS, 0, BM>(p, c, ring, between); break;
    }
  } else {
    if (nq == 1) gemm_body<PASS, 1, BM>(p, c, ring, between);
    else gemm_body<PASS, 0, BM>(p, c, ring, between);
  }
}

// The call's tiles (as TileMap numbers them) kept in LDS for a persistent
// workgroup: per expert its first tile number and first row; tile t of the
// routed experts belongs to the last expert whose first tile is <= t.
struct TileList {
  int first_tile[kMaxTileExperts + 1];
  int first_row[kMaxTileExperts + 1];
};

__device__ inline Tile tile_at(const TileList& tl, int n_experts, int rows, int routed, int t,
                               int bm) {
  Tile r{-1, 0, 0};
  if (t < routed) {
    int lo = 0, hi = n_experts - 1;  // the last e with first_tile[e] <= t
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (tl.first_tile[mid] <= t) lo = mid;
      else hi = mid - 1;
    }
    r.expert = lo;
    r.start = tl.first_row[lo] + (t - tl.first_tile[lo]) * bm;
    r.count = min(bm, tl.first_row[lo + 1] - r.start);
  } else {
    const int st = t - routed;
    r.expert = n_experts;
    r.start = st * bm;
    r.count = min(bm, rows - st * bm);
  }
  return r;
}

// Item k of XCD x is tile (k / n_nb) * 8 + x, weight-row block k % n_nb:
// the workgroups that share a token tile run on one XCD and share its L2,
// and the live tiles spread over all eight XCDs.  Tiles are numbered with
// the shared expert's (all full but the last) first, so the longest items
// start first and the short routed tiles fill the tail.
// Persistent workgroups (one per CU for 128-row tiles, two for 32-row
// tiles): block b runs on XCD b % 8 and takes that XCD's items b / 8,
// b / 8 + G, ... for G workgroups per XCD.  Each item's tile is found in a
// list built once into LDS, and the next item's tile, rows and first chunks
// go out before this item's epilogue, so no item waits for its own prologue.
#ifndef GEMM_SHORT_PERSISTENT
#define GEMM_SHORT_PERSISTENT 1
#endif
template <int BM> constexpr bool gemm_persistent() {
  return BM == kBMFull || GEMM_SHORT_PERSISTENT;
}
template <int PASS, int BM>
__global__ __launch_bounds__(gemm_waves<BM>() * 64, 2) void gemm_kernel(GemmArgs p) {
  __shared__ Stage<BM> ring[kRing];
  const int n_nb = p.rg_total / kBNGroups;
  const int xcd = (int)(blockIdx.x % 8), slot = (int)(blockIdx.x / 8);
  if constexpr (gemm_persistent<BM>()) {
    __shared__ TileList s_tl;
    __shared__ int s_routed, s_shared;
    if (threadIdx.x < 64) {  // wave 0 counts the tiles (TileMap) and lists them in LDS
      TileMap<BM> m;
      m.load(p.offsets, p.n_experts, p.has_shared, p.rows);
      int ft = m.incl - m.lsum;
      const int per = (p.n_experts + 63) >> 6;  // this lane's experts: e0 .. e0 + per - 1
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int e = m.e0 + i;
        if (i < per && e < p.n_experts) {
          s_tl.first_tile[e] = ft;
          s_tl.first_row[e] = m.o[i];
        }
        ft += m.nt[i];
      }
      if (threadIdx.x == 0) {
        s_tl.first_tile[p.n_experts] = m.routed;
        s_tl.first_row[p.n_experts] = p.offsets[p.n_experts];
        s_routed = m.routed;
        s_shared = m.shared_tiles;
      }
    }
    __syncthreads();
    const int routed = uniform(s_routed), shared_tiles = uniform(s_shared);
    const int n_tiles = routed + shared_tiles;
    const int per_xcd = (int)(gridDim.x / 8);
    auto item = [&](int k, Tile& t, int& nb) -> bool {  // (the same for the whole workgroup)
      const int tile_idx = (k / n_nb) * 8 + xcd;
      if (tile_idx >= n_tiles) return false;
      t = tile_at(s_tl, p.n_experts, p.rows, routed,
                  tile_idx < shared_tiles ? routed + tile_idx : tile_idx - shared_tiles, BM);
      nb = k % n_nb;
      return uniform(t.expert) >= 0;
    };
    int k = slot;
    Tile t;
    int nb;
    if (!item(k, t, nb)) return;
    GemmCtx c = gemm_ctx<PASS, BM>(p, t, nb);
    gemm_issue_first<PASS, BM>(p, c, ring);
    for (;;) {
      // the next item's sorted-list entries are loaded now (they land while
      // this item runs); its tile is found again in LDS, and the entries
      // made rows, when its first chunks go out
      Tile t2;
      int nb2, br2, dr2;  // (set and read only with a next item: no write
                          // to them may wait for the loads in flight)
      const bool more = item(k + per_xcd, t2, nb2);
      if (more) gemm_rows<PASS, BM>(p, t2, br2, dr2);
      auto between = [&]() {
        if (!more) return;  // workgroup-uniform
        ring_barrier();
        Tile tn;
        int nbn;
        item(k + per_xcd, tn, nbn);
        gemm_issue_first<PASS, BM>(p, gemm_ctx_rows<PASS, BM>(p, tn, nbn, br2, dr2), ring);
      };
      gemm_item<PASS, BM>(p, c, ring, between);
      if (!more) break;
      k += per_xcd;
      item(k, t2, nb2);
      c = gemm_ctx_rows<PASS, BM>(p, t2, nb2, br2, dr2);
    }
  } else {
    const int tile_idx = (slot / n_nb) * 8 + xcd;
    if (tile_idx * n_nb >= p.n_items) return;
    TileMap<BM> m;
    m.load(p.offsets, p.n_experts, p.has_shared, p.rows);
    // (the grid is sized from a bound on the tiles: past the last tile the
    // renumbering below would land on the shared expert's tiles again)
    if (tile_idx >= m.n_tiles()) return;
    const Tile t = m.lookup(p.n_experts, p.rows,
                            tile_idx < m.shared_tiles ? m.routed + tile_idx
                                                      : tile_idx - m.shared_tiles);
    if (uniform(t.expert) < 0) return;
    const GemmCtx c = gemm_ctx<PASS, BM>(p, t, slot % n_nb);
    gemm_issue_first<PASS, BM>(p, c, ring);
    gemm_item<PASS, BM>(p, c, ring, []() {});
  }
}

// Raw buffer resource over [base, base + bytes): 48-bit base, stride 0, the
// size in bytes (reads past it return zero), raw dword access.
static u32x4 buffer_rsrc(const void* base, int64_t bytes) {
  const uint64_t ba = (uint64_t)(uintptr_t)base;
  return u32x4{(uint32_t)ba, (uint32_t)(ba >> 32) & 0xFFFFu,
               (uint32_t)std::min<int64_t>(bytes, 0xFFFFFFFFll), 0x00020000u};
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
    // persistent workgroups: at most one per CU (128-row tiles) or two
    // (32-row tiles), a multiple of 8 (one share per XCD); else one per item
    const unsigned items = (unsigned)((tiles + 7) / 8 * 8 * (g.rg_total / kBNGroups));
    const unsigned cus8 = (unsigned)std::max(8, device_cu_count() / 8 * 8);
    const unsigned grid = short_tiles ? (gemm_persistent<kBMShort>() ? std::min(items, 2 * cus8) : items)
                                      : std::min(items, cus8);
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
    const int64_t ld_xp = (int64_t)(L->d_model / 32) * kDigitBlock;
    if (!(stages & MOE_STAGE_REUSE_ACTS)) {
      const int64_t threads = (int64_t)rows * (L->d_model / 32);
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
    g.xp_rsrc = buffer_rsrc(xp, (int64_t)rows * ld_xp);
    g.xs_rsrc = buffer_rsrc(qs, (int64_t)rows * ld_qs * 4);
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
    const int64_t hrows = (int64_t)A + (L->has_shared ? rows : 0);
    d.xp_rsrc = buffer_rsrc(a.h, hrows * a.ld_h);
    d.xs_rsrc = buffer_rsrc(a.hs, hrows * a.ld_hs * 4);
    d.y = (float*)(base + lay.partials);
    d.ld_y = L->d_model;
    launch(GEMM_DOWN, d);
    launch_combine((const float*)(base + lay.partials), ids, w, rows, L->top_k, L->has_shared,
                   L->d_model, y, ld_y, s);
  }
  return launch_status();
}

}  // namespace moe
