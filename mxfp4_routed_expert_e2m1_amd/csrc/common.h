// common.h -- internal helpers shared by the gfx950 kernels of libmoe_mxfp4.
//
// Packed MXFP4 layout (written by moe_pack_mxfp4, read by every projection).
// A matrix W[N][K] (N % 16 == 0, K % 128 == 0) is cut into 16-row groups
// ("row groups", RG = N/16) and 128-element K chunks (KC = K/128 = four
// 32-element blocks).  The unit of one wave load is a (row group, K chunk)
// tile of 1 KiB nibbles: lane l = 16*j + r holds the 16 canonical bytes of
// row r's block j (32 E2M1 codes, element 2i in the low nibble of byte i).
// A lane's 16 bytes are one row's 32-element block in the form the scaled
// matrix-core instructions take an E2M1 operand slot, so the prefill GEMM
// reads one row's block per lane from LDS copies of the tiles and feeds it
// to the 32x32x64 instruction untouched; the bf16 16x16x32 instruction of
// the decode kernels wants lane
// 16*g + r to hold elements 8g..8g+7 of every block instead, which four
// lane-group swaps per loaded tile produce (tile_to_bf16_frags).
//   nibbles: [RG][KC slots][64 lanes][16 B]
// Within a row group the chunks are stored interleaved by 4 when KC % 4 ==
// 0: chunk c sits in slot (c % 4) * (KC/4) + c / 4.  The decode streams give
// each of their KC/4 waves a run of 4 chunks (wave w: chunks 4w..4w+3) and
// step through the runs together, so at every step the waves of a
// workgroup read KC/4 adjacent tiles (one contiguous burst) instead of tiles
// 4 KiB apart; on MI355X that order streamed 3-10% faster at 1-4 tokens.
// Other KC keep chunk order.
//   scales : [RG][SC][16 rows][16 B]   SC = ceil(K/512); byte i of row r in
//            super-chunk s is the E8M0 byte of block 16*s + i (0-padded).
// Gate/up matrices interleave row groups: packed group 2j = gate group j,
// 2j+1 = up group j, so a workgroup holding 4 consecutive packed groups holds
// gate and up of the same 32 features.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe_mxfp4.h"

namespace moe {

// ------------------------------------------------------------------ types
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int v8i32 __attribute__((ext_vector_type(8)));

constexpr int kRowsPerGroup = 16;
constexpr int kChunkK = 128;     // elements per K chunk (4 blocks)
constexpr int kBlock = 32;       // elements per scale block
constexpr int kSuperBlocks = 16; // blocks per scale super-chunk

// ----------------------------------------------------------- layout sizes
struct PackedDims {
  int64_t rg, kc, sc;
  int64_t nib_bytes, scale_bytes;
  __host__ __device__ PackedDims(int n_out, int d_in) {
    rg = n_out / kRowsPerGroup;
    kc = d_in / kChunkK;
    sc = (d_in / kBlock + kSuperBlocks - 1) / kSuperBlocks;
    nib_bytes = rg * kc * 1024;
    scale_bytes = rg * sc * 256;
  }
  __host__ __device__ int64_t total() const { return nib_bytes + scale_bytes; }
};

// chunk <-> storage slot inside a row group (see the layout above)
__host__ __device__ inline int chunk_slot(int c, int kc) {
  return (kc & 3) ? c : (c & 3) * (kc >> 2) + (c >> 2);
}
__host__ __device__ inline int slot_chunk(int s, int kc) {
  return (kc & 3) ? s : 4 * (s % (kc >> 2)) + s / (kc >> 2);
}

// packed row group -> first canonical row
__host__ __device__ inline int packed_group_src_row(int pr, int n_out, int interleave) {
  if (!interleave) return pr * kRowsPerGroup;
  const int f = n_out / 2;
  return (pr & 1) ? f + (pr >> 1) * kRowsPerGroup : (pr >> 1) * kRowsPerGroup;
}

// ------------------------------------------------------ device primitives
// E8M0 byte -> fp32 2^(u-127) (exact for u in 1..254).  Folded into the
// bf16 A fragment (value x 2^(u-127), E2M1 magnitudes up to 6) it stays
// finite up to u = 252, but the matrix-core result, the block dot times
// 2^(u-128), needs |dot| x 2^(u-128) < 2^128: with |dot| up to 48768
// (32 x 127 x 12, in units of half an E2M1 step) that holds for u <= 240.
__device__ inline float e8m0_to_f32(uint32_t u) { return __uint_as_float(u << 23); }

// A packed tile as loaded (lane 16*j + r: dword g = bytes 4g..4g+3 of row
// r's block j) -> the bf16 instruction's fragments (lane 16*g + r: dword j =
// those same bytes), a 4 x 4 transpose of dwords across the four 16-lane
// groups: one 32-lane swap between registers (0, 2) and (1, 3), then one
// 16-lane swap between (0, 1) and (2, 3).  Every lane must be active.
__device__ inline u32x4 tile_to_bf16_frags(u32x4 t) {
  const auto s02 = __builtin_amdgcn_permlane32_swap(t[0], t[2], false, false);
  const auto s13 = __builtin_amdgcn_permlane32_swap(t[1], t[3], false, false);
  const auto s01 = __builtin_amdgcn_permlane16_swap(s02[0], s13[0], false, false);
  const auto s23 = __builtin_amdgcn_permlane16_swap(s02[1], s13[1], false, false);
  return u32x4{s01[0], s01[1], s23[0], s23[1]};
}

// One A fragment: the 8 E2M1 codes of a dword (element 2i in the low nibble of
// byte i/2) -> 8 bf16 values value*scale, via the gfx950 FP4 converter.
// Exact: E2M1 values have 2 significant bits and scale is a power of two.
__device__ inline bf16x8 fp4x8_to_bf16x8(uint32_t w, float scale) {
  bf16x2 a0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0);
  bf16x2 a1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1);
  bf16x2 a2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2);
  bf16x2 a3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3);
  return bf16x8{a0[0], a0[1], a1[0], a1[1], a2[0], a2[1], a3[0], a3[1]};
}

// 8 int8 codes -> 8 bf16 (exact: |q| <= 127 needs 7 significant bits).
__device__ inline bf16x8 i8x8_to_bf16x8(u32x2 v) {
  uint32_t out[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t word = (p < 2) ? v[0] : v[1];
    const int sh = (p & 1) * 16;
    const float lo = (float)(int32_t)(int8_t)((word >> sh) & 0xFF);
    const float hi = (float)(int32_t)(int8_t)((word >> (sh + 8)) & 0xFF);
    out[p] = (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
  }
  u32x4 r = {out[0], out[1], out[2], out[3]};
  return __builtin_bit_cast(bf16x8, r);
}

// D[16][16] = A[16][32] * B[32][16] on the matrix core, fp32 result, zero C.
// Lane l supplies A row l%16 / B column l%16, K elements 8*(l/16)..+7, and
// receives D rows 4*(l/16)+i (i = 0..3) of column l%16.  With A holding
// value*2^(u-127) and B integer codes every product and partial sum is a
// multiple of 2^(u-128) below 2^16 units, so the result is exact.
__device__ inline f32x4 mfma_block(bf16x8 a, bf16x8 b) {
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, zero, 0, 0, 0);
}

// D[32][32] = A[32][64] * B[64][32] on gfx950's scaled matrix core, zero C,
// with E2M1 codes in A and E3M2 codes in B.  Lane l supplies A row l%32 and
// B column l%32, each with the 32 elements of K slot l/32: A as 16 bytes
// (element 2i in the low nibble of byte i, dwords 0-3), B as 24 bytes
// (element e in bits 6e..6e+5 of dwords 0-5).  Each (row or column, K slot)
// is scaled by 2^(byte - 127) of its lane's scale register: byte J of sa,
// byte 0 of sb.  Lane l receives column l%32 of D, element i at row
// 8 (i/4) + 4 (l/32) + i%4.
typedef float f32x16 __attribute__((ext_vector_type(16)));
template <int J>
__device__ inline f32x16 mfma_fp4_bf6_32(v8i32 a, v8i32 b, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, f32x16{}, 4, 3, J, sa, 0, sb);
}
// j: a compile-time constant after unrolling (the byte select is part of the
// instruction)
__device__ __forceinline__ f32x16 mfma_fp4_bf6_block(v8i32 a, v8i32 b, int j, int sa, int sb) {
  switch (j) {
    case 0: return mfma_fp4_bf6_32<0>(a, b, sa, sb);
    case 1: return mfma_fp4_bf6_32<1>(a, b, sa, sb);
    case 2: return mfma_fp4_bf6_32<2>(a, b, sa, sb);
    default: return mfma_fp4_bf6_32<3>(a, b, sa, sb);
  }
}

__device__ inline int lane_id() { return threadIdx.x & 63; }

// Uniform (wave-wide) values live in scalar registers: the compiler cannot
// see that a value read from LDS or a shuffle is the same in every lane, and
// a buffer resource it cannot prove uniform costs a loop over the lanes at
// every load.  Pointers stay kernel arguments plus a uniform offset, so the
// loads keep their global address space (an integer-to-pointer cast would
// make them flat loads, which also count as LDS traffic).
__device__ inline int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ inline int64_t uniform(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)(uint64_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// exp in fp32 by a fixed, named sequence of operations, so a CPU reference
// can repeat it bit for bit (exact rows): Cody-Waite reduction x = k ln2 + r
// with ln2 split in two (the high part exact in 16 bits), the degree-7 Taylor
// polynomial of exp on |r| <= ln2/2 in Horner form with fused multiply-adds
// (coefficients 1/n! rounded to fp32), then scaling by 2^k.  Within 1 ulp
// of exp over the normal range (0.92 ulp at most); 0 below -104, infinity
// above 89.
__device__ inline float exp_rows(float x) {
  if (!(x >= -104.0f)) return x != x ? x : 0.0f;
  if (x > 89.0f) return __builtin_inff();
  const float k = rintf(x * 0x1.715476p+0f);
  float r = fmaf(-k, 0x1.62e4p-1f, x);
  r = fmaf(-k, 0x1.7f7d1cp-20f, r);
  float p = 0x1.a01a02p-13f;
  p = fmaf(p, r, 0x1.6c16c2p-10f);
  p = fmaf(p, r, 0x1.111112p-7f);
  p = fmaf(p, r, 0x1.555556p-5f);
  p = fmaf(p, r, 0x1.555556p-3f);
  p = fmaf(p, r, 0x1p-1f);
  p = fmaf(p, r, 1.0f);
  p = fmaf(p, r, 1.0f);
  return ldexpf(p, (int)k);
}

// Gate/up epilogue arithmetic, shared by every kernel that finishes a gate/up
// pass so all of them round alike: h = silu(gate) * up, then the group-32
// int8 code of h for the group scale d = amax/127 (0 when the group is zero).
__device__ inline float swiglu(float gate, float up) {
  return gate / (1.0f + exp_rows(-gate)) * up;
}
// BF16 rounding of the intermediate (layer flag MOE_LAYER_BF16_INTERMEDIATE):
// to nearest, ties to even, on the fp32 bits; infinities and NaN unchanged.
__device__ inline float round_bf16(float x) {
  const uint32_t b = __float_as_uint(x);
  if ((b & 0x7F800000u) == 0x7F800000u) return x;
  return __uint_as_float((b + 0x7FFFu + ((b >> 16) & 1u)) & 0xFFFF0000u);
}
__device__ inline float mid_round(float h, int bf16_mid) { return bf16_mid ? round_bf16(h) : h; }
__device__ inline float q8_code(float v, float d) {
  return d != 0.f ? fminf(fmaxf(rintf(v / d), -127.f), 127.f) : 0.f;
}

// Lane moves on DPP (a VALU operand modifier: no LDS round trip).
template <int CTRL>
__device__ inline float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF,
                                                            0xF, false));
}
// DPP move limited to the rows in ROWS (other rows keep v).
template <int CTRL, int ROWS>
__device__ inline float dpp_rows(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, v),
                                                              __builtin_bit_cast(int, v), CTRL,
                                                              ROWS, 0xF, false));
}

// The quantiser's arithmetic for 8 consecutive elements of a 32-element
// block, 4 aligned lanes per block (all 4 must call it together): amax by
// two lane swaps within the quad, d = amax / 127 in fp32, codes packed
// little-endian into w0 (elements 0-3) and w1 (4-7).  Returns d.
__device__ inline float q8_quant8(const float (&v)[8], uint32_t& w0, uint32_t& w1) {
  float m = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) m = fmaxf(m, fabsf(v[k]));
  m = fmaxf(m, dpp_mov<0xB1>(m));  // quad_perm [1,0,3,2]: lane ^ 1
  m = fmaxf(m, dpp_mov<0x4E>(m));  // quad_perm [2,3,0,1]: lane ^ 2
  const float d = m / 127.0f;
  w0 = 0;
  w1 = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint32_t byte = (uint32_t)((int32_t)q8_code(v[k], d)) & 0xFFu;
    if (k < 4) w0 |= byte << (8 * k);
    else w1 |= byte << (8 * (k - 4));
  }
  return d;
}

// Activation quantiser, one thread's share: thread i of a launch-wide index
// handles 8 consecutive elements (i / (cols/8) is the row), 4 aligned lanes
// form one 32-element block (amax by two lane xors), d = amax / 127 in fp32
// and q = clamp(rint(x / d), +-127) (gfx90a report §6.1: INT8 per 32
// elements; the rounding rule is the library's reading).  Threads past the
// data take part in the shuffles and store nothing; cols % 32 == 0 keeps a
// 4-lane group wholly in or out.
__device__ inline void quant_q8_thread(int64_t i, const float* __restrict__ x, int64_t ld_x,
                                       int rows, int cols, int8_t* __restrict__ q, int64_t ld_q,
                                       float* __restrict__ s, int64_t ld_s) {
  const int per_row = cols / 8;
  const int64_t total = (int64_t)rows * per_row;
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
  uint32_t w0, w1;
  const float d = q8_quant8(v, w0, w1);
  if (valid) {
    u32x2 packed = {w0, w1};
    *(u32x2*)(q + (int64_t)r * ld_q + (int64_t)c8 * 8) = packed;
    if ((c8 & 3) == 0) s[(int64_t)r * ld_s + c8 / 4] = d;
  }
}

// Max over the whole wave, returned as a wave-uniform value: row maxima on
// DPP, row broadcasts 15 and 31 fold them into lane 63, read from there.
__device__ inline float wave_max(float v) {
  v = fmaxf(v, dpp_mov<0xB1>(v));        // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_mov<0x4E>(v));        // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_mov<0x141>(v));       // row_half_mirror
  v = fmaxf(v, dpp_mov<0x140>(v));       // row_mirror
  v = fmaxf(v, dpp_rows<0x142, 0xA>(v)); // row_bcast:15 into rows 1, 3
  v = fmaxf(v, dpp_rows<0x143, 0xC>(v)); // row_bcast:31 into rows 2, 3
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// Max over each aligned group of 32 lanes (lanes 0-31, 32-63), returned in
// every lane: quad swaps and the row half-mirror / mirror on DPP give each
// 16-lane row its max, then one lane-xor-16 shuffle combines rows 0/1 and
// 2/3.  Exact: max does not round.  (permlane16_swap(v, v) would do the last
// step without LDS, but this compiler folds the max of its two results away.)
__device__ inline float max32(float v) {
  v = fmaxf(v, dpp_mov<0xB1>(v));   // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_mov<0x4E>(v));   // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_mov<0x141>(v));  // row_half_mirror
  v = fmaxf(v, dpp_mov<0x140>(v));  // row_mirror
  return fmaxf(v, __shfl_xor(v, 16, 32));
}

// Direct global -> LDS load (no registers; counted by vmcnt): lane l of the
// wave writes `bytes` (4 or 16) at lds_base + l * bytes, lds_base uniform.
typedef __attribute__((address_space(3))) void* lds_ptr;
__device__ inline void load_to_lds(const void* src, void* lds_base, int bytes) {
  if (bytes == 16) __builtin_amdgcn_global_load_lds(src, (lds_ptr)lds_base, 16, 0, 0);
  else __builtin_amdgcn_global_load_lds(src, (lds_ptr)lds_base, 4, 0, 0);
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS accesses
// (lgkmcnt 0) but not for its global loads, which stay in flight across it
// (__syncthreads would also wait for vmcnt 0).
__device__ inline void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // vmcnt 63, expcnt 7, lgkmcnt 0
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// inclusive prefix sum over a wave64 on DPP: row shifts 1, 2, 4, 8 (zero
// shifted in) scan each 16-lane row, row broadcasts 15 and 31 carry the row
// totals forward.  Every lane must be active.
template <int CTRL, int ROWS, bool ZERO_FILL>
__device__ inline int dpp_add_src(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROWS, 0xF, ZERO_FILL);
}
__device__ inline int wave_incl_scan(int v) {
  v += dpp_add_src<0x111, 0xF, true>(v);   // row_shr:1
  v += dpp_add_src<0x112, 0xF, true>(v);   // row_shr:2
  v += dpp_add_src<0x114, 0xF, true>(v);   // row_shr:4
  v += dpp_add_src<0x118, 0xF, true>(v);   // row_shr:8
  v += dpp_add_src<0x142, 0xA, false>(v);  // row_bcast:15 into rows 1, 3
  v += dpp_add_src<0x143, 0xC, false>(v);  // row_bcast:31 into rows 2, 3
  return v;
}

// ------------------------------------------------------------- tiles
// A "tile" is up to 16 token columns of one expert that share one weight
// pass.  Tiles run over routed experts in expert order (ceil(count/16)
// tiles each), then over the shared expert (ceil(rows/16) tiles).
struct Tile {
  int expert;  // 0..E-1, or E for the shared expert; -1 if beyond the last
  int start;   // first sorted position (routed) or first token (shared)
  int count;   // 1..TM columns
};

// The offsets of the call, spread over the lanes of a wave: each lane holds
// the offsets of its (up to 8) experts and a wave scan of per-lane tile
// counts.  Loading it is the only memory round trip; lookups are register and
// shuffle work, so a persistent workgroup loads it once.  Tiles hold up to TM
// columns.
template <int TM = 16>
struct TileMap {
  int o[9];    // offsets[e0 .. e0+8] of this lane's experts
  int nt[8];   // tiles of each of them
  int e0;      // first expert of this lane
  int lsum;    // tiles of this lane
  int incl;    // inclusive scan of lsum over the wave
  int routed;  // routed tiles in total
  int shared_tiles;

  __device__ inline void load(const int32_t* __restrict__ offsets, int n_experts, int has_shared,
                              int rows) {
    fetch(offsets, n_experts);
    count(n_experts, has_shared, rows);
  }

  // the loads alone (so a caller can put other loads in the same round trip)
  __device__ inline void fetch(const int32_t* __restrict__ offsets, int n_experts) {
    const int per = (n_experts + 63) >> 6;  // <= 8 (n_experts <= 512)
    e0 = lane_id() * per;
#pragma unroll
    for (int i = 0; i <= 8; ++i) o[i] = (i <= per && e0 + i <= n_experts) ? offsets[e0 + i] : 0;
  }

  // the tile counts, from the fetched offsets
  __device__ inline void count(int n_experts, int has_shared, int rows) {
    const int per = (n_experts + 63) >> 6;
    lsum = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = (i < per && e0 + i < n_experts) ? o[i + 1] - o[i] : 0;
      nt[i] = (c + TM - 1) / TM;
      lsum += nt[i];
    }
    incl = wave_incl_scan(lsum);
    routed = __shfl(incl, 63, 64);
    shared_tiles = has_shared ? (rows + TM - 1) / TM : 0;
  }

  __device__ inline int n_tiles() const { return routed + shared_tiles; }

  // Every lane of the calling wave gets the same answer.
  __device__ inline Tile lookup(int n_experts, int rows, int tile) const {
    Tile t{-1, 0, 0};
    if (tile < routed) {
      int rem = tile - (incl - lsum);
      int se = -1, ss = 0, sc = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (se < 0) {
          if (rem < nt[i]) {
            se = e0 + i;
            ss = o[i] + rem * TM;
            sc = min(TM, o[i + 1] - o[i] - rem * TM);
          } else {
            rem -= nt[i];
          }
        }
      }
      const uint64_t m = __ballot(incl > tile);
      const int L = __ffsll((unsigned long long)m) - 1;
      t.expert = __shfl(se, L, 64);
      t.start = __shfl(ss, L, 64);
      t.count = __shfl(sc, L, 64);
    } else if (tile - routed < shared_tiles) {
      const int st = tile - routed;
      t.expert = n_experts;
      t.start = st * TM;
      t.count = min(TM, rows - st * TM);
    }
    return t;
  }
};

// One-shot lookup; *n_tiles receives the total number of tiles of the call
// (routed + shared).
template <int TM = 16>
__device__ inline Tile find_tile(const int32_t* __restrict__ offsets, int n_experts,
                                 int has_shared, int rows, int tile, int* n_tiles) {
  TileMap<TM> m;
  m.load(offsets, n_experts, has_shared, rows);
  *n_tiles = m.n_tiles();
  return m.lookup(n_experts, rows, tile);
}

// -------------------------------------------------------------- routing
// gfx90a report §3.2 (top-6 of 256 routed experts) and §5.3 (membership
// ties broken by logical id, selected positions in a fixed order).
// Order-preserving integer key of a logit: a larger value gets a larger key,
// -0 and +0 the same one (x + 0 turns -0 into +0), and every real logit a key
// >= 1, so 0 can mark an expert that is absent or already picked.
__device__ inline uint32_t logit_key(float x) {
  const uint32_t b = __float_as_uint(x + 0.0f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ inline float logit_of_key(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Max of an unsigned value over the whole wave (the DPP steps of wave_max).
__device__ inline uint32_t wave_max_u32(uint32_t v) {
  auto f = [](uint32_t u) { return __builtin_bit_cast(float, u); };
  auto u = [](float x) { return __builtin_bit_cast(uint32_t, x); };
  v = max(v, u(dpp_mov<0xB1>(f(v))));
  v = max(v, u(dpp_mov<0x4E>(f(v))));
  v = max(v, u(dpp_mov<0x141>(f(v))));
  v = max(v, u(dpp_mov<0x140>(f(v))));
  v = max(v, u(dpp_rows<0x142, 0xA>(f(v))));
  v = max(v, u(dpp_rows<0x143, 0xC>(f(v))));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Max of a 64-bit unsigned value over the whole wave (the DPP steps of
// wave_max on both halves), returned wave-uniform.
__device__ inline uint64_t wave_max_u64(uint64_t v) {
  auto step = [](uint64_t a, uint64_t b) { return b > a ? b : a; };
  auto hi = [](uint64_t x) { return __builtin_bit_cast(float, (uint32_t)(x >> 32)); };
  auto lo = [](uint64_t x) { return __builtin_bit_cast(float, (uint32_t)x); };
  auto mk = [](float h, float l) {
    return ((uint64_t)__builtin_bit_cast(uint32_t, h) << 32) | __builtin_bit_cast(uint32_t, l);
  };
  v = step(v, mk(dpp_mov<0xB1>(hi(v)), dpp_mov<0xB1>(lo(v))));
  v = step(v, mk(dpp_mov<0x4E>(hi(v)), dpp_mov<0x4E>(lo(v))));
  v = step(v, mk(dpp_mov<0x141>(hi(v)), dpp_mov<0x141>(lo(v))));
  v = step(v, mk(dpp_mov<0x140>(hi(v)), dpp_mov<0x140>(lo(v))));
  v = step(v, mk(dpp_rows<0x142, 0xA>(hi(v)), dpp_rows<0x142, 0xA>(lo(v))));
  v = step(v, mk(dpp_rows<0x143, 0xC>(hi(v)), dpp_rows<0x143, 0xC>(lo(v))));
  const uint32_t h = (uint32_t)__builtin_amdgcn_readlane((int)(v >> 32), 63);
  const uint32_t l = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 63);
  return ((uint64_t)h << 32) | l;
}

// One wave: the top_k picks of one row of logits; lane s < top_k receives
// pick s (its expert and its key).  Expert e sits in lane e % 64, slot
// e / 64.  Each round takes the wave max of the lanes' largest keys, then
// the lowest expert holding it (a ballot per slot: the first slot with a
// match, its lowest lane), whose key becomes 0: the larger key first, the
// lower index among equal keys.  A round that finds no key left (only
// logits whose key is 0, the all-ones NaN, remain: outside the contract)
// yields the sentinel -1, never an expert past the row.  The loads are
// unconditional, the index clamped into the row, so they all go out at
// once.
template <int PER_LANE>
__device__ inline void topk_load(const float* __restrict__ l, int n_experts, float (&lv)[PER_LANE]) {
  const int lane = lane_id();
#pragma unroll
  for (int j = 0; j < PER_LANE; ++j) lv[j] = l[min(lane + 64 * j, n_experts - 1)];
}
// (the rounds, on logits topk_load brought in)
template <int PER_LANE>
__device__ inline void topk_pick_loaded(float (&lv)[PER_LANE], int n_experts, int top_k,
                                        int* my_id, uint32_t* my_key) {
  const int lane = lane_id();
  // (an empty asm reading every value keeps the compiler from moving a load
  // under the select below, where it would wait for each load in turn)
#pragma unroll
  for (int j = 0; j < PER_LANE; ++j) asm volatile("" : "+v"(lv[j]));
  uint32_t k[PER_LANE];
#pragma unroll
  for (int j = 0; j < PER_LANE; ++j) k[j] = lane + 64 * j < n_experts ? logit_key(lv[j]) : 0u;
  uint32_t my_k = 0;
  int id = 0;
  for (int s = 0; s < top_k; ++s) {
    uint32_t lm = k[0];
#pragma unroll
    for (int j = 1; j < PER_LANE; ++j) lm = max(lm, k[j]);
    const uint32_t bk = wave_max_u32(lm);
    int be = -1;
#pragma unroll
    for (int j = PER_LANE - 1; j >= 0; --j) {
      const uint64_t m = __ballot(k[j] == bk);
      if (m != 0ull) be = 64 * j + (__ffsll((unsigned long long)m) - 1);
    }
    if (bk == 0u) be = -1;
#pragma unroll
    for (int j = 0; j < PER_LANE; ++j)
      if (lane + 64 * j == be) k[j] = 0u;
    if (lane == s) {
      my_k = bk;
      id = be;
    }
  }
  *my_id = id;
  *my_key = my_k;
}
template <int PER_LANE>
__device__ inline void topk_pick(const float* __restrict__ l, int n_experts, int top_k,
                                 int* my_id, uint32_t* my_key) {
  float lv[PER_LANE];
  topk_load<PER_LANE>(l, n_experts, lv);
  topk_pick_loaded<PER_LANE>(lv, n_experts, top_k, my_id, my_key);
}

// The picks' weights (lane s < top_k: pick s): each pick's sigmoid in its
// own lane, then their sum in pick order, read lane by lane.
__device__ inline float topk_weight(uint32_t my_key, int top_k) {
  const float my_sig = 1.0f / (1.0f + exp_rows(-logit_of_key(my_key)));
  float sum = 0.f;
  for (int s = 0; s < top_k; ++s)
    sum += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_sig), s));
  return my_sig / sum;
}

// Both: lane s < top_k receives pick s and its weight.
template <int PER_LANE>
__device__ inline void topk_row(const float* __restrict__ l, int n_experts, int top_k,
                                int* my_id, float* my_w) {
  uint32_t my_key;
  topk_pick<PER_LANE>(l, n_experts, top_k, my_id, &my_key);
  *my_w = topk_weight(my_key, top_k);
}

// Raw buffer loads: a wave-uniform resource (base, size) in scalar registers,
// a per-lane byte offset in one vector register, a uniform byte offset in a
// scalar register and a constant in the instruction.  Offsets at or past the
// resource size read as zero (the hardware range check covers the per-lane
// offset and the constant).  The explicit form also keeps the compiler
// from merging or re-deriving addresses per load.
constexpr int kBufDword3 = 0x00020000;  // raw 32-bit data format (gfx9 family)
__device__ inline __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kBufDword3);
}
__device__ inline u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ inline u32x2 buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
}
__device__ inline uint32_t buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}

// ------------------------------------------------------------ host side
bool device_is_gfx950();  // cached per device
int device_cu_count();    // compute units of the current device, cached; 0 if unknown

inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Argument checks of the activation quantiser (MOE_OK or the first error);
// rows == 0 or cols == 0 passes with nothing to do.
int quant_args_check(const float* x, int64_t ld_x, int rows, int cols, const int8_t* q,
                     int64_t ld_q, const float* scales, int64_t ld_s);
// Argument checks of the router + grouping (MOE_OK or the first error).
int route_args_check(const float* logits, int64_t ld_l, int rows, int n_experts, int top_k,
                     const int32_t* ids, const float* w, const int32_t* counts,
                     const int32_t* offsets, const int32_t* sorted);

inline int launch_status() {
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace moe
