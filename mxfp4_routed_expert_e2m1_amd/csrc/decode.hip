// decode.hip -- the whole routed-expert layer for a decode step of 8..16 rows
// in one persistent kernel.
//
// At decode sizes the layer does almost no arithmetic per weight byte, so its
// speed is the rate at which expert weights stream from HBM (Strix record,
// "What worked").  Separate gate/up, down and combine kernels each pay a
// launch ramp, a tile lookup and a drain, and the down kernel cannot start
// streaming before the gate/up kernel has drained; here one launch does all
// of it and down weights stream while gate/up items finish.  (With fewer
// rows there is too little work to hide the gate/up -> down dependency and
// the separate kernels are faster; ffn.hip picks.)
//   * Items are numbered gate/up first (tile x 32-feature block), then down
//     (tile x 64-row block); workgroup b of G runs items b, b + G, b + 2G, ...
//     in that order.  No shared queue: one hot atomic word serialises the
//     whole grid (~20 ns per fetch).  A workgroup reaches its down items only
//     after its gate/up items, and gate/up items never wait, so waiting on
//     gate/up items cannot deadlock while all G workgroups are resident; G is
//     capped at the occupancy limit (two per CU).
//   * A gate/up item is the decode projection of ffn.hip: 8 waves split K,
//     one 16x16x32 bf16 matrix-core op per 32-element block (exact block dot
//     times the folded E8M0 scale), fp32 FMA with the activation scale,
//     cross-wave sum in LDS in wave order, then SwiGLU + group-32 int8
//     requant (gfx90a report §8.2).  It stores the hidden codes with
//     device-coherent stores and bumps its tile's counter.
//   * A down item waits until all gate/up items of its tile are counted,
//     then reads the hidden codes with device-coherent loads.  It stores fp32
//     partials (device-coherent) and bumps its row block's counter; the last
//     item of a row block adds the partials of all slots in slot order,
//     shared expert last (fixed order, no atomics on values).
//   * Each wave streams its K chunks through a two-slot register ring that
//     runs across items: while the workgroup reduces and finishes one item,
//     the first two chunks of its next item are already in flight (for a
//     down item only its weights: the hidden codes wait for the counter).
//     Two 8-wave workgroups per CU (<= 128 VGPRs).
//   * Cross-workgroup data only moves through device-coherent (sc1) atomic
//     loads and stores, so no whole-L2 writeback or invalidate is needed.
//   * Every wait is bounded; on timeout the error word is set and the kernel
//     still finishes.  The workgroup that combines the last row block (all
//     items are done by then) re-zeroes the counters, so the next call (or
//     graph replay) starts clean.
#include "ffn_internal.h"

namespace moe {

constexpr int kFusedWaves = 8;
constexpr int kFusedThreads = kFusedWaves * 64;
constexpr int kSpinLimit = 1 << 20;  // about a second of polling, then give up

struct FusedArgs {
  const uint8_t* gu;
  int64_t gu_stride;
  const uint8_t* gu_shared;
  int64_t gu_nib;
  int gu_kc, gu_sc, n_rb_gu;  // n_rb_gu = 2F/64 gate/up items per tile
  const uint8_t* dn;
  int64_t dn_stride;
  const uint8_t* dn_shared;
  int64_t dn_nib;
  int dn_kc, dn_sc, n_rb_dn;  // n_rb_dn = D/64 down items per tile
  const int32_t* offsets;
  const int32_t* sorted;
  const int32_t* ids;
  const float* w;
  int n_experts, top_k, has_shared, rows;
  const int8_t* q;
  int64_t ld_q;
  const float* qs;
  int64_t ld_qs;
  uint16_t* h;
  float* hs;
  int64_t ld_h, ld_hs;
  float* P;
  int64_t ld_p;
  float* y;
  int64_t ld_y;
  int* ctr;
};

// One K chunk of one wave for 4 packed row groups: weight fragments, their
// E8M0 words, activation codes (gate/up: int8 in .xy; down: 8 bf16 hidden
// codes) and the 4 activation block scales.
struct Slot {
  u32x4 a[4];
  uint32_t s[4];
  u32x4 b[4];
  f32x4 d;
};

enum ItemKind : int { ITEM_NONE = 0, ITEM_GATEUP = 1, ITEM_DOWN = 2 };

// A work item as one wave sees it (uniform values in scalar registers).
struct Item {
  int kind, tile, rb, count, start;
  bool shared;
  const uint8_t* nib;  // weight blob of the expert
  const uint8_t* scl;  // its scale region
  int kc_total, sc_total, pr0, kc0;
  int brow;  // activation (gate/up) or hidden (down) row of this lane's column
};

__device__ inline int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

template <int KG, int KD>
__device__ inline Item decode_item(const FusedArgs& p, const int4* s_tiles,
                                   const int* s_sorted, int item, int N1, int N2, int wave,
                                   int lane) {
  Item it{};
  item = uni(item);
  if (item >= N1 + N2) {
    it.kind = ITEM_NONE;
    return it;
  }
  const bool gu = item < N1;
  it.kind = gu ? ITEM_GATEUP : ITEM_DOWN;
  it.tile = uni(gu ? item / p.n_rb_gu : (item - N1) / p.n_rb_dn);
  it.rb = uni(gu ? item % p.n_rb_gu : (item - N1) % p.n_rb_dn);
  const int4 te = s_tiles[it.tile];
  const int expert = uni(te.x);
  it.start = uni(te.y);
  it.count = uni(te.z);
  it.shared = expert == p.n_experts;
  const uint8_t* blob = gu ? (it.shared ? p.gu_shared : p.gu + (int64_t)expert * p.gu_stride)
                           : (it.shared ? p.dn_shared : p.dn + (int64_t)expert * p.dn_stride);
  it.nib = blob;
  it.scl = blob + (gu ? p.gu_nib : p.dn_nib);
  it.kc_total = gu ? p.gu_kc : p.dn_kc;
  it.sc_total = gu ? p.gu_sc : p.dn_sc;
  it.pr0 = it.rb * 4;
  it.kc0 = wave * (gu ? KG : KD);
  const int col = lane & 15;
  const int ccol = col < it.count ? col : 0;
  if (gu) it.brow = it.shared ? it.start + ccol : s_sorted[it.start + ccol] / p.top_k;
  else it.brow = it.shared ? p.rows * p.top_k + it.start + ccol : it.start + ccol;
  return it;
}

// weights + scales of chunk j of the item (and its activation codes for a
// gate/up item; MAY_GU = false when the item is known to be a down item)
template <bool MAY_GU = true>
__device__ inline void issue_chunk(const FusedArgs& p, const Item& it, int j, Slot& sl,
                                   int lane) {
  const int kc = it.kc0 + j;
#pragma unroll
  for (int g = 0; g < 4; ++g)
    sl.a[g] = ((const u32x4*)it.nib)[((int64_t)(it.pr0 + g) * it.kc_total + kc) * 64 + lane];
#pragma unroll
  for (int g = 0; g < 4; ++g)
    sl.s[g] = *(const uint32_t*)(it.scl + (((int64_t)(it.pr0 + g) * it.sc_total + (kc >> 2)) *
                                               16 + (lane & 15)) * 16 + (kc & 3) * 4);
  if (MAY_GU && it.kind == ITEM_GATEUP) {
    const int g8 = 8 * (lane >> 4);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const u32x2 v = *(const u32x2*)(p.q + (int64_t)it.brow * p.ld_q + (int64_t)kc * kChunkK +
                                      jj * kBlock + g8);
      sl.b[jj] = u32x4{v[0], v[1], 0u, 0u};
    }
    sl.d = *(const f32x4*)(p.qs + (int64_t)it.brow * p.ld_qs + (int64_t)kc * 4);
  }
}

// hidden codes and scales of chunk j of a down item: written by other
// workgroups in this launch, so device-coherent loads
__device__ inline void issue_hidden(const FusedArgs& p, const Item& it, int j, Slot& sl,
                                    int lane) {
  const int kc = it.kc0 + j;
  const int g8 = 8 * (lane >> 4);
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const uint64_t* src = (const uint64_t*)(p.h + (int64_t)it.brow * p.ld_h +
                                            (int64_t)kc * kChunkK + jj * kBlock + g8);
    const uint64_t lo = ld_coherent(src), hi = ld_coherent(src + 1);
    sl.b[jj] = u32x4{(uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi, (uint32_t)(hi >> 32)};
  }
  const uint64_t* dsrc = (const uint64_t*)(p.hs + (int64_t)it.brow * p.ld_hs + (int64_t)kc * 4);
  const uint64_t d01 = ld_coherent(dsrc), d23 = ld_coherent(dsrc + 1);
  sl.d = f32x4{__uint_as_float((uint32_t)d01), __uint_as_float((uint32_t)(d01 >> 32)),
               __uint_as_float((uint32_t)d23), __uint_as_float((uint32_t)(d23 >> 32))};
}

// The 16 matrix-core ops of a chunk (4 blocks x 4 row groups).  The empty asm
// pins each block's rescale FMAs: left alone, the compiler sinks them to the
// end of the item and keeps every matrix-core result live (spills).
template <bool DOWN>
__device__ inline void compute_chunk(const Slot& sl, f32x4 (&acc)[4]) {
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const bf16x8 bb = DOWN ? __builtin_bit_cast(bf16x8, sl.b[jj])
                           : i8x8_to_bf16x8(u32x2{sl.b[jj][0], sl.b[jj][1]});
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float sc = e8m0_to_f32((sl.s[g] >> (8 * jj)) & 0xFFu);
      acc[g] += mfma_block(fp4x8_to_bf16x8(sl.a[g][jj], sc), bb) * sl.d[jj];
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) asm volatile("" : "+v"(acc[g]));
  }
}

// Sum the waves' partial tiles in wave order into red[0].
__device__ inline void reduce_waves(float (*red)[16][64], const f32x4 (&acc)[4], int tid) {
  const int wave = tid >> 6, lane = tid & 63;
#pragma unroll
  for (int g = 0; g < 4; ++g)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][g * 4 + i][lane] = acc[g][i];
  lds_barrier();
  for (int e = tid; e < 16 * 64; e += kFusedThreads) {
    float v = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < kFusedWaves; ++w2) v += red[w2][e >> 6][e & 63];
    red[0][e >> 6][e & 63] = v;
  }
  lds_barrier();
}

// SwiGLU + group-32 requant of a gate/up item: thread (column n, feature pair
// fp) of 16 x 16; the 16 threads of a column are one 16-lane group, so amax
// is a 16-lane reduce.  Rows 4rb..4rb+3 of the packed matrix = (gate, up) x 2
// groups of 16 features, i.e. features 32rb .. 32rb+31.
__device__ inline void gateup_epilogue(const FusedArgs& p, const Item& it,
                                       float (*red)[16][64], int tid) {
  if (tid < 256) {
    const int n = tid >> 4, fp = tid & 15;
    float hv[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int f = 2 * fp + u;
      const int gsel = 2 * (f >> 4);
      const int l = 16 * ((f & 15) >> 2) + n;
      const float gv = red[0][gsel * 4 + (f & 3)][l];
      const float uv = red[0][(gsel + 1) * 4 + (f & 3)][l];
      hv[u] = gv / (1.0f + expf(-gv)) * uv;
    }
    float m = fmaxf(fabsf(hv[0]), fabsf(hv[1]));
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 16));
    const float d = m / 127.0f;
    const float q0 = d != 0.f ? fminf(fmaxf(rintf(hv[0] / d), -127.f), 127.f) : 0.f;
    const float q1 = d != 0.f ? fminf(fmaxf(rintf(hv[1] / d), -127.f), 127.f) : 0.f;
    if (n < it.count) {
      const int64_t hrow = it.shared ? (int64_t)p.rows * p.top_k + it.start + n : it.start + n;
      const int f0 = it.rb * 32;
      st_coherent((uint32_t*)(p.h + hrow * p.ld_h + f0 + 2 * fp),
                  (__float_as_uint(q0) >> 16) | (__float_as_uint(q1) & 0xFFFF0000u));
      if (fp == 0) st_coherent((uint32_t*)(p.hs + hrow * p.ld_hs + (f0 >> 5)), __float_as_uint(d));
    }
  }
  wait_stores();
  lds_barrier();
  if (tid == 0) add_coherent(&p.ctr[kCtrTiles + it.tile], 1);
}

// fp32 partials of a down item, then (last item of the row block) the
// fixed-order combine of the block's 64 output rows into y
__device__ inline void down_epilogue(const FusedArgs& p, const Item& it, int n_tiles,
                                     float (*red)[16][64], const int* s_sorted, int* s_flag,
                                     int tid) {
  const int A = p.rows * p.top_k;
  for (int e = tid; e < 16 * 64; e += kFusedThreads) {
    const int gi = e >> 6, l = e & 63, n = l & 15;
    if (n >= it.count) continue;
    const int row = (it.pr0 + (gi >> 2)) * 16 + 4 * (l >> 4) + (gi & 3);
    const int64_t orow = it.shared ? (int64_t)A + it.start + n : s_sorted[it.start + n];
    st_coherent((uint32_t*)(p.P + orow * p.ld_p + row), __float_as_uint(red[0][gi][l]));
  }
  wait_stores();
  lds_barrier();
  if (tid == 0)
    *s_flag = add_coherent(&p.ctr[kCtrTiles + kMaxDecodeTiles + it.rb], 1) == n_tiles - 1;
  lds_barrier();
  if (*s_flag) {
    for (int e = tid; e < p.rows * 64; e += kFusedThreads) {
      const int tok = e >> 6;
      const int row = it.rb * 64 + (e & 63);
      float v = 0.f;
      for (int s2 = 0; s2 < p.top_k; ++s2) {
        const int64_t a2 = (int64_t)tok * p.top_k + s2;
        if (p.ids[a2] < 0) continue;
        v += p.w[a2] * __uint_as_float(ld_coherent((const uint32_t*)(p.P + a2 * p.ld_p + row)));
      }
      if (p.has_shared)
        v += __uint_as_float(
            ld_coherent((const uint32_t*)(p.P + ((int64_t)A + tok) * p.ld_p + row)));
      p.y[(int64_t)tok * p.ld_y + row] = v;
    }
    // the last row block combined: every item of the call is done, so the
    // counters can be re-zeroed for the next call
    wait_stores();
    lds_barrier();
    if (tid == 0) *s_flag = add_coherent(&p.ctr[kCtrCombined], 1) == p.n_rb_dn - 1;
    lds_barrier();
    if (*s_flag) {
      for (int i = tid; i < n_tiles; i += kFusedThreads) st_coherent(&p.ctr[kCtrTiles + i], 0);
      for (int i = tid; i < p.n_rb_dn; i += kFusedThreads)
        st_coherent(&p.ctr[kCtrTiles + kMaxDecodeTiles + i], 0);
      if (tid == 0) st_coherent(&p.ctr[kCtrCombined], 0);
    }
  }
}

// The K loop of the current item over its KP chunks.  Slot c & 1 holds chunk
// c; after computing it the slot is refilled with chunk c + 2 of the stream:
// of this item, or (the last two refills) chunk 0 / 1 of the workgroup's next
// item.  After a down item the next one is a down item too, so it needs no
// activations.
template <int KG, int KD, int KP, bool DOWN>
__device__ inline void k_loop(const FusedArgs& p, const Item& cur, Item& nxt, int next_id,
                              Slot (&sl)[2], f32x4 (&acc)[4], const int4* s_tiles,
                              const int* s_sorted, int N1, int N2, int tid) {
  const int wave = tid >> 6, lane = tid & 63;
#pragma unroll
  for (int c = 0; c < KP; ++c) {
    compute_chunk<DOWN>(sl[c & 1], acc);
    __builtin_amdgcn_sched_barrier(0);
    if (c + 2 < KP) {
      issue_chunk<!DOWN>(p, cur, c + 2, sl[c & 1], lane);
      if (DOWN) issue_hidden(p, cur, c + 2, sl[c & 1], lane);
    } else {
      if (c + 2 == KP) nxt = decode_item<KG, KD>(p, s_tiles, s_sorted, next_id, N1, N2, wave, lane);
      if (nxt.kind != ITEM_NONE) issue_chunk<!DOWN>(p, nxt, c + 2 - KP, sl[c & 1], lane);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int KG, int KD>
__global__ __launch_bounds__(kFusedThreads, 4) void fused_decode_kernel(FusedArgs p) {
  static_assert(KG % 2 == 0 && KD % 2 == 0, "the ring holds two chunks of every item");
  __shared__ float red[kFusedWaves][16][64];
  __shared__ int4 s_tiles[kMaxDecodeTiles];  // expert, start, count of every tile
  __shared__ int s_sorted[MOE_MAX_DECODE_ROWS * MOE_MAX_TOP_K];
  __shared__ int s_flag, s_ntiles;
  const int A = p.rows * p.top_k;  // <= 256 (host-checked)
  // tile table: wave 0 expands the offsets (host-checked: <= kMaxDecodeTiles tiles)
  if (threadIdx.x < 64) {
    TileMap<16> tm;
    tm.load(p.offsets, p.n_experts, p.has_shared, p.rows);
    int idx = tm.incl - tm.lsum;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      for (int r = 0; r < tm.nt[i] && idx < kMaxDecodeTiles; ++r, ++idx)
        s_tiles[idx] = int4{tm.e0 + i, tm.o[i] + 16 * r, min(16, tm.o[i + 1] - tm.o[i] - 16 * r), 0};
    const int st = tm.routed + threadIdx.x;
    if ((int)threadIdx.x < tm.shared_tiles && st < kMaxDecodeTiles)
      s_tiles[st] =
          int4{p.n_experts, 16 * (int)threadIdx.x, min(16, p.rows - 16 * (int)threadIdx.x), 0};
    if (threadIdx.x == 0) s_ntiles = min(tm.n_tiles(), kMaxDecodeTiles);
  }
  for (int i = threadIdx.x; i < A; i += kFusedThreads) s_sorted[i] = p.sorted[i];
  __syncthreads();
  const int n_tiles = s_ntiles;
  const int N1 = n_tiles * p.n_rb_gu, N2 = n_tiles * p.n_rb_dn;
  if (n_tiles == 0) {  // every slot a sentinel and no shared expert: y = 0
    const int D = p.n_rb_dn * 64;
    for (int e = blockIdx.x * kFusedThreads + threadIdx.x; e < p.rows * D;
         e += gridDim.x * kFusedThreads)
      p.y[(int64_t)(e / D) * p.ld_y + e % D] = 0.f;
    return;
  }

  // an opaque copy of the thread id: keeps the compiler from hoisting
  // lane-dependent addresses out of the loops (they would stay live in VGPRs
  // for the whole kernel)
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int wave = tid >> 6, lane = tid & 63;
  const int G = gridDim.x;
  int cur_id = blockIdx.x;
  Item cur = decode_item<KG, KD>(p, s_tiles, s_sorted, cur_id, N1, N2, wave, lane);
  Slot sl[2];
  if (cur.kind != ITEM_NONE) {
    issue_chunk(p, cur, 0, sl[0], lane);
    issue_chunk(p, cur, 1, sl[1], lane);
  }
  // gate/up items, then down items; each phase is one loop
  while (cur.kind == ITEM_GATEUP) {
    asm volatile("" : "+v"(tid));
    f32x4 acc[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) acc[g] = f32x4{0.f, 0.f, 0.f, 0.f};
    Item nxt{};
    k_loop<KG, KD, KG, false>(p, cur, nxt, cur_id + G, sl, acc, s_tiles, s_sorted, N1, N2, tid);
    reduce_waves(red, acc, tid);
    gateup_epilogue(p, cur, red, tid);
    cur = nxt;
    cur_id += G;
  }
  while (cur.kind == ITEM_DOWN) {
    asm volatile("" : "+v"(tid));
    // the item's weights are in flight; wait for its tile's hidden codes
    if (tid == 0) {
      int it = 0;
      while (ld_coherent(&p.ctr[kCtrTiles + cur.tile]) < p.n_rb_gu) {
        __builtin_amdgcn_s_sleep(2);
        if (++it > kSpinLimit) {
          st_coherent(&p.ctr[kCtrError], 1);
          break;
        }
      }
    }
    lds_barrier();
    issue_hidden(p, cur, 0, sl[0], lane);
    issue_hidden(p, cur, 1, sl[1], lane);
    f32x4 acc[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) acc[g] = f32x4{0.f, 0.f, 0.f, 0.f};
    Item nxt{};
    k_loop<KG, KD, KD, true>(p, cur, nxt, cur_id + G, sl, acc, s_tiles, s_sorted, N1, N2, tid);
    reduce_waves(red, acc, tid);
    down_epilogue(p, cur, n_tiles, red, s_sorted, &s_flag, tid);
    cur = nxt;
    cur_id += G;
  }
}

static int decode_tiles_max(const moe_layer_t* L, int rows) {
  const int A = rows * L->top_k;
  return std::min(L->n_experts, A) + (A + 15) / 16 + (L->has_shared ? (rows + 15) / 16 : 0);
}

bool fused_decode_supported(const moe_layer_t* L) {
  const int kg = L->d_model / kChunkK, kd = L->d_ff / kChunkK;  // K chunks of gate/up, down
  auto ok = [](int kc) { return kc == 16 || kc == 32 || kc == 64; };  // 2, 4, 8 per wave
  return ok(kg) && ok(kd) && (2 * L->d_ff) % 64 == 0 && L->d_model % 64 == 0;
}

// Grid: every workgroup resident at once (a workgroup may wait on items of
// any other), two per CU or what the occupancy allows, a multiple of 8 so
// consecutive items spread over the XCDs evenly.
template <int KG, int KD>
static int launch_fused(const FusedArgs& a, int n_cu, hipStream_t s) {
  static int per_cu[64] = {0};  // per device, by device ordinal (< 64)
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return MOE_ERR_HIP;
  if (per_cu[dev] == 0) {
    int occ = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, fused_decode_kernel<KG, KD>,
                                                     kFusedThreads, 0) != hipSuccess || occ < 1)
      return MOE_ERR_HIP;
    per_cu[dev] = std::min(occ, 2);
  }
  const int grid = std::max(8, (per_cu[dev] * n_cu) & ~7);
  hipLaunchKernelGGL((fused_decode_kernel<KG, KD>), dim3(grid), dim3(kFusedThreads), 0, s, a);
  return MOE_OK;
}

int fused_decode_run(const moe_layer_t* L, const int8_t* q, int64_t ld_q, const float* qs,
                     int64_t ld_qs, int rows, const int32_t* ids, const float* w,
                     const int32_t* offsets, const int32_t* sorted, float* y, int64_t ld_y,
                     void* ws, hipStream_t s) {
  const WsLayout lay = ws_layout(L, rows);
  uint8_t* base = (uint8_t*)ws;
  const PackedDims pg(2 * L->d_ff, L->d_model), pdn(L->d_model, L->d_ff);
  FusedArgs a{};
  a.gu = (const uint8_t*)L->gate_up;
  a.gu_stride = L->gate_up_stride;
  a.gu_shared = (const uint8_t*)L->shared_gate_up;
  a.gu_nib = pg.nib_bytes;
  a.gu_kc = (int)pg.kc;
  a.gu_sc = (int)pg.sc;
  a.n_rb_gu = (int)pg.rg / 4;
  a.dn = (const uint8_t*)L->down;
  a.dn_stride = L->down_stride;
  a.dn_shared = (const uint8_t*)L->shared_down;
  a.dn_nib = pdn.nib_bytes;
  a.dn_kc = (int)pdn.kc;
  a.dn_sc = (int)pdn.sc;
  a.n_rb_dn = (int)pdn.rg / 4;
  a.offsets = offsets;
  a.sorted = sorted;
  a.ids = ids;
  a.w = w;
  a.n_experts = L->n_experts;
  a.top_k = L->top_k;
  a.has_shared = L->has_shared;
  a.rows = rows;
  a.q = q;
  a.ld_q = ld_q;
  a.qs = qs;
  a.ld_qs = ld_qs;
  a.h = (uint16_t*)(base + lay.hidden);
  a.hs = (float*)(base + lay.hidden_scales);
  a.ld_h = L->d_ff;
  a.ld_hs = L->d_ff / kBlock;
  a.P = (float*)(base + lay.partials);
  a.ld_p = L->d_model;
  a.y = y;
  a.ld_y = ld_y;
  a.ctr = (int*)(base + lay.counters);
  if (decode_tiles_max(L, rows) > kMaxDecodeTiles) return MOE_ERR_SHAPE;
  int dev = 0, n_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n_cu <= 0)
    return MOE_ERR_HIP;
  const int kg = a.gu_kc / kFusedWaves, kd = a.dn_kc / kFusedWaves;
#define MOE_FUSED_CASE(G, D)                  \
  if (kg == G && kd == D) {                   \
    const int rc = launch_fused<G, D>(a, n_cu, s); \
    return rc != MOE_OK ? rc : launch_status(); \
  }
  MOE_FUSED_CASE(8, 8)
  MOE_FUSED_CASE(8, 4)
  MOE_FUSED_CASE(8, 2)
  MOE_FUSED_CASE(4, 8)
  MOE_FUSED_CASE(4, 4)
  MOE_FUSED_CASE(4, 2)
  MOE_FUSED_CASE(2, 8)
  MOE_FUSED_CASE(2, 4)
  MOE_FUSED_CASE(2, 2)
#undef MOE_FUSED_CASE
  return MOE_ERR_SHAPE;
}

}  // namespace moe
