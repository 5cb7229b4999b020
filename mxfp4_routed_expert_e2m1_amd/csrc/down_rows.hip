// down_rows.hip -- down projection + fixed-order combine for one-row decode
// steps, organised by output rows.
//
// One row touches 7 experts (six routed + the shared one) and the down
// projection's cost is latency: a per-expert kernel has to store fp32
// partials, and a combine kernel has to read them back.
// Here a workgroup owns 16 output rows (one packed row group) of every tile.
// The workgroup copies every hidden row of the step (codes and scales, 4.3
// KB per row at d_ff 2048) into LDS in the same round trip that brings the
// routes and the tile map; then each wave issues its first tile's weight
// chunks and streams them with a fixed number in flight.  Wave w streams row
// group `blockIdx.x` of tiles w, w+8, ... against the LDS copy and keeps the
// 16x16 partial tile in LDS; when all tiles are done the workgroup adds, for
// every token and row, the partials of the token's slots in slot order,
// shared expert last (gfx90a report §8.2: fp32 partials, fixed reduction
// order) and writes y.  No partials leave the chip and no combine kernel runs.
// Same exact block dots as every other projection here (FP4 converter with
// the E8M0 scale folded in, one 16x16x32 bf16 matrix-core op per 32-element
// block, fp32 FMA with the hidden scale).
#include <atomic>
#include <type_traits>

#include "ffn_internal.h"

namespace moe {

constexpr int kDRWaves = 8;
constexpr int kDRThreads = kDRWaves * 64;
constexpr int kDRGroup = 16;  // K chunks of a wave's weight registers (16 KiB)
constexpr int kDRAhead = kDownRowsHead;  // chunks a wave keeps in flight ahead of its math

struct DownRowsArgs {
  const uint8_t* dn;  // routed expert 0 blob
  int64_t dn_stride;
  const uint8_t* dn_shared;
  int64_t nib_bytes;
  int kc_total, sc_total, rg_total;
  const int32_t* offsets;
  const int32_t* sorted;
  const int32_t* ids;
  const float* w;
  int n_experts, top_k, has_shared, rows;
  const uint16_t* h;  // hidden codes (bf16 bits) and scales
  const float* hs;
  int64_t ld_h, ld_hs;
  float* y;
  int64_t ld_y;
};

// Dynamic LDS: partials [n_tiles][16 columns][16 rows] f32, then the hidden
// rows of the step [R][d_ff] bf16 and their scales [R][d_ff/32] f32, R =
// rows * top_k + shared rows, in the workspace's order (row r < rows * top_k
// is sorted position r, row rows * top_k + t the shared expert's row of
// token t).
// NC: 16-byte pieces of hidden codes each thread copies (a constant, so the
// number of loads in flight is known when the copy waits).
// ONE: a one-row step.  Its tiles are the shared expert's (first: it needs
// no route, so wave 0 issues its weights before the ids arrive), then its
// valid slots (ids >= 0) in the stable order by expert (by id, then by
// slot) -- the order the sorted list and offsets of moe_route_group give --
// each of one column.  Every wave finds them from the ids alone: no round
// trip for the offsets and no tile-map scan before its weights go out.
template <int NC, bool ONE>
__global__ __launch_bounds__(kDRThreads, 2) void down_rows_kernel(DownRowsArgs p,
                                                                    int tiles_cap) {
  extern __shared__ __align__(16) float dyn[];
  float* part = dyn;
  __shared__ int4 s_tiles[kMaxDecodeTiles];  // expert, start, count
  __shared__ int s_pos[MOE_MAX_DECODE_ROWS * MOE_MAX_TOP_K];  // assignment -> sorted position
  __shared__ int s_ptile[MOE_MAX_DECODE_ROWS * MOE_MAX_TOP_K];  // sorted position -> tile
  __shared__ float s_wt[MOE_MAX_DECODE_ROWS * MOE_MAX_TOP_K];  // the step's weights
  __shared__ int s_ntiles, s_routed;
  const int tid = threadIdx.x, wave = uniform(tid >> 6), lane = tid & 63;
  const int F = p.kc_total * kChunkK;
  const int rg = blockIdx.x;  // 16 output rows 16*rg .. 16*rg+15
  const int col = lane & 15, g8 = 8 * (lane >> 4);

  // One round trip for everything the weights do not need: the sorted list
  // (positions past the valid ones hold -1), ids and weights, the tile map,
  // and every hidden row of the step (codes and scales).  The copy takes
  // all A = rows * top_k routed rows (sorted positions; those past the
  // valid count are never read) and the shared rows after them, the
  // workspace's own order, so its addresses do not wait for the routes.
  const int n_assign = p.rows * p.top_k;  // <= kDRThreads
  const int R = n_assign + (p.has_shared ? p.rows : 0);
  const int per_row = F / 8;             // 16-byte pieces of codes per row
  const int per_row_s = F / kBlock / 4;  // 16-byte pieces of scales per row
  const int n_pc = R * per_row, n_ps = R * per_row_s;
  // ONE: every wave reads the ids and weights (lane s: slot s); else thread
  // a reads assignment a's, and every wave reads the offsets and finds its
  // own first tile, so its weights go out without a workgroup barrier
  const int ra = ONE ? lane : tid;
  const int ra_c = min(ra, n_assign - 1);  // (unconditional loads)
  const int idv_raw = p.ids[ra_c];
  const float wv_raw = p.w[ra_c];
  const int srt = (!ONE && tid < n_assign) ? p.sorted[tid] : -1;
  TileMap<16> tm;
  if constexpr (!ONE) tm.fetch(p.offsets, p.n_experts);
  // (copy pieces past the end read piece 0 of hidden row 0, which always
  // exists)
  u32x4 cp[NC];
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    const int e = k * kDRThreads + tid;
    const int64_t off = e < n_pc ? (int64_t)(e / per_row) * p.ld_h + (e % per_row) * 8 : 0;
    cp[k] = *(const u32x4*)(p.h + off);
  }
  f32x4 cs;
  {
    const int64_t off = tid < n_ps ? (int64_t)(tid / per_row_s) * p.ld_hs + (tid % per_row_s) * 4 : 0;
    cs = *(const f32x4*)(p.hs + off);
  }
  // What the first weight loads need besides the route -- the blobs' base
  // addresses and the head chunks' offsets (every head starts at chunk 0) --
  // is in scalar registers before the ids arrive.
  const uint32_t blob_bytes = (uint32_t)(p.nib_bytes + (int64_t)p.rg_total * p.sc_total * 256);
  const uint32_t nib_row = (uint32_t)rg * (uint32_t)p.kc_total * 1024u;
  const uint32_t scl_row = (uint32_t)p.nib_bytes + (uint32_t)rg * (uint32_t)p.sc_total * 256u;
  const uint32_t a_lane = (uint32_t)lane * 16u, s_lane = (uint32_t)col * 16u;
  const uint8_t* dn = p.dn;
  const uint8_t* dn_shared = p.dn_shared;
  int64_t dn_stride = p.dn_stride;
  asm volatile("" : "+s"(dn), "+s"(dn_shared), "+s"(dn_stride));
  uint32_t head_a[kDRAhead], head_s[kDRAhead];
#pragma unroll
  for (int kk = 0; kk < kDRAhead; ++kk) {
    const int kc = min(kk, min(kDRGroup, p.kc_total) - 1);
    head_a[kk] = nib_row + (uint32_t)chunk_slot(kc, p.kc_total) * 1024u;
    head_s[kk] = scl_row + (uint32_t)(kc >> 2) * 256u + (uint32_t)(kc & 3) * 4u;
    asm volatile("" : "+s"(head_a[kk]), "+s"(head_s[kk]));
  }
  // this wave's weight stream: row group rg of tile ti, K chunks kg..kg+15,
  // as raw buffer loads (one resource per tile, the chunk's offset in a
  // scalar register, the lane's in a vector register)
  u32x4 a[kDRGroup];
  uint32_t s[kDRGroup];
  auto tile_rsrc = [&](const int4 te) {
    const int ex = uniform(te.x);
    const uint8_t* blob = ex == p.n_experts ? dn_shared : dn + (int64_t)ex * dn_stride;
    return buf_rsrc(blob, blob_bytes);
  };
  // chunk kk of the group at kg (a group shorter than kDRGroup repeats its
  // last chunk, so every issue is unconditional and the count in flight a
  // constant)
  auto issue_chunk = [&](__amdgpu_buffer_rsrc_t r, int kg, int kk) {
    const int kc = kg + min(kk, min(kDRGroup, p.kc_total - kg) - 1);
    a[kk] = buf_load16(r, a_lane, nib_row + (uint32_t)chunk_slot(kc, p.kc_total) * 1024u);
    s[kk] = buf_load4(r, s_lane, scl_row + (uint32_t)(kc >> 2) * 256u + (uint32_t)(kc & 3) * 4u);
  };
  auto issue_head = [&](const int4 te) {  // chunks 0 .. kDRAhead-1
    const __amdgpu_buffer_rsrc_t r = tile_rsrc(te);
#pragma unroll
    for (int kk = 0; kk < kDRAhead; ++kk) {
      a[kk] = buf_load16(r, a_lane, head_a[kk]);
      s[kk] = buf_load4(r, s_lane, head_s[kk]);
    }
  };
  __builtin_amdgcn_sched_barrier(0);  // every load of the round trip goes out first
  // the ids and weights, taken where each path first needs them (the empty
  // asm keeps the compiler from hoisting the wait for them)
  int idv = -1;
  float wv = 0.f;
  auto take_ids = [&]() {
    int r = idv_raw;
    float f = wv_raw;
    asm volatile("" : "+v"(r), "+v"(f));
    idv = ra < n_assign ? r : -1;
    wv = ra < n_assign ? f : 0.f;
  };
  // ONE: lane s's place among the valid slots in the stable order, their
  // number, and the expert of this wave's tile (and of tile 0)
  int rank1 = 0, nv1 = 0;
  auto ranks = [&]() {
    // (a valid slot's key is its expert, then its slot (< 16): unique; a
    // sentinel's sorts after every pick)
    const int key = idv >= 0 ? (idv << 4) | lane : INT_MAX;
    for (int s2 = 0; s2 < p.top_k; ++s2) rank1 += __builtin_amdgcn_readlane(key, s2) < key ? 1 : 0;
    nv1 = (int)__popcll(__ballot(idv >= 0));
  };
  // ONE with a shared expert: its tile comes first, wave 0's, and needs no
  // route, so wave 0 issues it before the ids arrive and ranks after
  const bool early0 = ONE && p.has_shared && wave == 0;
  if constexpr (ONE) {
    if (!early0) {
      take_ids();
      ranks();
    }
  } else {
    take_ids();
    tm.count(p.n_experts, p.has_shared, p.rows);
  }

  // Every wave issues: a wave without a tile repeats tile 0's addresses
  // (they merge with that tile's misses in L2); with no tile at all (no
  // shared expert and every slot a sentinel) routed expert 0's row group,
  // which always exists.  So the issue is unconditional.
  if constexpr (ONE) {
    // ONE: tile 0 is the shared expert's (if any), then the valid slots by
    // place: wave w's routed place is w - has_shared
    const int sh = p.has_shared;
    int4 te0 = int4{0, 0, 0, 0};
    if (early0) {
      te0 = int4{p.n_experts, 0, 1, 0};
    } else {
      const int want = (wave < nv1 + sh ? wave : 0) - sh;
      if (want >= 0 && want < nv1) {
        const uint64_t m = __ballot(idv >= 0 && rank1 == want);
        te0 = int4{__builtin_amdgcn_readlane(idv, __ffsll((unsigned long long)m) - 1), want, 1, 0};
      } else if (sh) {
        te0 = int4{p.n_experts, 0, 1, 0};
      }
    }
    issue_head(te0);
    if (early0) {
      __builtin_amdgcn_sched_barrier(0);
      take_ids();
      ranks();
    }
  } else {
    const int total = tm.n_tiles();
    const Tile t0 = tm.lookup(p.n_experts, p.rows, wave < total ? wave : 0);
    const int4 te0 = t0.expert >= 0 ? int4{t0.expert, t0.start, t0.count, 0} : int4{0, 0, 0, 0};
    issue_head(te0);
  }
  __builtin_amdgcn_sched_barrier(0);

  // the tile map, positions, ids, weights and hidden rows go to LDS while
  // the weights are in flight
  if (ONE && wave == 0) {
    // tile has_shared + r: the valid slot of place r; tile 0 the shared
    // expert's
    if (idv >= 0) s_tiles[p.has_shared + rank1] = int4{idv, rank1, 1, 0};
    if (lane == 0) {
      if (p.has_shared) s_tiles[0] = int4{p.n_experts, 0, 1, 0};
      s_ntiles = nv1 + p.has_shared;
      s_routed = nv1;
    }
  } else if (!ONE && wave == 0) {
    int idx = tm.incl - tm.lsum;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      for (int r = 0; r < tm.nt[i] && idx < kMaxDecodeTiles; ++r, ++idx) {
        const int start = tm.o[i] + 16 * r;
        const int cnt = min(16, tm.o[i + 1] - tm.o[i] - 16 * r);
        s_tiles[idx] = int4{tm.e0 + i, start, cnt, 0};
        for (int c = 0; c < cnt; ++c) s_ptile[start + c] = idx;
      }
    const int st = tm.routed + lane;
    if (lane < tm.shared_tiles && st < kMaxDecodeTiles)
      s_tiles[st] = int4{p.n_experts, 16 * lane, min(16, p.rows - 16 * lane), 0};
    if (lane == 0) {
      s_ntiles = min(tm.n_tiles(), kMaxDecodeTiles);
      s_routed = tm.routed;
    }
  }
  if (!ONE && srt >= 0) s_pos[srt] = tid;
  if (!ONE && tid < n_assign) s_wt[tid] = wv;
  uint16_t* hl = (uint16_t*)(part + (size_t)tiles_cap * 256);
  float* hsl = (float*)(hl + (size_t)R * F);
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    const int e = k * kDRThreads + tid;
    if (e < n_pc) *(u32x4*)(hl + (size_t)e * 8) = cp[k];
  }
  if (tid < n_ps) *(f32x4*)(hsl + (size_t)tid * 4) = cs;
  lds_barrier();  // LDS only: the weights stay in flight
  const int n_tiles = s_ntiles;
  // the combine's index of each assignment's partial row (-1: a sentinel),
  // found now, while the weights are in flight: s_pos[a] becomes
  // (tile * 16 + column) * 16 (only thread a reads or writes entry a)
  if (!ONE && tid < n_assign) {
    int pidx = -1;
    if (idv >= 0) {
      const int pos = s_pos[tid];
      const int ti = s_ptile[pos];
      pidx = (ti * 16 + (pos - s_tiles[ti].y)) * 16;
    }
    s_pos[tid] = pidx;
  }

  for (int ti = wave; ti < n_tiles; ti += kDRWaves) {
    const int4 te = s_tiles[ti];
    const __amdgpu_buffer_rsrc_t rt = tile_rsrc(te);
    const bool shared = te.x == p.n_experts;
    const int ccol = col < te.z ? col : 0;  // columns past the tile repeat column 0
    const int lrow = shared ? n_assign + te.y + ccol : te.y + ccol;  // row of the LDS copy
    auto load_h = [&](int kc, u32x4 (&b)[4], f32x4& d) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b[j] = *(const u32x4*)(hl + (size_t)lrow * F + kc * kChunkK + j * kBlock + g8);
      d = *(const f32x4*)(hsl + (size_t)lrow * (F / kBlock) + kc * 4);
    };
    // Exact rows: the sum over K is taken as the streaming down kernel takes
    // it for 5-16 rows -- a partial per run of 4 chunks (one wave's share
    // there), each from zero in chunk and block order, the partials added in
    // run order -- so a row's output does not depend on how many rows share
    // its step.
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};  // the runs so far
    f32x4 run = {0.f, 0.f, 0.f, 0.f};  // the current run of 4 chunks
    for (int kg = 0; kg < p.kc_total; kg += kDRGroup) {
      if (kg > 0) {  // the head of the first group is already in flight
        const __amdgpu_buffer_rsrc_t r = tile_rsrc(te);
#pragma unroll
        for (int kk = 0; kk < kDRAhead; ++kk) issue_chunk(r, kg, kk);
      }
      const int n_in = min(kDRGroup, p.kc_total - kg);
      u32x4 b[2][4];
      f32x4 d[2];
      load_h(kg, b[0], d[0]);
      // streamed: chunk kk's math waits for chunk kk only, then chunk
      // kk + kDRAhead goes out, so the wave never stalls on a full queue
#pragma unroll
      for (int kk = 0; kk < kDRGroup; ++kk) {
        if (kk < n_in) {
          if (kk % 4 == 0) {  // (kg % 4 == 0) a run starts: fold the last one in
            acc += run;
            run = f32x4{0.f, 0.f, 0.f, 0.f};
          }
          if (kk + 1 < n_in) load_h(kg + kk + 1, b[(kk + 1) & 1], d[(kk + 1) & 1]);
          const u32x4 af = tile_to_bf16_frags(a[kk]);  // (kk < n_in is wave-uniform)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float sc = e8m0_to_f32((s[kk] >> (8 * j)) & 0xFFu);
            const f32x4 r = mfma_block(fp4x8_to_bf16x8(af[j], sc),
                                       __builtin_bit_cast(bf16x8, b[kk & 1][j]));
#pragma unroll
            for (int i = 0; i < 4; ++i) run[i] = fmaf(r[i], d[kk & 1][j], run[i]);
          }
        }
        if (kk + kDRAhead < kDRGroup) {
          __builtin_amdgcn_sched_barrier(0);  // keep the issue after this chunk's math
          issue_chunk(rt, kg, kk + kDRAhead);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    acc += run;
    // lane l holds rows 4*(l/16) + i of column l % 16
#pragma unroll
    for (int i = 0; i < 4; ++i) part[(ti * 16 + col) * 16 + 4 * (lane >> 4) + i] = acc[i];
    if (ti + kDRWaves < n_tiles) issue_head(s_tiles[ti + kDRWaves]);
  }
  __syncthreads();

  // y[t][16 rg + r] = sum over the token's slots in slot order, shared last
  if constexpr (ONE) {
    // (threads 0-15: row r = tid; each slot's partial index and weight come
    // from wave 0's lanes, all of the slots' partials are read at once)
    if (tid < 16) {
      const int pl = idv >= 0 ? (p.has_shared + rank1) * 256 : -1;  // (tile's partial)
      float pv[MOE_MAX_TOP_K];
#pragma unroll
      for (int s2 = 0; s2 < MOE_MAX_TOP_K; ++s2) {
        const int pi = s2 < p.top_k ? __builtin_amdgcn_readlane(pl, s2) : -1;
        pv[s2] = part[max(pi, 0) + tid];
      }
      float v = 0.f;
#pragma unroll
      for (int s2 = 0; s2 < MOE_MAX_TOP_K; ++s2) {
        if (s2 < p.top_k && __builtin_amdgcn_readlane(pl, s2) >= 0)
          v = fmaf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wv), s2)),
                   pv[s2], v);  // as the combine kernel
      }
      if (p.has_shared) v = v + part[tid];  // tile 0
      p.y[16 * rg + tid] = v;
    }
    return;
  }
  for (int e = tid; e < p.rows * 16; e += kDRThreads) {
    const int t = e >> 4, r = e & 15;
    float v = 0.f;
    for (int s2 = 0; s2 < p.top_k; ++s2) {
      const int a2 = t * p.top_k + s2;
      const int pidx = s_pos[a2];
      if (pidx >= 0) v = fmaf(s_wt[a2], part[pidx + r], v);  // as the combine kernel
    }
    if (p.has_shared) {
      const int ti = s_routed + (t >> 4);
      v = v + part[(ti * 16 + (t & 15)) * 16 + r];
    }
    p.y[(int64_t)t * p.ld_y + 16 * rg + r] = v;
  }
}

// Tiles of a decode step with `rows` rows: at most min(E, A) + ceil(A/16)
// routed plus ceil(rows/16) shared.
static int tiles_bound(const moe_layer_t* L, int rows) {
  const int A = rows * L->top_k;
  return std::min(L->n_experts, A) + (A + 15) / 16 + (L->has_shared ? (rows + 15) / 16 : 0);
}

// LDS of one workgroup: partials + every hidden row (codes and scales)
static size_t down_rows_lds(const moe_layer_t* L, int rows) {
  const size_t R = (size_t)rows * L->top_k + (L->has_shared ? rows : 0);
  return (size_t)tiles_bound(L, rows) * 1024 + R * (size_t)L->d_ff * 2 +
         R * (size_t)(L->d_ff / kBlock) * 4;
}

// Copy pieces per thread for the largest hidden-row count of a step.
static int copy_pieces(const moe_layer_t* L, int rows) {
  const int r_max = rows * L->top_k + (L->has_shared ? rows : 0);
  return (r_max * (L->d_ff / 8) + kDRThreads - 1) / kDRThreads;
}

// Rows up to DOWN_ROWS_MAX: measured on MI355X against the streaming down
// kernel + combine (DS-V4 layer): 2 rows 16.6 vs 21.2 us for the down stage,
// whole steps 63.7 vs 66.1 us at 3 rows and 79.2 vs 80.9 us at 4; at 5 rows
// and more the hidden rows no longer fit in LDS next to the partials.  The
// copy takes at most 16 code pieces and one scale piece per thread.
#ifndef DOWN_ROWS_MAX
#define DOWN_ROWS_MAX 4
#endif
bool down_rows_supported(const moe_layer_t* L, int rows) {
  const int r_max = rows * L->top_k + (L->has_shared ? rows : 0);
  return rows <= DOWN_ROWS_MAX && down_rows_lds(L, rows) <= kDownRowsMaxLds &&
         copy_pieces(L, rows) <= 16 && r_max * (L->d_ff / kBlock / 4) <= kDRThreads;
}

int down_rows_run(const moe_layer_t* L, int rows, const int32_t* ids, const float* w,
                  const int32_t* offsets, const int32_t* sorted, const uint16_t* h,
                  const float* hs, float* y, int64_t ld_y, hipStream_t s) {
  const PackedDims pd(L->d_model, L->d_ff);
  DownRowsArgs a{};
  a.dn = (const uint8_t*)L->down;
  a.dn_stride = L->down_stride;
  a.dn_shared = (const uint8_t*)L->shared_down;
  a.nib_bytes = pd.nib_bytes;
  a.kc_total = (int)pd.kc;
  a.sc_total = (int)pd.sc;
  a.rg_total = (int)pd.rg;
  a.offsets = offsets;
  a.sorted = sorted;
  a.ids = ids;
  a.w = w;
  a.n_experts = L->n_experts;
  a.top_k = L->top_k;
  a.has_shared = L->has_shared;
  a.rows = rows;
  a.h = h;
  a.hs = hs;
  a.ld_h = L->d_ff;
  a.ld_hs = L->d_ff / kBlock;
  a.y = y;
  a.ld_y = ld_y;
  const size_t lds = down_rows_lds(L, rows);
  if (lds > (size_t)kDownRowsMaxLds) return MOE_ERR_SHAPE;
  // the copy's pieces per thread, a template constant: 1..8, else 12 or 16
  // (pieces past the end are dummy loads, never stored)
  int nc = copy_pieces(L, rows);
  if (nc < 1 || nc > 16) return MOE_ERR_SHAPE;
  if (nc > 8) nc = nc <= 12 ? 12 : 16;
  // allow more than 64 KiB of dynamic LDS: once per device and variant (an
  // atomic flag: concurrent first calls from several host threads both set
  // the attribute, which is harmless)
  static std::atomic<bool> lds_raised[64][17][2];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return MOE_ERR_HIP;
  const bool one = rows == 1;
  const void* fn = nullptr;
  auto pick = [&](auto nc_c) {
    constexpr int NC = decltype(nc_c)::value;
    fn = one ? (const void*)down_rows_kernel<NC, true> : (const void*)down_rows_kernel<NC, false>;
  };
  switch (nc) {
    case 1: pick(std::integral_constant<int, 1>{}); break;
    case 2: pick(std::integral_constant<int, 2>{}); break;
    case 3: pick(std::integral_constant<int, 3>{}); break;
    case 4: pick(std::integral_constant<int, 4>{}); break;
    case 5: pick(std::integral_constant<int, 5>{}); break;
    case 6: pick(std::integral_constant<int, 6>{}); break;
    case 7: pick(std::integral_constant<int, 7>{}); break;
    case 8: pick(std::integral_constant<int, 8>{}); break;
    case 12: pick(std::integral_constant<int, 12>{}); break;
    default: pick(std::integral_constant<int, 16>{}); break;
  }
  if (!lds_raised[dev][nc][one].load(std::memory_order_acquire)) {
    if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, kDownRowsMaxLds) !=
        hipSuccess)
      return MOE_ERR_HIP;
    lds_raised[dev][nc][one].store(true, std::memory_order_release);
  }
  const int cap = tiles_bound(L, rows);
  void* args[] = {&a, (void*)&cap};
  if (hipLaunchKernel(fn, dim3((unsigned)pd.rg), dim3(kDRThreads), args, lds, s) != hipSuccess)
    return MOE_ERR_HIP;
  return launch_status();
}

}  // namespace moe
