// stream.hip -- persistent decode projections.
//
// The decode passes (gate/up + SwiGLU + requant, and the down projection into
// per-slot partials) and the k-row matvec stream each weight byte once for
// every resident row (Strix record, "The exact-rows contract"; lucebox PR,
// "Tune small HIP batches").  Their cost is HBM time, so the kernel is shaped
// to keep HBM busy rather than around one work item:
//   * An item is one tile (up to 16 token columns of one expert) x 4 packed
//     row groups (64 weight rows; 32 gate/up features).  A workgroup of W
//     waves splits the item's K range, 4 chunks of 128 per wave, exactly as
//     the one-item kernel does, so every block dot, every fp32 FMA and the
//     wave-order reduction are the same operations in the same order.
//   * Workgroups are persistent (one per CU for 8 waves) and walk a static
//     item list (item = blockIdx.x + i * gridDim.x).  A wave's chunks form
//     one sequence over all its items; as soon as it has consumed one chunk
//     it issues the chunk STREAM_AHEAD places further on (into registers
//     whose chunk has already been consumed), which near an item's end is
//     the first chunk of the next item.  So the next item's weights, scales and activations are in
//     flight while the current item is reduced across waves and its epilogue
//     runs.
//   * The cross-wave reduction goes through a double-buffered LDS array with
//     an LDS-only barrier: loads in flight are never drained.
//   * The tile map (the call's expert offsets) and the sorted assignment list
//     are read once per workgroup, not once per item.
#include <algorithm>
#include <type_traits>

#include "ffn_internal.h"

namespace moe {

// Packed row groups per item.  Measured on the 14336 x 4096 matvec (one item
// per workgroup at 4 groups; 1.75 or 3.5 items per workgroup at 2 or 1):
// 10.0 us at 4 groups, 11.2 at 2, 14.6 at 1.
constexpr int kSRGW = 4;
constexpr int kSKPW = 4;  // K chunks of a wave per item
// Chunks a wave keeps in flight ahead of its math, over the item sequence
// (kSKPW: the next item's chunk kk goes out after this item's chunk kk).
#ifndef STREAM_AHEAD
#define STREAM_AHEAD 2
#endif
constexpr int kSAhead = STREAM_AHEAD;
// Chunks per row group of the down matrix that the one-row step's early
// finishers read ahead for the down launch.
#ifndef DOWN_PREFETCH_CHUNKS
#define DOWN_PREFETCH_CHUNKS kDownRowsHead
#endif
constexpr int kDownPrefetch = DOWN_PREFETCH_CHUNKS;
static_assert(kSAhead >= 1 && kSAhead <= kSKPW, "prefetch distance");

// F1 (gate/up only): a one-row step straight from the layer input; see the
// prologue.
template <int PASS, int W, bool F1, int TOPK_PL = 4>
__device__ inline void stream_body(const ProjArgs& p, const StepIn& in) {
  constexpr int RGW = kSRGW, KPW = kSKPW, NT = W * 64;
  static_assert(!F1 || PASS == STREAM_GATEUP, "the one-row step fuses gate/up only");
  static_assert(PASS != STREAM_GATEUP || RGW == 4, "gate/up needs 2 gate/up pairs = 32 features");
  using BV = std::conditional_t<PASS == STREAM_DOWN, u32x4, u32x2>;
  constexpr int kBBytes = PASS == STREAM_DOWN ? 2 : 1;  // bytes per B element
  __shared__ float red[2][W][RGW * 4][64];
  __shared__ int s_sorted[MOE_MAX_DECODE_ROWS * MOE_MAX_TOP_K];
  __shared__ int4 s_tiles[PASS == STREAM_MATVEC ? 1 : kMaxDecodeTiles];  // expert, start, count
  __shared__ int s_ntiles;
  __shared__ uint32_t s_amax[2][16];  // gate/up: per-column amax bits, by reduction buffer
  // F1: the row's int8 codes and scales (K <= 4096), its picked experts
  __shared__ __align__(16) uint8_t s_q8[F1 ? 4096 : 1];
  __shared__ __align__(16) float s_qs[F1 ? 128 : 1];
  __shared__ int s_rid[F1 ? MOE_MAX_TOP_K : 1];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15;
  const int n_rb = p.rg_total / RGW;
  const int n_tok_assign = p.rows * p.top_k;
  const int kc0 = wave * KPW;

  // per-item values, all wave-uniform
  struct Item {
    int expert, start, count, rb;
    bool shared;
    __amdgpu_buffer_rsrc_t w;  // the expert's blob
    uint32_t a_soff, s_soff;   // row group pr0 in its nibble and scale regions
  };
  const uint32_t blob_bytes =
      (uint32_t)(p.nib_bytes + (int64_t)p.rg_total * p.sc_total * 256);
  // tile te's row block rb
  auto item_of = [&](const int4 te, int rb) {
    Item x;
    x.rb = rb;
    const uint8_t* blob = p.w;
    int64_t eoff = 0;
    if constexpr (PASS == STREAM_MATVEC) {
      x.expert = 0;
      x.start = 0;
      x.count = p.rows;
      x.shared = false;
    } else {
      x.expert = uniform(te.x);
      x.start = uniform(te.y);
      x.count = uniform(te.z);
      x.shared = x.expert == p.n_experts;
      if (x.shared) blob = p.w_shared;
      else eoff = (int64_t)x.expert * p.w_stride;
    }
    x.w = buf_rsrc(blob + uniform(eoff), blob_bytes);
    const int pr0 = x.rb * RGW;
    x.a_soff = (uint32_t)pr0 * (uint32_t)p.kc_total * 1024u;
    x.s_soff = (uint32_t)p.nib_bytes + (uint32_t)pr0 * (uint32_t)p.sc_total * 256u;
    return x;
  };
  auto item_at = [&](int i) {
    return item_of(PASS == STREAM_MATVEC ? int4{0, 0, 0, 0} : s_tiles[i / n_rb], i % n_rb);
  };
  // this lane's B row; columns past the tile point one row past the operand,
  // where the buffer range check returns zeros without reading memory (their
  // outputs are never stored)
  auto brow_of = [&](const Item& x) -> int {
    if (col >= x.count) return PASS == STREAM_DOWN ? n_tok_assign + (p.has_shared ? p.rows : 0) : p.rows;
    const int ccol = col;
    if (PASS == STREAM_MATVEC) return ccol;
    if (PASS == STREAM_GATEUP) return x.shared ? x.start + ccol : s_sorted[x.start + ccol] / p.top_k;
    return x.shared ? n_tok_assign + x.start + ccol : x.start + ccol;
  };

  // B operand rows: tokens (MATVEC, GATEUP) or hidden rows (DOWN)
  const int b_rows = PASS == STREAM_DOWN ? n_tok_assign + (p.has_shared ? p.rows : 0) : p.rows;
  const __amdgpu_buffer_rsrc_t rb_b = buf_rsrc(p.b, (uint32_t)(b_rows * p.ld_b * kBBytes));
  const __amdgpu_buffer_rsrc_t rb_d = buf_rsrc(p.bs, (uint32_t)(b_rows * p.ld_bs * 4));
  // lane offsets that do not depend on the item
  // chunk kc0 + kk of a row group sits in slot W * kk + wave (KC = 4W, the
  // interleaved chunk order of the packed layout): at each kk the waves read
  // adjacent tiles
  const uint32_t a_lane = (uint32_t)(wave * 1024 + lane * 16);
  const uint32_t a_gstride = (uint32_t)p.kc_total * 1024u;
  const uint32_t s_lane = (uint32_t)(((kc0 >> 2) * 16 + col) * 16);
  const uint32_t s_gstride = (uint32_t)p.sc_total * 256u;
  const uint32_t b_lane = (uint32_t)((kc0 * kChunkK + 8 * (lane >> 4)) * kBBytes);

  u32x4 a[KPW][RGW];
  u32x4 sv[RGW], sv_n[RGW];
  BV b[KPW][4];
  f32x4 d[KPW];
  // the 16 scale bytes of row `col` for this wave's 4 chunks (kc0 % 4 == 0)
  auto issue_s = [&](const Item& x, u32x4 (&sd)[RGW]) {
#pragma unroll
    for (int g = 0; g < RGW; ++g) sd[g] = buf_load16(x.w, s_lane, x.s_soff + g * s_gstride);
  };
  auto issue_w = [&](const Item& x, int kk) {  // the weights of chunk kk
#pragma unroll
    for (int g = 0; g < RGW; ++g) a[kk][g] = buf_load16(x.w, a_lane + kk * W * 1024, x.a_soff + g * a_gstride);
  };
  auto issue_b = [&](int brow, int kk) {  // the B operand of chunk kk
    if constexpr (F1) {
      // the row from LDS, in every column: columns past the tile's one are
      // computed alike and never stored (and their amax is their own)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b[kk][j] = *(const u32x2*)(s_q8 + (kc0 + kk) * kChunkK + j * kBlock + 8 * (lane >> 4));
      d[kk] = *(const f32x4*)(s_qs + (kc0 + kk) * 4);
    } else {
      const uint32_t bo = (uint32_t)(brow * p.ld_b * kBBytes) + b_lane;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t o = bo + (kk * kChunkK + j * kBlock) * kBBytes;
        if constexpr (PASS == STREAM_DOWN) b[kk][j] = buf_load16(rb_b, o, 0);
        else b[kk][j] = buf_load8(rb_b, o, 0);
      }
      d[kk] = __builtin_bit_cast(f32x4, buf_load16(rb_d, (uint32_t)(brow * p.ld_bs * 4 + (kc0 + kk) * 16), 0));
    }
  };
  auto issue = [&](const Item& x, int brow, int kk) {
    issue_w(x, kk);
    issue_b(brow, kk);
  };
  // The call's tiles (one round trip, wave 0) and sorted list go to LDS.
  int n_items = n_rb;
  int my_id = 0;        // F1, wave 0: lane s < top_k holds pick s
  uint32_t my_key = 0;  // and its logit key
  bool early = false;   // F1: this workgroup's first item went out before the route
  if constexpr (F1) {
    // One row, straight from the layer input.  Wave 0 routes it (top-k of
    // the logits) while the other waves quantise it into LDS (8 elements
    // per piece, K/8 = NT pieces: one per thread of waves 1.., and wave 0's
    // pieces by wave 1), all in one round trip, so no earlier launch has to
    // finish first.  With one row every picked expert is a tile of one
    // column and its sorted position is its rank by expert id (the picks
    // are distinct).  The shared expert's tile comes first: a workgroup
    // whose first item is one of its row blocks (blockIdx.x < n_rb) needs no
    // route for it, so that item's weights and scales go out right after the
    // row's and the logits' own loads, while the route and the quantiser
    // run.  Workgroup 0 also writes what the quantiser and the router would:
    // codes, scales, ids, weights, counts, offsets, sorted (after its first
    // loads go out).
    auto quant_piece = [&](int pc, const float4 x0, const float4 x1) {
      const float v[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
      uint32_t w0, w1;
      const float dq = q8_quant8(v, w0, w1);
      *(u32x2*)(s_q8 + 8 * pc) = u32x2{w0, w1};
      if ((pc & 3) == 0) s_qs[pc >> 2] = dq;
      if (blockIdx.x == 0) {
        *(u32x2*)(in.q + 8 * pc) = u32x2{w0, w1};
        if ((pc & 3) == 0) in.qs[pc >> 2] = dq;
      }
    };
    early = p.has_shared && (int)blockIdx.x < n_rb;
    const float4* xv = (const float4*)in.x;
    float lv[TOPK_PL];
    float4 a0, a1, b0, b1;
    if (wave == 0) {
      topk_load<TOPK_PL>(in.logits, p.n_experts, lv);
    } else {
      a0 = xv[2 * tid];
      a1 = xv[2 * tid + 1];
      if (wave == 1) {
        b0 = xv[2 * lane];
        b1 = xv[2 * lane + 1];
      }
    }
    auto route_or_quantise = [&]() {
    if (wave == 0) {
      topk_pick_loaded<TOPK_PL>(lv, p.n_experts, p.top_k, &my_id, &my_key);
      // (an id < 0 -- the router found no pick, e.g. NaN logits, outside the
      // contract -- is a sentinel as in moe_route_group: in no tile)
      const bool ok = lane < p.top_k && my_id >= 0;
      const int key = ok ? my_id : INT_MAX;  // (the picks are distinct)
      int rank = 0;
      for (int s2 = 0; s2 < p.top_k; ++s2) rank += __builtin_amdgcn_readlane(key, s2) < key ? 1 : 0;
      const int n_valid = (int)__popcll(__ballot(ok));
      if (lane < p.top_k) s_rid[lane] = my_id;
      const int sh = p.has_shared;
      if (ok) {
        s_sorted[rank] = lane;
        s_tiles[sh + rank] = int4{my_id, rank, 1, 0};
      }
      if (lane == 0) {
        if (sh) s_tiles[0] = int4{p.n_experts, 0, 1, 0};
        s_ntiles = n_valid + sh;
      }
    } else {
      quant_piece(tid, a0, a1);
      if (wave == 1) quant_piece(lane, b0, b1);
      if (tid < 96) s_amax[(tid - 64) >> 4][tid & 15] = 0u;
    }
    };
    // (two copies, so each keeps its own load-counter waits: with the early
    // loads in flight they wait only for the row's and the logits' loads)
    if (early) {
      const Item x0 = item_of(int4{p.n_experts, 0, 1, 0}, (int)blockIdx.x);
      __builtin_amdgcn_sched_barrier(0);
      issue_s(x0, sv);
#pragma unroll
      for (int kk = 0; kk < kSAhead; ++kk) issue_w(x0, kk);
      __builtin_amdgcn_sched_barrier(0);
      route_or_quantise();
    } else {
      route_or_quantise();
    }
    lds_barrier();
    n_items = uniform(s_ntiles) * n_rb;
  } else if constexpr (PASS != STREAM_MATVEC) {
    // sorted list and tile map are loaded together: one round trip
    constexpr int NS = (MOE_MAX_DECODE_ROWS * MOE_MAX_TOP_K + NT - 1) / NT;
    int srt[NS];
#pragma unroll
    for (int k = 0; k < NS; ++k) srt[k] = tid + k * NT < n_tok_assign ? p.sorted[tid + k * NT] : 0;
    if (PASS == STREAM_GATEUP && tid < 32) s_amax[tid >> 4][tid & 15] = 0u;
    if (wave == 0) {
      TileMap<16> tm;
      tm.load(p.offsets, p.n_experts, p.has_shared, p.rows);
      int idx = tm.incl - tm.lsum;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        for (int r = 0; r < tm.nt[i]; ++r, ++idx)
          s_tiles[idx] = int4{tm.e0 + i, tm.o[i] + 16 * r, min(16, tm.o[i + 1] - tm.o[i] - 16 * r), 0};
      if (lane < tm.shared_tiles)
        s_tiles[tm.routed + lane] = int4{p.n_experts, 16 * lane, min(16, p.rows - 16 * lane), 0};
      if (lane == 0) s_ntiles = tm.n_tiles();
    }
#pragma unroll
    for (int k = 0; k < NS; ++k)
      if (tid + k * NT < n_tok_assign) s_sorted[tid + k * NT] = srt[k];
    lds_barrier();
    n_items = uniform(s_ntiles) * n_rb;
  }
  // F1, workgroup 0: the router's outputs for the down stage
  auto publish = [&]() {
    if constexpr (F1) {
      if (blockIdx.x != 0) return;
      if (wave == 0) {
        const float my_w = topk_weight(my_key, p.top_k);
        int n_valid = 0;
        for (int s2 = 0; s2 < p.top_k; ++s2) n_valid += __builtin_amdgcn_readlane(my_id, s2) >= 0;
        if (lane < p.top_k) {
          in.ids[lane] = my_id;
          in.w[lane] = my_w;
          if (lane >= n_valid) in.sorted[lane] = -1;
        }
      }
      if (tid < p.top_k && s_rid[tid] >= 0) {
        int rank = 0;
        for (int s2 = 0; s2 < p.top_k; ++s2) rank += s_rid[s2] >= 0 && s_rid[s2] < s_rid[tid];
        in.sorted[rank] = tid;
      }
      for (int e = tid; e <= p.n_experts; e += NT) {
        int below = 0, same = 0;
        for (int s2 = 0; s2 < p.top_k; ++s2) {
          const int o = s_rid[s2];
          below += o >= 0 && o < e ? 1 : 0;
          same += o == e ? 1 : 0;
        }
        in.offsets[e] = below;
        if (e < p.n_experts) in.counts[e] = same;
      }
    }
  };
  int it = blockIdx.x;
  if (it >= n_items) {  // the same for the whole workgroup
    publish();
    return;
  }

  auto compute = [&](int kk, const u32x4 (&sc4)[RGW], f32x4 (&acc)[RGW]) {
    u32x4 af[RGW];
#pragma unroll
    for (int g = 0; g < RGW; ++g) af[g] = tile_to_bf16_frags(a[kk][g]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf16x8 bb;
      if constexpr (PASS == STREAM_DOWN) bb = __builtin_bit_cast(bf16x8, b[kk][j]);
      else bb = i8x8_to_bf16x8(b[kk][j]);
#pragma unroll
      for (int g = 0; g < RGW; ++g) {
        const float sc = e8m0_to_f32((sc4[g][kk] >> (8 * j)) & 0xFFu);
        const f32x4 r = mfma_block(fp4x8_to_bf16x8(af[g][j], sc), bb);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[g][i] = fmaf(r[i], d[kk][j], acc[g][i]);
      }
    }
  };
  // reduced item in red[buf] -> epilogue (fixed wave order, from 0.f)
  auto epilogue = [&](const Item& x, int buf) {
    if constexpr (PASS == STREAM_GATEUP) {
      // Wave w reduces the (pair gp, row i) slices w*S .. w*S+S-1 over all 64
      // lanes (contiguous LDS rows: no bank conflicts).  Lane l of slice
      // (gp, i) holds feature 16 gp + 4 (l / 16) + i of column l % 16; its
      // gate sits in packed group 2 gp, its up in 2 gp + 1.  The group-32
      // amax of a column spans the 8 slices and the 4 lane rows: two lane
      // xors, then an LDS max over the slices (exact, order-free: |h| >= 0
      // compares like its bits).
      constexpr int S = 8 / W;
      const int f0 = x.rb * 32;
      if (wave == 0 && lane < 16) s_amax[buf ^ 1][lane] = 0u;  // last item's slot is free
      float hv[S];
      float mq = 0.f;
#pragma unroll
      for (int s2 = 0; s2 < S; ++s2) {
        const int sl = wave * S + s2, gp = sl >> 2, i = sl & 3;
        float gv = 0.f, uv = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < W; ++w2) gv += red[buf][w2][8 * gp + i][lane];
#pragma unroll
        for (int w2 = 0; w2 < W; ++w2) uv += red[buf][w2][8 * gp + 4 + i][lane];
        hv[s2] = mid_round(swiglu(gv, uv), p.bf16_mid);
        mq = fmaxf(mq, fabsf(hv[s2]));
      }
      mq = fmaxf(mq, __shfl_xor(mq, 16, 64));
      mq = fmaxf(mq, __shfl_xor(mq, 32, 64));
      if (lane < 16) atomicMax(&s_amax[buf][lane], __float_as_uint(mq));
      lds_barrier();
      const float dd = __uint_as_float(s_amax[buf][col]) / 127.0f;
      if (col < x.count) {
        const int64_t hrow = x.shared ? n_tok_assign + x.start + col : x.start + col;
#pragma unroll
        for (int s2 = 0; s2 < S; ++s2) {
          const int sl = wave * S + s2, gp = sl >> 2, i = sl & 3;
          const float qf = q8_code(hv[s2], dd);
          p.h[hrow * p.ld_h + f0 + 16 * gp + 4 * (lane >> 4) + i] =
              (uint16_t)(__float_as_uint(qf) >> 16);
        }
        if (wave == 0 && lane < 16) p.hs[hrow * p.ld_hs + (f0 >> 5)] = dd;
      }
    } else {
      for (int e = tid; e < RGW * 4 * 64; e += NT) {
        const int gi = e >> 6, l = e & 63;
        const int n = l & 15;
        if (n >= x.count) continue;
        float v = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < W; ++w2) v += red[buf][w2][gi][l];
        const int row = (x.rb * RGW + (gi >> 2)) * 16 + 4 * (l >> 4) + (gi & 3);
        int orow;
        if (PASS == STREAM_MATVEC) orow = n;
        else orow = x.shared ? n_tok_assign + x.start + n : s_sorted[x.start + n];
        p.y[(int64_t)orow * p.ld_y + row] = v;
      }
    }
  };

  Item cur = item_at(it);
  int br_cur = brow_of(cur);
  if (F1 && early) {  // (its weights and scales are in flight)
#pragma unroll
    for (int kk = 0; kk < kSAhead; ++kk) issue_b(br_cur, kk);
  } else {
    issue_s(cur, sv);
#pragma unroll
    for (int kk = 0; kk < kSAhead; ++kk) issue(cur, br_cur, kk);
  }
  publish();  // (its first loads are in flight)

  // One item: (NEXT) the next item's scales into the other scale registers,
  // then compute chunk kk and issue the chunk kSAhead places further on in
  // the wave's chunk sequence; reduce; epilogue.
  int buf = 0;
  auto step = [&](auto next_c, const Item& nx, const u32x4 (&sc_cur)[RGW], u32x4 (&sc_nxt)[RGW]) {
    constexpr bool NEXT = decltype(next_c)::value;
    int br_n = 0;
    if constexpr (NEXT) {
      br_n = brow_of(nx);
      issue_s(nx, sc_nxt);
    }
    f32x4 acc[RGW];
#pragma unroll
    for (int g = 0; g < RGW; ++g) acc[g] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KPW; ++kk) {
      compute(kk, sc_cur, acc);
      // then chunk kk + kSAhead of the sequence: this item's, or the next's
      // (its registers are chunk kk's, just consumed, or an older slot)
      const int ka = kk + kSAhead;
      if (ka < KPW || NEXT) {
        // keep the scheduler from moving the loads across the math
        __builtin_amdgcn_sched_barrier(0);
        if (ka < KPW) issue(cur, br_cur, ka);
        else issue(nx, br_n, ka - KPW);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int g = 0; g < RGW; ++g)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[buf][wave][g * 4 + i][lane] = acc[g][i];
    lds_barrier();
    epilogue(cur, buf);
    buf ^= 1;
  };
  // two items per trip so the scale registers alternate without copies
  bool in_sv_n = false;
  for (;;) {
    int in = it + (int)gridDim.x;
    if (in >= n_items) break;
    Item nx = item_at(in);
    step(std::true_type{}, nx, sv, sv_n);
    cur = nx;
    br_cur = brow_of(cur);
    it = in;
    in = it + (int)gridDim.x;
    if (in >= n_items) {
      in_sv_n = true;
      break;
    }
    nx = item_at(in);
    step(std::true_type{}, nx, sv_n, sv);
    cur = nx;
    br_cur = brow_of(cur);
    it = in;
  }
  if (in_sv_n) step(std::false_type{}, cur, sv_n, sv);
  else step(std::false_type{}, cur, sv, sv_n);

  if constexpr (F1) {
    // With grid < n_items < 2 grid, workgroups from n_items - grid on hold
    // one item fewer and finish early.  They read the down launch's head
    // chunks toward the caches: reader r takes row groups r, r + R, ... (R
    // readers; at most 4 each), wave w tile w, the first kDownPrefetch
    // chunks and their scale bytes, two row groups at a time.  With R and
    // n_items - grid multiples of 8, a row group is read on the XCD of the
    // down workgroup that owns it (workgroup i runs on XCD i % 8).  The
    // values are only waited for.
    const int grid = (int)gridDim.x, first1 = n_items - grid, R = grid - first1;
    const int n_tiles = uniform(s_ntiles);
    if (in.dn != nullptr && first1 > 0 && R > 0 && (int)blockIdx.x >= first1 &&
        in.dn_rg <= 4 * R && wave < n_tiles) {
      const int ex = uniform(s_tiles[wave].x);
      const uint8_t* blob = ex == p.n_experts ? in.dn_shared : in.dn + (int64_t)ex * in.dn_stride;
      const __amdgpu_buffer_rsrc_t r =
          buf_rsrc(blob, (uint32_t)(in.dn_nib_bytes + (int64_t)in.dn_rg * in.dn_sc * 256));
      const int rd = (int)blockIdx.x - first1;
#pragma unroll
      for (int i0 = 0; i0 < 4; i0 += 2) {  // two row groups at a time
        u32x4 v[2][kDownPrefetch];
        constexpr int NS = (kDownPrefetch + 3) / 4;  // scale rows (4 chunks each)
        uint32_t sv2[2][NS];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int rg = min(rd + (i0 + i) * R, in.dn_rg - 1);  // (a repeat past the end)
#pragma unroll
          for (int kk = 0; kk < kDownPrefetch; ++kk) {
            const int kc = min(kk, in.dn_kc - 1);
            v[i][kk] = buf_load16(r, (uint32_t)lane * 16u,
                                  (uint32_t)(rg * in.dn_kc + chunk_slot(kc, in.dn_kc)) * 1024u);
          }
#pragma unroll
          for (int j = 0; j < NS; ++j)
            sv2[i][j] = buf_load4(r, (uint32_t)lane * 4u,
                                  (uint32_t)(in.dn_nib_bytes + ((int64_t)rg * in.dn_sc + min(j, in.dn_sc - 1)) * 256));
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
#pragma unroll
          for (int kk = 0; kk < kDownPrefetch; ++kk) asm volatile("" ::"v"(v[i][kk]));
#pragma unroll
          for (int j = 0; j < NS; ++j) asm volatile("" ::"v"(sv2[i][j]));
        }
      }
    }
  }
}

template <int PASS, int W>
__global__ __launch_bounds__(W * 64, 2) void stream_kernel(ProjArgs p) {
  stream_body<PASS, W, false>(p, StepIn{});
}

// PL: logits per lane of the router's wave (n_experts <= 64 * PL)
template <int W, int PL>
__global__ __launch_bounds__(W * 64, 2) void stream_step1_kernel(ProjArgs p, StepIn in) {
  stream_body<STREAM_GATEUP, W, true, PL>(p, in);
}

// KPW = 4 chunks per wave: K/128 = 4W for W = 2, 4, 8 waves.
bool stream_supported(int kc_total, int rg_total) {
  return (kc_total == 8 || kc_total == 16 || kc_total == 32) && rg_total % kSRGW == 0;
}

template <int PASS>
static void launch_stream_w(const ProjArgs& a, int items_bound, hipStream_t s) {
  const int cus = std::max(1, device_cu_count());
  auto grid = [&](int wgs_per_cu) {
    return (unsigned)std::max(1, std::min(items_bound, cus * wgs_per_cu));
  };
  switch (a.kc_total) {
    case 32:
      hipLaunchKernelGGL((stream_kernel<PASS, 8>), dim3(grid(1)), dim3(512), 0, s, a);
      return;
    case 16:
      hipLaunchKernelGGL((stream_kernel<PASS, 4>), dim3(grid(2)), dim3(256), 0, s, a);
      return;
    default:
      hipLaunchKernelGGL((stream_kernel<PASS, 2>), dim3(grid(4)), dim3(128), 0, s, a);
      return;
  }
}

void launch_stream_step1(const ProjArgs& a, const StepIn& in, hipStream_t s) {
  const int items = (a.top_k + a.has_shared) * (a.rg_total / kSRGW);
  const int cus = std::max(1, device_cu_count());
  auto grid = [&](int wgs_per_cu) { return (unsigned)std::max(1, std::min(items, cus * wgs_per_cu)); };
  const bool pl4 = a.n_experts <= 256;
  switch (a.kc_total) {
    case 32:
      if (pl4) hipLaunchKernelGGL((stream_step1_kernel<8, 4>), dim3(grid(1)), dim3(512), 0, s, a, in);
      else hipLaunchKernelGGL((stream_step1_kernel<8, 8>), dim3(grid(1)), dim3(512), 0, s, a, in);
      return;
    case 16:
      if (pl4) hipLaunchKernelGGL((stream_step1_kernel<4, 4>), dim3(grid(2)), dim3(256), 0, s, a, in);
      else hipLaunchKernelGGL((stream_step1_kernel<4, 8>), dim3(grid(2)), dim3(256), 0, s, a, in);
      return;
    default:
      if (pl4) hipLaunchKernelGGL((stream_step1_kernel<2, 4>), dim3(grid(4)), dim3(128), 0, s, a, in);
      else hipLaunchKernelGGL((stream_step1_kernel<2, 8>), dim3(grid(4)), dim3(128), 0, s, a, in);
      return;
  }
}

void launch_stream(int pass, const ProjArgs& a, int tiles_bound, hipStream_t s) {
  const int items_bound = tiles_bound * (a.rg_total / kSRGW);
  if (pass == STREAM_GATEUP) launch_stream_w<STREAM_GATEUP>(a, items_bound, s);
  else if (pass == STREAM_DOWN) launch_stream_w<STREAM_DOWN>(a, items_bound, s);
  else launch_stream_w<STREAM_MATVEC>(a, items_bound, s);
}

}  // namespace moe
