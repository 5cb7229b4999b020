// ffn_internal.h -- workspace layout and the entries ffn.hip shares with
// stream.hip, down_rows.hip and prefill.hip.
#pragma once

#include "common.h"

namespace moe {

// Workspace regions (each 256-byte aligned), for A' = rows*top_k (+ rows when
// a shared expert is present) hidden rows:
//   hidden        [A'][2 d_ff bytes]   requantised intermediate codes: exact
//                                      bf16 values (decode; prefill off the
//                                      GEMM path), or E3M2 digit planes
//                                      [d_ff/32][48 B] in the first 1.5 d_ff
//                                      bytes of the row (prefill GEMM path)
//   hidden_scales f32  [A'][d_ff/32]
//   partials      f32  [A'][d_model]   per-slot down projections
//   act           [rows][1.5 d_model bytes]  prefill GEMM path: each token's
//                                      activation codes as digit planes
struct WsLayout {
  size_t hidden, hidden_scales, partials, act, total;
};

inline size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }


inline WsLayout ws_layout(const moe_layer_t* L, int rows) {
  const size_t hrows = (size_t)rows * L->top_k + (L->has_shared ? (size_t)rows : 0);
  WsLayout w;
  w.hidden = 0;
  w.hidden_scales = w.hidden + round256(hrows * L->d_ff * 2);
  w.partials = w.hidden_scales + round256(hrows * (L->d_ff / kBlock) * 4);
  w.act = w.partials + round256(hrows * L->d_model * 4);
  w.total = w.act + round256((size_t)rows * (L->d_model / kBlock) * 48);
  return w;
}

// Persistent decode projections (stream.hip).  MATVEC: y[n][row] for the rows
// columns of q; GATEUP: SwiGLU + group-32 requant into h/hs; DOWN: per-slot
// fp32 partials into y (assignment rows, shared-expert rows after them).
enum StreamPass : int { STREAM_MATVEC = 0, STREAM_GATEUP = 1, STREAM_DOWN = 2 };

// Arguments of a projection pass (ffn.hip one-item kernels and stream.hip).
struct ProjArgs {
  const uint8_t* w;         // matrix blob (matvec) or routed expert 0 blob
  int64_t w_stride;         // bytes between routed experts
  const uint8_t* w_shared;  // shared expert blob
  int64_t nib_bytes;        // offset of the scale region inside a blob
  int rg_total, kc_total, sc_total;
  const int32_t* offsets;   // [n_experts + 1] (not read by MATVEC)
  const int32_t* sorted;    // [rows * top_k] (not read by MATVEC)
  int n_experts, top_k, has_shared, rows;  // rows <= MOE_MAX_DECODE_ROWS
  const void* b;            // int8 codes (MATVEC, GATEUP) or bf16 hidden codes (DOWN)
  int64_t ld_b;
  const float* bs;
  int64_t ld_bs;
  float* y;                 // MATVEC output / DOWN partials
  int64_t ld_y;
  uint16_t* h;              // GATEUP: requantised hidden codes (bf16 bits) and scales
  float* hs;
  int64_t ld_h, ld_hs;
  int bf16_mid;             // GATEUP: round the intermediate to bf16 before its requant
};

// K/128 in {8, 16, 32} and whole 4-group items
// router projection (router.hip)
int router_args_check(const float* x, int64_t ld_x, int rows, int d_model, const void* w_router,
                      int64_t ld_w, int n_experts, const float* logits, int64_t ld_l);
int launch_router(const float* x, int64_t ld_x, int rows, int d_model, const void* w_router,
                  int64_t ld_w, int n_experts, float* logits, int64_t ld_l, hipStream_t s);

bool stream_supported(int kc_total, int rg_total);
// tiles_bound: an upper bound on the call's tiles (1 for MATVEC)
void launch_stream(int pass, const ProjArgs& a, int tiles_bound, hipStream_t s);

// A one-row decode step from the layer input (x row, router logits): the
// gate/up stream quantises and routes the row itself and writes the
// quantiser's and the router's outputs (device pointers, row 0 only).
struct StepIn {
  const float* x;       // [d_model]
  const float* logits;  // [n_experts]
  int8_t* q;            // out [d_model]
  float* qs;            // out [d_model / 32]
  int32_t* ids;         // out [top_k]
  float* w;             // out [top_k]
  int32_t* counts;      // out [n_experts]
  int32_t* offsets;     // out [n_experts + 1]
  int32_t* sorted;      // out [top_k]
  // The down matrix the one-row down-by-rows launch reads next (dn null:
  // none).  The workgroups holding one item fewer read its head chunks (the
  // first kDownRowsHead chunks of every row group of every tile) toward the
  // caches after their item.
  const uint8_t* dn;
  int64_t dn_stride;
  const uint8_t* dn_shared;
  int64_t dn_nib_bytes;
  int dn_kc, dn_sc, dn_rg;
};
// needs stream_supported(kc_total, rg_total) for the gate/up matrix
void launch_stream_step1(const ProjArgs& a, const StepIn& in, hipStream_t s);

// y = weighted combine of the partials (slot order, shared expert last)
void launch_combine(const float* P, const int32_t* ids, const float* w, int rows, int top_k,
                    int has_shared, int d_model, float* y, int64_t ld_y, hipStream_t s);

// Down projection + combine by output rows for one-row decode steps (partials,
// 1 KiB per tile, and the step's hidden rows in at most kDownRowsMaxLds bytes
// of LDS; a decode step has at most min(E, 256) + 16 + 1 <= kMaxDecodeTiles
// tiles).
constexpr int kDownRowsMaxLds = 150 * 1024;
constexpr int kDownRowsHead = 6;  // chunks a wave issues before its first math
constexpr int kMaxDecodeTiles = 288;
bool down_rows_supported(const moe_layer_t* L, int rows);
int down_rows_run(const moe_layer_t* L, int rows, const int32_t* ids, const float* w,
                  const int32_t* offsets, const int32_t* sorted, const uint16_t* h,
                  const float* hs, float* y, int64_t ld_y, hipStream_t s);

// Prefill stages on the grouped matrix-core GEMM (validated arguments).
int prefill_run(const moe_layer_t* L, int stages, const int8_t* q, int64_t ld_q,
                const float* qs, int64_t ld_qs, int rows, const int32_t* ids, const float* w,
                const int32_t* offsets, const int32_t* sorted, float* y, int64_t ld_y,
                void* ws, hipStream_t s);

}  // namespace moe
