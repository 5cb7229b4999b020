/*
 * moe_mxfp4.h -- C ABI of the MI355X (gfx950) routed-expert MXFP4 MoE FFN.
 *
 * The library computes one routed-expert feed-forward layer of a
 * DeepSeek-V4-style model: MXFP4 expert weights (E2M1 nibbles, one E8M0
 * exponent per 32 weights) times int8 activations quantised per 32-element
 * block, as gate/up projection, SwiGLU, group-32 requantisation, down
 * projection and a fixed-order top-k weighted combine with an always-on
 * shared expert.
 *
 * Pages cited:
 *   [gfx90a]  "DeepSeek-V4-Flash on AMD gfx90a: Correctness Recovery and
 *             Inference Performance Engineering" (technical report)
 *   [strix]   "Optimizing DeepSeek V4 Flash Inference on a Strix Halo Pair:
 *             An Engineering Record"
 *   [lucebox] "feat(ds4): add concurrent serving on Strix Halo and R9700 +
 *             Strix" (pull-request review page)
 *
 * Conventions for every call:
 *   - Pointers marked "device" are HIP device pointers; "host" are host
 *     memory.  The caller allocates and frees every buffer, including the
 *     workspace; the library allocates nothing and keeps no state between
 *     calls except per-device caches of the architecture check and a kernel
 *     attribute.  Calls are re-entrant; FFN calls that share a workspace
 *     must not overlap (order them on one stream).
 *   - `stream` is a hipStream_t passed as void* (NULL = default stream).
 *     Work is enqueued asynchronously; results are valid after the stream
 *     is synchronised; buffers must stay alive until then.  No call
 *     synchronises the host or reads device memory back.
 *   - Strides (ld_*) are in elements of the pointed-to type unless stated.
 *   - Return value: MOE_OK (0) or a negative MOE_ERR_*.  All argument
 *     validation happens before anything is enqueued, so a call that fails
 *     validation has no effect.  Nothing aborts, throws or prints.
 *   - Only gfx950 devices are supported (MOE_ERR_UNSUPPORTED_ARCH otherwise).
 *   - Calls are capture-safe: no allocation, no memset nodes, no host sync.
 */
#ifndef MOE_MXFP4_H
#define MOE_MXFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_OK 0
#define MOE_ERR_INVALID_ARG (-1)      /* null pointer, negative count, bad flag */
#define MOE_ERR_SHAPE (-2)            /* a dimension the kernels do not support */
#define MOE_ERR_STRIDE (-3)           /* leading dimension smaller than a row  */
#define MOE_ERR_WORKSPACE (-4)        /* workspace or destination too small    */
#define MOE_ERR_ALIGNMENT (-5)        /* pointer or stride misaligned          */
#define MOE_ERR_UNSUPPORTED_ARCH (-6) /* current device is not gfx950          */
#define MOE_ERR_HIP (-7)              /* a HIP runtime call failed             */

/* Largest top-k the router supports, and the most rows one decode call takes
 * (decode shares one weight pass among all of its rows). */
#define MOE_MAX_TOP_K 16
#define MOE_MAX_DECODE_ROWS 16

/* ------------------------------------------------------------------------ */
/* Weight packing ([gfx90a] §3.2, §6.1: routed experts stay packed FP4 with
 * E8M0 scales, no offline expansion -- Table 4 shows expanding to INT8 costs
 * more in traffic than it saves; [gfx90a] §5.2: layout changes are a
 * one-time load transformation with no decode hot-path cost; §5.3: scales
 * must be read through the address map that matches the packed weights).
 *
 * Canonical input of one matrix W[n_out][d_in] (row = output feature, the
 * contraction runs along d_in):
 *   codes  uint8 [n_out][ld_codes] (device): two E2M1 codes per byte, element
 *          2i in the low nibble, 2i+1 in the high nibble; ld_codes >= d_in/2.
 *   scales uint8 [n_out][ld_scales] (device): E8M0 exponent byte of each run
 *          of 32 consecutive elements of a row; ld_scales >= d_in/32.
 * Supported shapes: n_out % 16 == 0, d_in % 128 == 0.  codes and ld_codes
 * must be 4-byte aligned.  E8M0 bytes 2..240 are within the contract: every
 * block term (the exact integer block dot times 2^(u-128)) is then an exact,
 * finite fp32 value.  From 241 up a block term whose |dot| nears its
 * maximum of 48768 (32 x 127 x 12, in half E2M1 steps) overflows fp32 before
 * the activation scale is applied, so an output can be infinite where the
 * exact result is finite; bytes 0, 1 and above 240 are outside the contract.
 * Outputs are fp32 sums: a row whose exact partial sums exceed fp32's range
 * overflows like any fp32 accumulation.
 *
 * gate_up_interleave = 1 declares a gate/up matrix (n_out = 2F, the F gate
 * rows first, then the F up rows; F % 16 == 0): the packer interleaves
 * 16-row groups of gate and up so one workgroup sees matching gate and up
 * features.  0 packs rows in order (down projections, stand-alone matrices).
 *
 * dst (device, 256-byte aligned) receives moe_packed_bytes(n_out, d_in)
 * bytes in an opaque layout; dst_bytes is its capacity.  The packed blob is
 * position-independent and may be copied.  The canonical input is read-only.
 */
size_t moe_packed_bytes(int n_out, int d_in);
int moe_pack_mxfp4(const uint8_t* codes, int64_t ld_codes, const uint8_t* scales,
                   int64_t ld_scales, int n_out, int d_in, int gate_up_interleave,
                   void* dst, size_t dst_bytes, void* stream);
/* Inverse of moe_pack_mxfp4 (for tests and tools): writes the canonical
 * codes/scales (device) back from a packed blob; padding bytes of the
 * canonical rows (beyond d_in/2 or d_in/32) are left untouched. */
int moe_unpack_mxfp4(const void* src, int n_out, int d_in, int gate_up_interleave,
                     uint8_t* codes, int64_t ld_codes, uint8_t* scales,
                     int64_t ld_scales, void* stream);

/* ------------------------------------------------------------------------ */
/* Activation quantiser ([gfx90a] §6.1: online INT8 quantisation per 32
 * elements; §7.1 item 7: native HIP INT8 quantisation).  The pages do not
 * print the rounding rule; this library uses, per 32-element block of a row,
 *   amax = max |x|,  d = amax / 127 (fp32, correctly rounded),
 *   q = clamp(rint(x / d), -127, 127) (fp32 division, ties to even),
 *   an all-zero block gives d = 0 and q = 0.
 *   x      f32  [rows][ld_x] (device, 16-byte aligned, ld_x % 4 == 0)
 *   q      int8 [rows][ld_q] (device, 8-byte aligned, ld_q % 8 == 0)
 *   scales f32  [rows][ld_s] (device, ld_s >= cols/32)
 * cols % 32 == 0.  rows == 0 is a no-op.  NaN/Inf inputs are outside the
 * contract. */
int moe_quant_act_q8(const float* x, int64_t ld_x, int rows, int cols, int8_t* q,
                     int64_t ld_q, float* scales, int64_t ld_s, void* stream);

/* ------------------------------------------------------------------------ */
/* Router + expert grouping.
 * Routing ([gfx90a] §3.2: top-6 of 256 routed experts; §5.3: membership ties
 * broken by logical id, selected positions in a fixed order): per row, the
 * top_k experts by logit (larger first, ties to the lower index) fill slots
 * 0..top_k-1 in that order; w = sigmoid(logit) renormalised over the chosen
 * slots (fp32).
 * Grouping ([gfx90a] §7.1 item 8: an expert sorter groups assignments so an
 * expert scans its packed weights once): assignment a = row*top_k + slot;
 * counts[e], offsets = exclusive prefix (offsets[E] = rows*top_k), sorted =
 * assignments grouped by expert, ascending a within an expert (stable, so
 * the result is unique and bit-exact; no atomics decide the order).
 *   logits  f32   [rows][ld_l] (device), ld_l >= n_experts
 *   ids     int32 [rows][top_k] (device, out)
 *   w       f32   [rows][top_k] (device, out)
 *   counts  int32 [n_experts] (device, out)
 *   offsets int32 [n_experts+1] (device, out)
 *   sorted  int32 [rows*top_k] (device, out)
 * 1 <= top_k <= min(n_experts, MOE_MAX_TOP_K), 1 <= n_experts <= 512,
 * rows*top_k <= 2^24.  rows == 0 writes zero counts/offsets.  NaN logits are
 * outside the contract.
 * Downstream calls also accept ids/sorted produced elsewhere, where a
 * negative id marks a route this device does not own ([lucebox] "Reduce
 * expert-route overhead": non-owner routes use negative sentinels): such
 * assignments must be absent from sorted (offsets[E] counts only owned
 * ones) and their slots are skipped by the combine. */
int moe_route_group(const float* logits, int64_t ld_l, int rows, int n_experts,
                    int top_k, int32_t* ids, float* w, int32_t* counts,
                    int32_t* offsets, int32_t* sorted, void* stream);

/* Router projection ([gfx90a] Fig. 1 "Router Top-6": the router reads the
 * layer input; Table 4: the router GEMM runs in BF16):
 *   logits[t][e] = sum_k bf16(x[t][k]) * w_router[e][k]   (fp32)
 *   x, ld_x        f32 [rows][ld_x] (device) layer input; each element is
 *                  rounded to BF16 (nearest, ties to even) first
 *   w_router, ld_w BF16 [n_experts][ld_w] (device) router weights
 *   logits, ld_l   f32 [rows][ld_l] (device) out, the input of moe_route_group
 * Every product is exact in fp32; the sum runs in one fixed order, so a
 * logit has the same bits for any rows and tiling: 64 partial sums, partial l
 * folding the elements k = 512 j + 8 l + i (j ascending, then i = 0..7) with
 * fused multiply-adds from zero, then p[l] += p[l ^ m] for m = 32, 16, 8, 4,
 * 2, 1; the logit is p[0].
 * rows >= 0 (0: nothing is read, written or enqueued, and the pointers may
 * be null); d_model % 32 == 0 and <= 8192;
 * 1 <= n_experts <= 4096; ld_x >= d_model, ld_w >= d_model, ld_l >= n_experts
 * (MOE_ERR_STRIDE); x 16-byte aligned with ld_x % 4 == 0, w_router 16-byte
 * aligned with ld_w % 8 == 0 (MOE_ERR_ALIGNMENT).  The caller owns every
 * buffer. */
int moe_router_logits(const float* x, int64_t ld_x, int rows, int d_model,
                      const void* w_router, int64_t ld_w, int n_experts, float* logits,
                      int64_t ld_l, void* stream);

/* Decode-step inputs in one launch: moe_quant_act_q8 of x and
 * moe_route_group of logits for the same rows, which depend on nothing from
 * each other ([gfx90a] Fig. 1: the router and the activation quantisation
 * both read only the layer input; [lucebox] "Reduce expert-route overhead":
 * per-step routing work is overhead on the decode path).  One workgroup
 * routes and groups while the others quantise, so the step pays one launch
 * and one round trip instead of two.  Every output has the same bits as the
 * two separate calls.  Arguments, layouts and checks are theirs:
 *   x, ld_x, cols, q, ld_q, scales, ld_s   as for moe_quant_act_q8 (rows rows)
 *   logits .. sorted                      as for moe_route_group
 * 1 <= rows <= MOE_MAX_DECODE_ROWS (else MOE_ERR_SHAPE, nothing enqueued). */
int moe_decode_prep(const float* x, int64_t ld_x, int cols, int8_t* q, int64_t ld_q,
                    float* scales, int64_t ld_s, const float* logits, int64_t ld_l,
                    int rows, int n_experts, int top_k, int32_t* ids, float* w,
                    int32_t* counts, int32_t* offsets, int32_t* sorted, void* stream);

/* ------------------------------------------------------------------------ */
/* One routed-expert layer ([gfx90a] Fig. 1: router top-6, shared expert and
 * FP4 routed experts gate/up -> down, partials added; §6.1 the INT8-dot MoE
 * decode route; §8.2 group-32 INT8 requant of the intermediate, FP32 top-k
 * partials with a fixed reduction).
 * Packed weights come from moe_pack_mxfp4: gate_up of each expert packed
 * with gate_up_interleave = 1 from [2*d_ff][d_model]; down packed with 0
 * from [d_model][d_ff].  Expert e's blobs are at gate_up + e*gate_up_stride
 * and down + e*down_stride (bytes, multiples of 256); the shared expert's at
 * shared_gate_up / shared_down (used when has_shared != 0). */
typedef struct moe_layer {
  int d_model;    /* D: % 128 == 0 */
  int d_ff;       /* F: % 128 == 0 */
  int n_experts;  /* E routed experts, 1..512 */
  int top_k;      /* 1..MOE_MAX_TOP_K */
  int has_shared; /* 0 or 1: one always-on shared expert with weight 1 */
  const void* gate_up;
  int64_t gate_up_stride;
  const void* down;
  int64_t down_stride;
  const void* shared_gate_up;
  const void* shared_down;
  int flags;      /* MOE_LAYER_* bits; 0 = the default arithmetic */
  /* optional BF16 router weights [n_experts][router_ld] (device; NULL: none).
   * When set, moe_ffn_decode_step computes the logits from x itself
   * (moe_router_logits) into its logits buffer.  16-byte aligned,
   * router_ld >= d_model and % 8 == 0, d_model <= 8192. */
  const void* router;
  int64_t router_ld;
} moe_layer_t;

/* Layer flag: round the SwiGLU intermediate to BF16 (to nearest, ties to even)
 * before its group-32 INT8 requant, as the gfx90a report's down chain reads
 * an already-rounded BF16 intermediate ([gfx90a] §8.2).  Without it the fp32
 * intermediate is requantised directly.  Other flag bits are rejected. */
#define MOE_LAYER_BF16_INTERMEDIATE 1

/* Workspace of one FFN call with `rows` tokens (same for decode/prefill).
 * With A' = rows*top_k + (has_shared ? rows : 0) hidden rows, it holds, in
 * order, each region 256-byte aligned:
 *   hidden codes  [A'][2*d_ff bytes]  requantised intermediate.  Decode calls,
 *                                      and prefill calls off the grouped GEMM
 *                                      (d_model or 2*d_ff not a multiple of
 *                                      256), store each int8 code as the exact
 *                                      bf16 value.  Prefill calls on the GEMM
 *                                      store each run of 32 codes as two E3M2
 *                                      (OCP FP6, bias 3) digit planes in 48
 *                                      bytes, in the first 1.5*d_ff bytes of
 *                                      the row: code = d0 + 16 d1 with d0 in
 *                                      [-8, 7] and d1 in [-8, 8]; plane s is a
 *                                      192-bit little-endian word holding d_s
 *                                      of element e in bits 6e..6e+5; the 48
 *                                      bytes are plane 0 bytes 0-15, plane 1
 *                                      bytes 0-15, plane 0 bytes 16-23, plane
 *                                      1 bytes 16-23.
 *   hidden scales f32  [A'][d_ff/32]
 *   partials      f32  [A'][d_model]  per-slot down projections
 *   activations   [rows][1.5*d_model bytes]  prefill GEMM: each token's int8
 *                                      codes as digit planes, as above
 * Hidden row of routed assignment at sorted position p is p; the shared
 * expert's row for token t is rows*top_k + t.  Partials row of routed
 * assignment a is a; shared: rows*top_k + t.  The byte offsets are returned
 * by moe_ffn_workspace_layout (any output pointer may be NULL).  No region
 * needs initialisation; a call overwrites what it reads. */
size_t moe_ffn_workspace_bytes(const moe_layer_t* L, int rows);
int moe_ffn_workspace_layout(const moe_layer_t* L, int rows, size_t* off_hidden,
                             size_t* off_hidden_scales, size_t* off_partials);

/* Decode ([strix] "The exact-rows contract" and [lucebox] "Tune small HIP
 * batches": each weight byte is read once for all resident rows; [gfx90a]
 * §1/§2: decode and prefill are given different kernel shapes).
 *   q       int8  [rows][ld_q]  (device) activation codes (moe_quant_act_q8)
 *   qs      f32   [rows][ld_qs] (device) their block scales
 *   ids, w  [rows][top_k] (device) from moe_route_group (or sentinel-edited)
 *   offsets int32 [n_experts+1], sorted int32 [rows*top_k] (device)
 *   y       f32   [rows][ld_y]  (device, out, overwritten), ld_y >= d_model
 *   ws      workspace (device, 256-byte aligned), ws_bytes >= the query
 * 1 <= rows <= MOE_MAX_DECODE_ROWS.  q, ld_q as for moe_quant_act_q8; qs and
 * ld_qs 16-byte aligned / % 4 == 0; ld_y % 4 == 0 and y 16-byte aligned.
 * The gate/up projection (+ SwiGLU + requant), the down projection and the
 * combine run as three kernels; with one row the down projection and the
 * combine are one kernel that keeps the partials on chip. */
int moe_ffn_decode(const moe_layer_t* L, const int8_t* q, int64_t ld_q,
                   const float* qs, int64_t ld_qs, int rows, const int32_t* ids,
                   const float* w, const int32_t* offsets, const int32_t* sorted,
                   float* y, int64_t ld_y, void* ws, size_t ws_bytes, void* stream);

/* One decode step from the layer input ([gfx90a] Fig. 1: the router and the
 * quantised activations both come from the layer input and feed the routed
 * experts; [lucebox] "Reduce expert-route overhead": per-step routing work is
 * decode overhead): moe_quant_act_q8(x), moe_route_group(logits) and
 * moe_ffn_decode in one call, every output written as those calls write it
 * (same bits).
 *   x, ld_x      f32 [rows][ld_x] (device) layer input, as for moe_quant_act_q8
 *   logits, ld_l f32 [rows][ld_l] (device) router logits, as for
 *                moe_route_group; with L->router set, an output instead: the
 *                step first writes moe_router_logits of x there
 *   q .. qs      out, as moe_quant_act_q8's (and as moe_ffn_decode requires)
 *   ids .. sorted out, as moe_route_group's
 *   y, ws        as for moe_ffn_decode
 * 1 <= rows <= MOE_MAX_DECODE_ROWS; every check of the three calls applies
 * and runs before anything is enqueued.  With one row (and d_model of 1024,
 * 2048 or 4096) the gate/up kernel quantises and routes the row itself, so
 * the step is two launches; otherwise it is the three calls in order (one
 * more launch, first, with L->router set). */
int moe_ffn_decode_step(const moe_layer_t* L, const float* x, int64_t ld_x,
                        float* logits, int64_t ld_l, int rows, int8_t* q,
                        int64_t ld_q, float* qs, int64_t ld_qs, int32_t* ids, float* w,
                        int32_t* counts, int32_t* offsets, int32_t* sorted, float* y,
                        int64_t ld_y, void* ws, size_t ws_bytes, void* stream);

/* moe_ffn_decode_step without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The workspace lives in a file-scope
 * device array of the library, MOE_NOALLOC_SCRATCH_BYTES (8 MiB) per GPU,
 * held from the first call on that GPU until the process ends; the call
 * itself allocates and frees nothing.  Its address is looked up once per
 * device, on the first call with that device current.  Arguments, checks and
 * results are those of moe_ffn_decode_step (same kernels, same bits), and a
 * layer whose workspace (moe_ffn_workspace_bytes(L, rows)) exceeds the array
 * is rejected with MOE_ERR_WORKSPACE before anything is enqueued (the
 * DeepSeek-V4 layer at 16 rows needs 3.3 MB).  Every call on one GPU shares
 * that GPU's array and nothing in it needs clearing, but calls that overlap
 * on one GPU (several streams, several host threads) race on it: order them
 * on one stream. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
int moe_ffn_decode_step_noalloc(const moe_layer_t* L, const float* x, int64_t ld_x,
                                float* logits, int64_t ld_l, int rows, int8_t* q,
                                int64_t ld_q, float* qs, int64_t ld_qs, int32_t* ids, float* w,
                                int32_t* counts, int32_t* offsets, int32_t* sorted, float* y,
                                int64_t ld_y, void* stream);

/* Prefill chunk: same arguments and results as moe_ffn_decode for any
 * rows >= 1 (tuned for 512..4096).  Grid sizes derive from host-known bounds
 * (rows, top_k, n_experts), never from device counts. */
int moe_ffn_prefill(const moe_layer_t* L, const int8_t* q, int64_t ld_q,
                    const float* qs, int64_t ld_qs, int rows, const int32_t* ids,
                    const float* w, const int32_t* offsets, const int32_t* sorted,
                    float* y, int64_t ld_y, void* ws, size_t ws_bytes, void* stream);

/* The two stages of moe_ffn_decode / moe_ffn_prefill, selectable:
 *   MOE_STAGE_GATE_UP  gate/up projection + SwiGLU + group-32 requant
 *                      (writes the workspace's hidden codes and scales)
 *   MOE_STAGE_DOWN     down projection of the hidden codes into fp32 per-slot
 *                      partials and their fixed-order weighted combine into y
 * Stages communicate only through the workspace, so running them in separate
 * calls (in order, same arguments) gives the same y as one full call; a stage
 * may be re-run on its own, e.g. to time it, once the workspace has seen a
 * GATE_UP stage of the same rows.  `prefill` = 0 selects the decode limits and
 * kernels (rows <= MOE_MAX_DECODE_ROWS), 1 the prefill ones.  Other arguments
 * and errors as moe_ffn_decode; stage_mask must hold GATE_UP or DOWN and no
 * bits beyond MOE_STAGE_ALL | MOE_STAGE_REUSE_ACTS. */
#define MOE_STAGE_GATE_UP 1
#define MOE_STAGE_DOWN 2
#define MOE_STAGE_ALL 3
/* With prefill = 1 and MOE_STAGE_GATE_UP: skip the preparation of the
 * activations (the digit planes of q in the workspace) and reuse what an
 * earlier gate/up stage of the same q left there, so the gate/up GEMM can be
 * timed alone.  Rejected (MOE_ERR_INVALID_ARG) with prefill = 0 or without
 * MOE_STAGE_GATE_UP; no effect off the grouped GEMM. */
#define MOE_STAGE_REUSE_ACTS 4
int moe_ffn_stages(const moe_layer_t* L, int prefill, int stage_mask, const int8_t* q,
                   int64_t ld_q, const float* qs, int64_t ld_qs, int rows,
                   const int32_t* ids, const float* w, const int32_t* offsets,
                   const int32_t* sorted, float* y, int64_t ld_y, void* ws,
                   size_t ws_bytes, void* stream);

/* The same two stages for moe_ffn_decode_step: MOE_STAGE_GATE_UP covers the
 * router projection (with L->router), the quantiser, the routing and the
 * gate/up stage (one launch with one row),
 * MOE_STAGE_DOWN the down stage and the combine, which read what a GATE_UP
 * stage of the same inputs left in the outputs and the workspace.  Arguments
 * and errors as moe_ffn_decode_step; stage_mask as for moe_ffn_stages. */
int moe_ffn_decode_step_stages(const moe_layer_t* L, int stage_mask, const float* x,
                               int64_t ld_x, float* logits, int64_t ld_l, int rows,
                               int8_t* q, int64_t ld_q, float* qs, int64_t ld_qs, int32_t* ids,
                               float* w, int32_t* counts, int32_t* offsets, int32_t* sorted,
                               float* y, int64_t ld_y, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Stand-alone k-row matvec ([strix] "The exact-rows contract": the weights
 * of a 4096x14336 matvec are read once for all K resident rows): y[t][n] =
 * sum_b dot_b(q[t], W[n]) * qs[t][b] * 2^(u[n][b]-128), fp32.
 *   w_packed (device) from moe_pack_mxfp4(..., gate_up_interleave = 0)
 *   q, qs, y as for moe_ffn_decode; 1 <= rows <= MOE_MAX_DECODE_ROWS. */
int moe_matvec_mxfp4(const void* w_packed, int n_out, int d_in, const int8_t* q,
                     int64_t ld_q, const float* qs, int64_t ld_qs, int rows,
                     float* y, int64_t ld_y, void* stream);

/* Test export: dots[t][n][b] (device, int32 [rows][n_out][d_in/32]) = the
 * integer block dot sum_i 2*e2m1(W[n][32b+i]) * q[t][32b+i], computed by the
 * same unpack and matrix-core device functions as the projections.
 * 1 <= rows <= MOE_MAX_DECODE_ROWS. */
int moe_debug_block_dots(const void* w_packed, int n_out, int d_in, const int8_t* q,
                         int64_t ld_q, int rows, int32_t* dots, void* stream);

/* Human-readable name of a status code (static storage). */
const char* moe_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MXFP4_H */
