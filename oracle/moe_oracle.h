/*
 * moe_oracle.h -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, obviously-correct CPU reference of the routed-expert MXFP4 MoE
 * feed-forward.  Only the tests, the smoke check and the benchmark's CPU
 * baseline may call it; the product library never links or loads it, and it
 * shares no code, header, table or constant with the HIP library.
 *
 * Pages cited (titles as published):
 *   [gfx90a]  "DeepSeek-V4-Flash on AMD gfx90a: Correctness Recovery and
 *             Inference Performance Engineering" (technical report)
 *   [strix]   "Optimizing DeepSeek V4 Flash Inference on a Strix Halo Pair:
 *             An Engineering Record"
 *   [lucebox] "feat(ds4): add concurrent serving on Strix Halo and R9700 +
 *             Strix" (pull-request review page)
 *
 * Canonical (unpacked) layouts used by every oracle function:
 *   codes  uint8 [n_out][ld_c]   two E2M1 codes per byte, element 2i in the
 *                                low nibble, element 2i+1 in the high nibble
 *   scales uint8 [n_out][ld_s]   one E8M0 exponent byte per 32 consecutive
 *                                elements of a row (the contraction axis)
 *   q      int8  [rows][ld_q]    activation codes, one fp32 scale per 32-block
 *   qs     f32   [rows][ld_qs]
 * Gate/up matrices hold the F gate rows first, then the F up rows.
 *
 * Arithmetic: block dots are exact int32; every scaled block term is exact in
 * fp64; sums over blocks are fp64 and rounded once to fp32.  Quantisation
 * decisions (absmax, d = amax/127, rint(x/d)) are taken in fp32, the
 * precision the kernels use.
 *
 * Exact-rows mode ([strix] "The exact-rows contract": every row keeps one
 * fixed operand order), off by default: the same steps in fp32 in one named
 * order, so results can be compared bit for bit -- projections sum the
 * scaled block terms of each run of 16 blocks (512 elements) from zero with
 * fused multiply-adds in block order and add the runs in order; SwiGLU and
 * the router's sigmoid use exp_rows (below) in fp32; router weights sum in
 * pick order; the combine folds the slots with fused multiply-adds in slot
 * order and adds the shared expert last.
 *
 * BF16-intermediate mode ([gfx90a] §8.2: the down chain reads an
 * already-rounded BF16 intermediate), off by default and independent of the
 * exact-rows mode: each SwiGLU output is rounded to the nearest BF16 value,
 * ties to even, before its group-32 requantisation.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORACLE_OK 0
#define ORACLE_EINVAL (-1)

/* threads used by the parallel loops (rows / assignments only, never inside a
 * reduction, so results do not depend on it) */
void oracle_set_threads(int n);
int oracle_get_threads(void);

/* exact-rows mode on (1) or off (0, the fp64 reference); returns the old one */
int oracle_set_exact_rows(int on);

/* BF16-intermediate mode on (1) or off (0); returns the old one */
int oracle_set_bf16_intermediate(int on);

/* y[i] = the BF16 value nearest x[i] (8 significant bits, BF16's exponent
 * range with its subnormals, ties to even; beyond the largest finite BF16
 * plus half its spacing -> infinity; infinities and NaN unchanged), as fp32 */
void oracle_round_bf16(const float* x, int n, float* y);

/* exp in fp32 by a named sequence: Cody-Waite reduction x = k ln2 + r (ln2 as
 * a 16-bit high part plus a low part), the degree-7 Taylor polynomial of exp
 * in r (coefficients 1/n! rounded to fp32) in Horner form with fused
 * multiply-adds, scaling by 2^k; 0 below -104, infinity above 89.  y[i] =
 * exp_rows(x[i]). */
void oracle_exp_rows(const float* x, int n, float* y);

/* E2M1 code -> 2*value (an integer in {0,+-1,+-2,+-3,+-4,+-6,+-8,+-12}) */
int oracle_e2m1_x2(int code);
/* E2M1 code -> value */
double oracle_e2m1(int code);
/* E8M0 byte -> 2^(u-127); u == 255 -> NaN */
double oracle_e8m0(int u);

/* exact int32 dot of one 32-element block: sum_i e2m1_x2(code_i) * q_i */
int32_t oracle_block_dot(const uint8_t* codes16, const int8_t* q32);

/* per-32-block symmetric int8 quantiser (fp32 decisions) */
int oracle_quant_q8(const float* x, int64_t ld_x, int rows, int cols,
                    int8_t* q, int64_t ld_q, float* s, int64_t ld_s);

/* top-k routing on logits + sigmoid renormalised weights */
int oracle_route(const float* logits, int64_t ld_l, int rows, int n_experts,
                 int top_k, int32_t* ids, float* w);

/* router projection ([gfx90a] Fig. 1 "Router Top-6"; Table 4: a BF16 router
 * GEMM): logits[t][e] = sum_k bf16(x[t][k]) * wr[e][k], x fp32 [rows][ld_x]
 * rounded to BF16 (oracle_round_bf16), wr BF16 bits [n_experts][ld_w].  Every
 * product is exact in fp32.  Default: fp64 sum rounded once to fp32.
 * Exact-rows mode: 64 partial sums, partial l taking k = 512 j + 8 l + i
 * (j ascending, then i = 0..7) with fused multiply-adds from zero, then
 * p[l] += p[l ^ m] for m = 32, 16, 8, 4, 2, 1; the logit is p[0].
 * d_model % 32 == 0. */
int oracle_router_logits(const float* x, int64_t ld_x, int rows, int d_model,
                         const uint16_t* wr, int64_t ld_w, int n_experts,
                         float* logits, int64_t ld_l);

/* per-expert histogram, exclusive prefix, stable permutation */
int oracle_group(const int32_t* ids, int n_assign, int n_experts,
                 int32_t* counts, int32_t* offsets, int32_t* sorted);

/* y[t][n] = (float) sum_b dot_b * qs[t][b] * 2^(u[n][b]-128) */
int oracle_matvec(const uint8_t* codes, int64_t ld_c, const uint8_t* scales,
                  int64_t ld_s, int n_out, int d_in, const int8_t* q,
                  int64_t ld_q, const float* qs, int64_t ld_qs, int rows,
                  float* y, int64_t ld_y);

/* dots[t][n][b] = block dot of row n, activation row t, block b */
int oracle_block_dots(const uint8_t* codes, int64_t ld_c, int n_out, int d_in,
                      const int8_t* q, int64_t ld_q, int rows, int32_t* dots);

/* h = (float)(silu(g) * u), silu(z) = z / (1 + exp(-z)), in fp64 */
void oracle_swiglu(const float* g, const float* u, int n, float* h);

/* gate/up projection + SwiGLU for one expert: h[t][f], f < d_ff (rounded
 * to BF16 in the BF16-intermediate mode) */
int oracle_expert_hidden(const uint8_t* gu_codes, const uint8_t* gu_scales,
                         int d_model, int d_ff, const int8_t* q, int64_t ld_q,
                         const float* qs, int64_t ld_qs, int rows, float* h,
                         int64_t ld_h);

/* fixed-slot-order weighted combine of per-slot partials.
 * Y is [rows][top_k + has_shared][d_model]; slots with ids < 0 are skipped;
 * the shared slot (index top_k) has weight 1. */
int oracle_combine(int rows, int top_k, int has_shared, int d_model,
                   const int32_t* ids, const float* w, const float* Y,
                   float* y, int64_t ld_y);

/* Whole routed-expert FFN layer.  Expert e's canonical weights are reached
 * through the pointer tables (entry n_experts is the shared expert); entries
 * for experts no route touches may be NULL.  Optional outputs (may be NULL):
 *   h_out  f32  [rows*(top_k+1)][d_ff]     SwiGLU output before requant
 *   hq_out int8 [rows*(top_k+1)][d_ff]     requantised intermediate
 *   hs_out f32  [rows*(top_k+1)][d_ff/32]
 *   Y_out  f32  [rows*(top_k+1)][d_model]  per-slot down projections
 * Row (t*(top_k+1) + i) holds slot i of token t; slot top_k is the shared
 * expert.  If hq_in/hs_in are given (same layout), steps up to the requant
 * are skipped and the down projection starts from those codes. */
int oracle_ffn(int d_model, int d_ff, int n_experts, int top_k, int has_shared,
               const uint8_t* const* gu_codes, const uint8_t* const* gu_scales,
               const uint8_t* const* dn_codes, const uint8_t* const* dn_scales,
               const int8_t* q, int64_t ld_q, const float* qs, int64_t ld_qs,
               int rows, const int32_t* ids, const float* w,
               const int8_t* hq_in, const float* hs_in,
               float* y, int64_t ld_y, float* h_out, int8_t* hq_out,
               float* hs_out, float* Y_out);

#ifdef __cplusplus
}
#endif
#endif
