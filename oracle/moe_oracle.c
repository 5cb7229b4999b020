/*
 * moe_oracle.c -- TEST INFRASTRUCTURE ONLY: plain CPU reference of the
 * routed-expert MXFP4 MoE feed-forward.  See moe_oracle.h for the page
 * abbreviations, layouts and the precision contract.
 *
 * Build: gcc -O2 -std=c11 -fno-fast-math -ffp-contract=off -fopenmp -fPIC
 *        -shared moe_oracle.c -o libmoe_oracle.so -lm
 * (-ffp-contract=off keeps every product and sum as written.)
 */
#include "moe_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static int g_threads = 1;
static int g_exact = 0;
static int g_bf16_mid = 0;

void oracle_set_threads(int n) { g_threads = n < 1 ? 1 : n; }
int oracle_get_threads(void) { return g_threads; }
int oracle_set_exact_rows(int on) {
  const int old = g_exact;
  g_exact = on ? 1 : 0;
  return old;
}

int oracle_set_bf16_intermediate(int on) {
  const int old = g_bf16_mid;
  g_bf16_mid = on ? 1 : 0;
  return old;
}

/* ------------------------------------------------------------ round_bf16 */

/* From the format's definition: a BF16 number has 8 significant bits and the
 * fp32 exponent range, so for |x| in [2^(e-1), 2^e) its spacing is 2^(e-8),
 * and below 2^-126 the spacing stays at the subnormal step 2^-133.  x / spacing
 * is taken to the nearest integer (ties to the even one) and scaled back; all
 * of it is exact in double. */
static float round_bf16_1(float x) {
  if (x != x || isinf(x) || x == 0.0f) return x;
  int e;
  (void)frexp((double)x, &e);
  if (e < -125) e = -125;
  const double step = ldexp(1.0, e - 8);
  const double q = (double)x / step;
  double n = floor(q);
  const double frac = q - n;
  if (frac > 0.5 || (frac == 0.5 && fmod(n, 2.0) != 0.0)) n += 1.0;
  const double v = n * step;
  const double max_bf16 = ldexp(255.0, 127 - 7); /* (2 - 2^-7) * 2^127 */
  if (fabs(v) > max_bf16) return x < 0 ? -INFINITY : INFINITY;
  if (v == 0.0) return x < 0 ? -0.0f : 0.0f;
  return (float)v;
}

void oracle_round_bf16(const float* x, int n, float* y) {
  for (int i = 0; i < n; ++i) y[i] = round_bf16_1(x[i]);
}

/* ------------------------------------------------------------ exp_rows */

/* Cody-Waite: k = nearest integer to x / ln2, r = x - k*ln2 taken in two
 * fused steps with ln2 = LN2_HI + LN2_LO (LN2_HI has 16 significant bits,
 * so k*LN2_HI is exact for |k| <= 256); exp(r) for |r| <= ln2/2 by its
 * Taylor series to r^7 (truncation below 1e-8 relative); exp(x) =
 * 2^k exp(r). */
static float exp_rows1(float x) {
  static const float LOG2E = 0x1.715476p+0f;   /* 1/ln2 rounded to fp32 */
  static const float LN2_HI = 0x1.62e4p-1f;    /* 0.693145751953125 */
  static const float LN2_LO = 0x1.7f7d1cp-20f; /* ln2 - LN2_HI, to fp32 */
  static const float C[8] = {1.0f, 1.0f, 0x1p-1f, 0x1.555556p-3f,
                             0x1.555556p-5f, 0x1.111112p-7f, 0x1.6c16c2p-10f,
                             0x1.a01a02p-13f}; /* 1/n!, n = 0..7, to fp32 */
  if (x != x) return x;
  if (x < -104.0f) return 0.0f;
  if (x > 89.0f) return INFINITY;
  const float k = rintf(x * LOG2E);
  float r = fmaf(-k, LN2_HI, x);
  r = fmaf(-k, LN2_LO, r);
  float p = C[7];
  for (int n = 6; n >= 0; --n) p = fmaf(p, r, C[n]);
  return ldexpf(p, (int)k);
}

void oracle_exp_rows(const float* x, int n, float* y) {
  for (int i = 0; i < n; ++i) y[i] = exp_rows1(x[i]);
}

/* ---------------------------------------------------------------- tables */

/* [gfx90a] §6.1 (Parallel decomposition): the decode route maps each E2M1
 * nibble to the integers 0, +-1, +-2, +-3, +-4, +-6, +-8, +-12, i.e. twice the
 * E2M1 value.  The bit fields are the MX E2M1 encoding: sign = bit 3,
 * exponent = bits 2..1 (bias 1), mantissa = bit 0; exponent 0 is subnormal
 * (value m/2).  So 2*value = m for e == 0, else 2^(e-1) * (2 + m). */
int oracle_e2m1_x2(int code) {
  const int s = (code >> 3) & 1;
  const int e = (code >> 1) & 3;
  const int m = code & 1;
  const int mag2 = (e == 0) ? m : (1 << (e - 1)) * (2 + m);
  return s ? -mag2 : mag2;
}

double oracle_e2m1(int code) { return 0.5 * (double)oracle_e2m1_x2(code); }

/* E8M0 shared block exponent: 2^(u-127), 0xFF is NaN.  [gfx90a] §6.1 names
 * the E8M0 scaling step without printing the bias; the MX definition is
 * used. */
double oracle_e8m0(int u) {
  if (u == 255) return NAN;
  return ldexp(1.0, u - 127);
}

/* ------------------------------------------------------------ block dot */

/* [gfx90a] §6.1: packed FP4 weights times int8 activations accumulate as an
 * integer dot (v_dot4_i32_i8 there) within one 32-element block; the
 * activation and E8M0 scales are applied afterwards.  Exact in int32:
 * |dot| <= 32 * 12 * 127. */
int32_t oracle_block_dot(const uint8_t* codes16, const int8_t* q32) {
  int32_t acc = 0;
  for (int i = 0; i < 32; ++i) {
    const int code = (codes16[i >> 1] >> ((i & 1) * 4)) & 0xF;
    acc += (int32_t)oracle_e2m1_x2(code) * (int32_t)q32[i];
  }
  return acc;
}

/* ------------------------------------------------------------ quantiser */

/* [gfx90a] §6.1: activations are quantised online to INT8 per 32 elements
 * (there from BF16; here from fp32).  The pages do not print the rule; the
 * reading used is the plain symmetric absmax one: d = amax / 127 (fp32,
 * correctly rounded), q = clamp(rint(x / d), -127, 127) with rint rounding
 * half to even; an all-zero block gives d = 0 and q = 0. */
int oracle_quant_q8(const float* x, int64_t ld_x, int rows, int cols,
                    int8_t* q, int64_t ld_q, float* s, int64_t ld_s) {
  if (rows < 0 || cols < 0 || (cols % 32) != 0) return ORACLE_EINVAL;
  if (ld_x < cols || ld_q < cols || ld_s < cols / 32) return ORACLE_EINVAL;
  for (int r = 0; r < rows; ++r) {
    for (int b = 0; b < cols / 32; ++b) {
      const float* xb = x + (int64_t)r * ld_x + (int64_t)b * 32;
      int8_t* qb = q + (int64_t)r * ld_q + (int64_t)b * 32;
      float amax = 0.0f;
      for (int i = 0; i < 32; ++i) {
        const float a = fabsf(xb[i]);
        if (a > amax) amax = a;
      }
      const float d = amax / 127.0f;
      s[(int64_t)r * ld_s + b] = d;
      for (int i = 0; i < 32; ++i) {
        if (d == 0.0f) {
          qb[i] = 0;
          continue;
        }
        float v = rintf(xb[i] / d);
        if (v > 127.0f) v = 127.0f;
        if (v < -127.0f) v = -127.0f;
        qb[i] = (int8_t)v;
      }
    }
  }
  return ORACLE_OK;
}

/* --------------------------------------------------------------- router */

static float bf16_bits_value(uint16_t b) {
  /* BF16 is the top half of an fp32: sign, 8 exponent bits, 7 fraction bits */
  const uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

int oracle_router_logits(const float* x, int64_t ld_x, int rows, int d_model,
                         const uint16_t* wr, int64_t ld_w, int n_experts,
                         float* logits, int64_t ld_l) {
  if (rows < 0 || d_model < 32 || d_model % 32 || n_experts < 1 ||
      ld_x < d_model || ld_w < d_model || ld_l < n_experts)
    return ORACLE_EINVAL;
  int rc = ORACLE_OK;
#pragma omp parallel for num_threads(g_threads) schedule(static)
  for (int t = 0; t < rows; ++t) {
    float* xb = (float*)malloc(sizeof(float) * (size_t)d_model);
    if (!xb) {
      rc = ORACLE_EINVAL;
      continue;
    }
    oracle_round_bf16(x + (int64_t)t * ld_x, d_model, xb);
    for (int e = 0; e < n_experts; ++e) {
      const uint16_t* we = wr + (int64_t)e * ld_w;
      if (g_exact) {
        float p[64];
        for (int l = 0; l < 64; ++l) {
          p[l] = 0.0f;
          for (int j = 0; 512 * j < d_model; ++j)
            for (int i = 0; i < 8; ++i) {
              const int k = 512 * j + 8 * l + i;
              if (k < d_model) p[l] = fmaf(xb[k], bf16_bits_value(we[k]), p[l]);
            }
        }
        for (int m = 32; m >= 1; m >>= 1) {
          float q[64];
          for (int l = 0; l < 64; ++l) q[l] = p[l] + p[l ^ m];
          memcpy(p, q, sizeof p);
        }
        logits[(int64_t)t * ld_l + e] = p[0];
      } else {
        double s = 0.0;
        for (int k = 0; k < d_model; ++k)
          s += (double)xb[k] * (double)bf16_bits_value(we[k]);
        logits[(int64_t)t * ld_l + e] = (float)s;
      }
    }
    free(xb);
  }
  return rc;
}

/* [gfx90a] §3.2 (Execution structure): 256 routed experts, top-6 per token.
 * [gfx90a] §5.3: membership ties are broken by logical expert id and the
 * selected positions come out in a fixed order.  Reading used: experts are
 * ranked by logit, larger first, ties to the lower index (ranking by logit is
 * ranking by sigmoid score, which is strictly monotone); slot i holds the
 * i-th pick; weights are sigmoid scores renormalised over the k picks. */
int oracle_route(const float* logits, int64_t ld_l, int rows, int n_experts,
                 int top_k, int32_t* ids, float* w) {
  if (rows < 0 || n_experts < 1 || top_k < 1 || top_k > n_experts ||
      ld_l < n_experts)
    return ORACLE_EINVAL;
  unsigned char* taken = (unsigned char*)malloc((size_t)n_experts);
  double* sg = (double*)malloc(sizeof(double) * (size_t)top_k);
  if (!taken || !sg) {
    free(taken);
    free(sg);
    return ORACLE_EINVAL;
  }
  for (int r = 0; r < rows; ++r) {
    const float* l = logits + (int64_t)r * ld_l;
    memset(taken, 0, (size_t)n_experts);
    for (int i = 0; i < top_k; ++i) {
      int best = -1;
      for (int e = 0; e < n_experts; ++e) {
        if (taken[e]) continue;
        if (best < 0 || l[e] > l[best]) best = e; /* strict: keeps lower id */
      }
      taken[best] = 1;
      ids[(int64_t)r * top_k + i] = best;
    }
    if (g_exact) { /* fp32: sigmoid with exp_rows, sum in pick order */
      float sum = 0.0f;
      float* sgf = (float*)sg;
      for (int i = 0; i < top_k; ++i) {
        const float z = l[ids[(int64_t)r * top_k + i]];
        sgf[i] = 1.0f / (1.0f + exp_rows1(-z));
        sum = sum + sgf[i];
      }
      for (int i = 0; i < top_k; ++i) w[(int64_t)r * top_k + i] = sgf[i] / sum;
      continue;
    }
    double sum = 0.0;
    for (int i = 0; i < top_k; ++i) {
      const double z = (double)l[ids[(int64_t)r * top_k + i]];
      sg[i] = 1.0 / (1.0 + exp(-z));
      sum += sg[i];
    }
    for (int i = 0; i < top_k; ++i)
      w[(int64_t)r * top_k + i] = (float)(sg[i] / sum);
  }
  free(taken);
  free(sg);
  return ORACLE_OK;
}

/* [gfx90a] §7.1 item 8 and §3.2: token-slot assignments are sorted by expert
 * so that each expert scans its packed weights once.  Assignment a = t*k + i.
 * counts[e] = #assignments routed to e (ids < 0 are sentinels for routes this
 * device does not own, [lucebox] "Reduce expert-route overhead", and are
 * skipped); offsets = exclusive prefix (offsets[E] = #valid); sorted lists
 * assignments grouped by expert, ascending a inside a group (stable); entries
 * past offsets[E] are -1. */
int oracle_group(const int32_t* ids, int n_assign, int n_experts,
                 int32_t* counts, int32_t* offsets, int32_t* sorted) {
  if (n_assign < 0 || n_experts < 1) return ORACLE_EINVAL;
  for (int a = 0; a < n_assign; ++a)
    if (ids[a] >= n_experts) return ORACLE_EINVAL;
  for (int e = 0; e < n_experts; ++e) counts[e] = 0;
  for (int a = 0; a < n_assign; ++a)
    if (ids[a] >= 0) counts[ids[a]] += 1;
  offsets[0] = 0;
  for (int e = 0; e < n_experts; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int32_t* pos = (int32_t*)malloc(sizeof(int32_t) * (size_t)n_experts);
  if (!pos) return ORACLE_EINVAL;
  for (int e = 0; e < n_experts; ++e) pos[e] = offsets[e];
  for (int a = 0; a < n_assign; ++a)
    if (ids[a] >= 0) sorted[pos[ids[a]]++] = a;
  for (int p = offsets[n_experts]; p < n_assign; ++p) sorted[p] = -1;
  free(pos);
  return ORACLE_OK;
}

/* ------------------------------------------------------------ projection */

/* [gfx90a] §6.1: integer block dot followed by activation and E8M0 scaling.
 * With e2m1_x2 = 2*value, the weight factor of block b is 2^(u-127)/2.  Each
 * term dot * d * 2^(u-128) is exact in fp64; the fp64 sum over b is rounded
 * once to fp32. */
static int matvec_impl(const uint8_t* codes, int64_t ld_c, const uint8_t* scales,
                       int64_t ld_s, int n_out, int d_in, const int8_t* q,
                       int64_t ld_q, const float* qs, int64_t ld_qs, int rows,
                       float* y, int64_t ld_y, int nthreads) {
  if (n_out < 0 || rows < 0 || d_in < 0 || (d_in % 32) != 0) return ORACLE_EINVAL;
  if (ld_c < d_in / 2 || ld_s < d_in / 32 || ld_q < d_in || ld_qs < d_in / 32 ||
      ld_y < n_out)
    return ORACLE_EINVAL;
  const int nb = d_in / 32;
  const int64_t total = (int64_t)rows * n_out;
#pragma omp parallel for num_threads(nthreads) schedule(static) if (nthreads > 1)
  for (int64_t idx = 0; idx < total; ++idx) {
    const int t = (int)(idx / n_out);
    const int n = (int)(idx % n_out);
    if (g_exact) {
      /* runs of 16 blocks: each from zero, block terms (exact in fp32: a
       * dot of at most 16 bits times a power of two) folded in with fmaf
       * against the activation scale, runs added in order */
      float total = 0.0f;
      for (int b0 = 0; b0 < nb; b0 += 16) {
        float run = 0.0f;
        for (int b = b0; b < nb && b < b0 + 16; ++b) {
          const int32_t dot = oracle_block_dot(codes + (int64_t)n * ld_c + b * 16,
                                               q + (int64_t)t * ld_q + b * 32);
          const double wscale = 0.5 * oracle_e8m0(scales[(int64_t)n * ld_s + b]);
          const float term = (float)((double)dot * wscale);
          run = fmaf(term, qs[(int64_t)t * ld_qs + b], run);
        }
        total = total + run;
      }
      y[(int64_t)t * ld_y + n] = total;
      continue;
    }
    double acc = 0.0;
    for (int b = 0; b < nb; ++b) {
      const int32_t dot = oracle_block_dot(codes + (int64_t)n * ld_c + b * 16,
                                           q + (int64_t)t * ld_q + b * 32);
      const double wscale = 0.5 * oracle_e8m0(scales[(int64_t)n * ld_s + b]);
      acc += (double)dot * (double)qs[(int64_t)t * ld_qs + b] * wscale;
    }
    y[(int64_t)t * ld_y + n] = (float)acc;
  }
  return ORACLE_OK;
}

int oracle_matvec(const uint8_t* codes, int64_t ld_c, const uint8_t* scales,
                  int64_t ld_s, int n_out, int d_in, const int8_t* q,
                  int64_t ld_q, const float* qs, int64_t ld_qs, int rows,
                  float* y, int64_t ld_y) {
  return matvec_impl(codes, ld_c, scales, ld_s, n_out, d_in, q, ld_q, qs, ld_qs,
                     rows, y, ld_y, g_threads);
}

int oracle_block_dots(const uint8_t* codes, int64_t ld_c, int n_out, int d_in,
                      const int8_t* q, int64_t ld_q, int rows, int32_t* dots) {
  if (n_out < 0 || rows < 0 || d_in < 0 || (d_in % 32) != 0) return ORACLE_EINVAL;
  if (ld_c < d_in / 2 || ld_q < d_in) return ORACLE_EINVAL;
  const int nb = d_in / 32;
  for (int t = 0; t < rows; ++t)
    for (int n = 0; n < n_out; ++n)
      for (int b = 0; b < nb; ++b)
        dots[((int64_t)t * n_out + n) * nb + b] = oracle_block_dot(
            codes + (int64_t)n * ld_c + b * 16, q + (int64_t)t * ld_q + b * 32);
  return ORACLE_OK;
}

/* ------------------------------------------------------------- SwiGLU */

/* SwiGLU between gate/up and down ([gfx90a] Fig. 1, gate/up followed by down;
 * [lucebox] "Tune small HIP batches": SwiGLU folded into the second
 * projection pass).  Reading used: h = silu(gate) * up with
 * silu(z) = z / (1 + exp(-z)), no clamp, evaluated in fp64 from the fp32
 * projections and rounded once to fp32. */
void oracle_swiglu(const float* g, const float* u, int n, float* h) {
  if (g_exact) { /* fp32 with exp_rows: (g / (1 + exp(-g))) * u */
    for (int i = 0; i < n; ++i) {
      const float den = 1.0f + exp_rows1(-g[i]);
      const float silu = g[i] / den;
      h[i] = silu * u[i];
    }
    return;
  }
  for (int i = 0; i < n; ++i) {
    const double z = (double)g[i];
    const double silu = z / (1.0 + exp(-z));
    h[i] = (float)(silu * (double)u[i]);
  }
}

int oracle_expert_hidden(const uint8_t* gu_codes, const uint8_t* gu_scales,
                         int d_model, int d_ff, const int8_t* q, int64_t ld_q,
                         const float* qs, int64_t ld_qs, int rows, float* h,
                         int64_t ld_h) {
  if (rows < 0 || d_model % 32 || d_ff < 1 || ld_h < d_ff) return ORACLE_EINVAL;
  const int64_t ldc = d_model / 2, lds = d_model / 32;
  float* g = (float*)malloc(sizeof(float) * (size_t)d_ff);
  float* u = (float*)malloc(sizeof(float) * (size_t)d_ff);
  int rc = (g && u) ? ORACLE_OK : ORACLE_EINVAL;
  for (int t = 0; rc == ORACLE_OK && t < rows; ++t) {
    const int8_t* qt = q + (int64_t)t * ld_q;
    const float* st = qs + (int64_t)t * ld_qs;
    /* single-threaded: callers parallelise over rows / assignments */
    rc = matvec_impl(gu_codes, ldc, gu_scales, lds, d_ff, d_model, qt, ld_q, st,
                     ld_qs, 1, g, d_ff, 1);
    if (rc == ORACLE_OK)
      rc = matvec_impl(gu_codes + (int64_t)d_ff * ldc, ldc,
                       gu_scales + (int64_t)d_ff * lds, lds, d_ff, d_model, qt,
                       ld_q, st, ld_qs, 1, u, d_ff, 1);
    if (rc == ORACLE_OK) {
      float* ht = h + (int64_t)t * ld_h;
      oracle_swiglu(g, u, d_ff, ht);
      if (g_bf16_mid) oracle_round_bf16(ht, d_ff, ht); /* [gfx90a] §8.2 */
    }
  }
  free(g);
  free(u);
  return rc;
}

/* -------------------------------------------------------------- combine */

/* [gfx90a] §8.2 and Table 4: per-slot FP32 top-k partials are kept and
 * reduced in a fixed order (BF16 partials were rejected; atomics make the
 * order non-deterministic).  Fig. 1: shared and routed experts join.
 * y[t] = sum_i w[t][i] * Y[t][i] (+ Y[t][shared], weight 1), fp64, in slot
 * order, rounded once to fp32. */
int oracle_combine(int rows, int top_k, int has_shared, int d_model,
                   const int32_t* ids, const float* w, const float* Y,
                   float* y, int64_t ld_y) {
  if (rows < 0 || top_k < 1 || d_model < 0 || ld_y < d_model) return ORACLE_EINVAL;
  const int slots = top_k + 1;
  for (int t = 0; t < rows; ++t) {
    for (int n = 0; n < d_model; ++n) {
      if (g_exact) { /* fmaf per slot in slot order from zero, shared last */
        float v = 0.0f;
        for (int i = 0; i < top_k; ++i) {
          if (ids[(int64_t)t * top_k + i] < 0) continue;
          v = fmaf(w[(int64_t)t * top_k + i], Y[((int64_t)t * slots + i) * d_model + n], v);
        }
        if (has_shared) v = v + Y[((int64_t)t * slots + top_k) * d_model + n];
        y[(int64_t)t * ld_y + n] = v;
        continue;
      }
      double acc = 0.0;
      for (int i = 0; i < top_k; ++i) {
        if (ids[(int64_t)t * top_k + i] < 0) continue;
        acc += (double)w[(int64_t)t * top_k + i] *
               (double)Y[((int64_t)t * slots + i) * d_model + n];
      }
      if (has_shared) acc += (double)Y[((int64_t)t * slots + top_k) * d_model + n];
      y[(int64_t)t * ld_y + n] = (float)acc;
    }
  }
  return ORACLE_OK;
}

/* ------------------------------------------------------------------ FFN */

/* One routed-expert layer, in the order of [gfx90a] Fig. 1 and §6.1/§8.2:
 * gate/up -> SwiGLU -> group-32 int8 requant of the intermediate -> down ->
 * fixed-order weighted combine with the shared expert.  The intermediate is
 * kept in fp32 before its requant (the report's BF16 rounding step is a
 * variant, not done here). */
int oracle_ffn(int d_model, int d_ff, int n_experts, int top_k, int has_shared,
               const uint8_t* const* gu_codes, const uint8_t* const* gu_scales,
               const uint8_t* const* dn_codes, const uint8_t* const* dn_scales,
               const int8_t* q, int64_t ld_q, const float* qs, int64_t ld_qs,
               int rows, const int32_t* ids, const float* w,
               const int8_t* hq_in, const float* hs_in,
               float* y, int64_t ld_y, float* h_out, int8_t* hq_out,
               float* hs_out, float* Y_out) {
  if (rows < 0 || d_model < 32 || d_model % 32 || d_ff < 32 || d_ff % 32 ||
      n_experts < 1 || top_k < 1 || top_k > n_experts)
    return ORACLE_EINVAL;
  for (int64_t a = 0; a < (int64_t)rows * top_k; ++a)
    if (ids[a] >= n_experts) return ORACLE_EINVAL;
  const int slots = top_k + 1;
  const int64_t nrow = (int64_t)rows * slots;
  float* Y = Y_out ? Y_out : (float*)calloc((size_t)(nrow * d_model), sizeof(float));
  if (!Y) return ORACLE_EINVAL;
  int rc = ORACLE_OK;

#pragma omp parallel for num_threads(g_threads) schedule(dynamic, 1)
  for (int64_t r = 0; r < nrow; ++r) {
    const int t = (int)(r / slots);
    const int i = (int)(r % slots);
    int e;
    if (i < top_k) {
      e = ids[(int64_t)t * top_k + i];
      if (e < 0) continue;
    } else {
      if (!has_shared) continue;
      e = n_experts;
    }
    if (!dn_codes[e] || !dn_scales[e] || (!hq_in && (!gu_codes[e] || !gu_scales[e]))) {
#pragma omp atomic write
      rc = ORACLE_EINVAL;
      continue;
    }
    float* h = (float*)malloc(sizeof(float) * (size_t)d_ff);
    int8_t* hq = (int8_t*)malloc((size_t)d_ff);
    float* hs = (float*)malloc(sizeof(float) * (size_t)(d_ff / 32));
    if (!h || !hq || !hs) {
#pragma omp atomic write
      rc = ORACLE_EINVAL;
    } else {
      if (hq_in) {
        memcpy(hq, hq_in + r * d_ff, (size_t)d_ff);
        memcpy(hs, hs_in + r * (d_ff / 32), sizeof(float) * (size_t)(d_ff / 32));
      } else {
        oracle_expert_hidden(gu_codes[e], gu_scales[e], d_model, d_ff,
                             q + (int64_t)t * ld_q, ld_q, qs + (int64_t)t * ld_qs,
                             ld_qs, 1, h, d_ff);
        /* [gfx90a] §8.2: the intermediate is requantised to group-32 INT8
         * values and scales before the down projection. */
        oracle_quant_q8(h, d_ff, 1, d_ff, hq, d_ff, hs, d_ff / 32);
        if (h_out) memcpy(h_out + r * d_ff, h, sizeof(float) * (size_t)d_ff);
      }
      if (hq_out) memcpy(hq_out + r * d_ff, hq, (size_t)d_ff);
      if (hs_out) memcpy(hs_out + r * (d_ff / 32), hs, sizeof(float) * (size_t)(d_ff / 32));
      matvec_impl(dn_codes[e], d_ff / 2, dn_scales[e], d_ff / 32, d_model, d_ff,
                  hq, d_ff, hs, d_ff / 32, 1, Y + r * d_model, d_model, 1);
    }
    free(h);
    free(hq);
    free(hs);
  }
  if (rc == ORACLE_OK)
    rc = oracle_combine(rows, top_k, has_shared, d_model, ids, w, Y, y, ld_y);
  if (!Y_out) free(Y);
  return rc;
}
