/*
 * nvfp4_oracle.c -- plain, slow, CPU oracle for NVFP4 (g16) W4A16 GEMV and
 * the MoE expert-slot variant. TEST INFRASTRUCTURE ONLY: see nvfp4_oracle.h.
 *
 * Sources of each definition:
 *  - "nvfp4/g16" weight = E2M1 codes with one UE4M3 scale per 16 elements and
 *    an fp32 tensor scale: blueprint page, Precision table; card.json
 *    performance[6].note; graph.json node "l0.kda.q" step list.
 *  - E2M1 / E4M3 bit layouts: OCP Microscaling (MX) v1.0 element formats
 *    (not on the pages).
 *  - Two-level scale recipe: the block scale encodes amax_block / 6 relative
 *    to the tensor scale g = max|W| / (6 * 448), so the largest block maps to
 *    the largest E4M3 value 448 and its largest element to the largest E2M1
 *    value 6.
 *  - GEMV: steps "act bf16", "weight nvfp4/g16->bf16", "mma bf16*bf16",
 *    "accumulate f32", "scale f32" of graph.json node "l0.kda.q": decode,
 *    multiply by the bf16 activation, accumulate, then apply the tensor
 *    scale once. Here the sum is exact-term fp64.
 *  - MoE: graph.json nodes "l3.moe.experts_gate_up" (gather by expert id),
 *    "l3.moe.experts_act" (silu_mul, bf16 out), "l3.moe.experts_down",
 *    "l3.moe.blend" (combine by gate weight, f32); llama.cpp SWIGLU op
 *    (ggml trace page, ffn_swiglu rows) = silu(gate) * up.
 *  - Shared expert: graph.json nodes "l3.moe.shared_gate_up",
 *    "l3.moe.shared_act", "l3.moe.shared_down"; card.json performance[4]
 *    and [9] (gate|up N = 768 + 768, down K = 768); "l3.moe.blend" adds it to
 *    the routed slots ("routed slots + shared in").
 *  - W4A4: card.json "W4A4 NVFP4 x NVFP4 (static input scale)",
 *    performance[20] and [24] (dense), [64] and [65] (MoE union sweeps);
 *    graph.json node "l0.mlp.xn_quant" (act_quant bf16 -> nvfp4/g16).
 *
 * Build: gcc -O2 -ffp-contract=off (no -ffast-math), optionally -fopenmp.
 * fp32 expressions below are evaluated in fp32 (SSE, FLT_EVAL_METHOD 0).
 */
#include "nvfp4_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- decode */

double oracle_e2m1_value(unsigned code) {
  /* FP4 E2M1: bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa.
     Exponent field 0 is subnormal: magnitude = mantissa * 0.5. */
  unsigned s = (code >> 3) & 1u, e = (code >> 1) & 3u, m = code & 1u;
  double mag = (e == 0) ? 0.5 * (double)m : ldexp(1.0 + 0.5 * (double)m, (int)e - 1);
  return s ? -mag : mag;
}

double oracle_e4m3_value(unsigned byte) {
  /* FP8 E4M3 (FN variant): bit 7 sign, bits 6..3 exponent (bias 7), bits 2..0
     mantissa. Exponent field 0 is subnormal: magnitude = m * 2^-9. Exponent 15
     with mantissa 7 is NaN; there are no infinities. */
  unsigned s = (byte >> 7) & 1u, e = (byte >> 3) & 15u, m = byte & 7u;
  double mag;
  if (e == 15u && m == 7u) return NAN;
  mag = (e == 0) ? ldexp((double)m, -9) : ldexp(1.0 + (double)m / 8.0, (int)e - 7);
  return s ? -mag : mag;
}

/* ---------------------------------------------------------------- encode */

/* Round to nearest integer, ties to even (default rounding mode). */
static double rne_int(double v) { return nearbyint(v); }

unsigned oracle_e4m3_encode(float r) {
  /* The input is an fp32 value; every step below is exact in fp64, so the
     only rounding is the final choice of representable value. */
  double v = (double)r;
  int ex, e;
  double q;
  unsigned code;
  if (!(v > 0.0)) return 0u;          /* zero, negative or NaN -> +0 */
  if (v > 448.0) return 0x7Eu;        /* saturate to the largest finite, 448 */
  if (v < ldexp(1.0, -6)) {
    /* subnormal binade: values m * 2^-9, m = 0..7; m = 8 is the smallest
       normal (code 0x08), which the same integer encodes */
    return (unsigned)rne_int(v * 512.0);
  }
  (void)frexp(v, &ex);                /* v = f * 2^ex, f in [0.5, 1) */
  e = ex - 1;                          /* v in [2^e, 2^(e+1)), e in -6..8 */
  q = rne_int(ldexp(v, 3 - e));        /* 1.mmm scaled by 8: in [8, 16] */
  if (q == 16.0) { q = 8.0; e += 1; }  /* rounded up into the next binade */
  code = ((unsigned)(e + 7) << 3) | ((unsigned)q - 8u);
  return code > 0x7Eu ? 0x7Eu : code;
}

unsigned oracle_e2m1_encode(float t) {
  double a = fabs((double)t);
  unsigned mag;
  if (a > 6.0) {
    mag = 7u;                          /* saturate to 6 */
  } else if (a < 1.0) {
    mag = (unsigned)rne_int(a * 2.0);  /* 0, 0.5 or 1.0: codes 0, 1, 2 */
  } else {
    int ex, e;
    double q;
    (void)frexp(a, &ex);
    e = ex - 1;                        /* a in [2^e, 2^(e+1)), e in 0..2 */
    q = rne_int(ldexp(a, 1 - e));      /* 1.m scaled by 2: in [2, 4] */
    if (q == 4.0) { q = 2.0; e += 1; }
    mag = ((unsigned)(e + 1) << 1) | ((unsigned)q - 2u);
    if (mag > 7u) mag = 7u;
  }
  return (t < 0.0f && mag != 0u) ? (mag | 8u) : mag;
}

/* ------------------------------------------------------------------ pack */

/* Steps 2-4 of the recipe for one block of 16 fp32 values w with tensor
   scale g: the scale byte and the 8 code bytes. */
static void quantize_block(const float* w, float g, uint8_t* c, uint8_t* scale) {
  const float d6 = 6.0f * g;
  float ab = 0.0f, r, s;
  unsigned sc;
  int j;
  /* Step 2: block amax relative to 6 * g. */
  for (j = 0; j < 16; ++j) {
    float a = fabsf(w[j]);
    if (a > ab) ab = a;
  }
  r = ab / d6;
  /* Step 3: the block scale byte and its value. */
  sc = oracle_e4m3_encode(r);
  *scale = (uint8_t)sc;
  s = (float)oracle_e4m3_value(sc);
  /* Step 4: element codes relative to s * g. */
  if (s == 0.0f) {
    memset(c, 0, 8);
  } else {
    const float dn = s * g;
    for (j = 0; j < 8; ++j) {
      unsigned lo = oracle_e2m1_encode(w[2 * j] / dn);
      unsigned hi = oracle_e2m1_encode(w[2 * j + 1] / dn);
      c[j] = (uint8_t)(lo | (hi << 4));
    }
  }
}

int oracle_pack(const float* W, int64_t N, int64_t K, uint8_t* codes,
                uint8_t* scales, float* gscale_out, const float* gscale_override) {
  int64_t i, n;
  float A = 0.0f, g;
  int bad = 0;
  if (N < 0 || K < 0 || (K % 16) != 0) return ORACLE_ERR_SHAPE;
  /* Step 1: tensor amax (exact) and the fp32 tensor scale. */
  for (i = 0; i < N * K; ++i) {
    float a = fabsf(W[i]);
    if (!isfinite(W[i])) { bad = 1; break; }
    if (a > A) A = a;
  }
  if (bad) return ORACLE_ERR_NONFINITE;
  if (gscale_override) {
    g = *gscale_override;
    if (!(g > 0.0f) || !isfinite(g)) return ORACLE_ERR_GSCALE;
  } else {
    g = (A == 0.0f) ? 1.0f : A / 2688.0f;
  }
  *gscale_out = g;

#pragma omp parallel for schedule(static)
  for (n = 0; n < N; ++n) {
    const int64_t nb = K / 16;
    int64_t b;
    for (b = 0; b < nb; ++b)
      quantize_block(W + n * K + b * 16, g, codes + n * (K / 2) + b * 8, scales + n * nb + b);
  }
  return ORACLE_OK;
}

/* --------------------------------------------------------------- dequant */

static unsigned code_at(const uint8_t* codes, int64_t K, int64_t n, int64_t k) {
  uint8_t byte = codes[n * (K / 2) + k / 2];
  return (k & 1) ? (unsigned)(byte >> 4) : (unsigned)(byte & 15u);
}

int oracle_dequant(const uint8_t* codes, const uint8_t* scales, float g,
                   int64_t N, int64_t K, float* W_out) {
  int64_t n;
  if (N < 0 || K < 0 || (K % 16) != 0) return ORACLE_ERR_SHAPE;
#pragma omp parallel for schedule(static)
  for (n = 0; n < N; ++n) {
    int64_t k;
    for (k = 0; k < K; ++k) {
      double e = oracle_e2m1_value(code_at(codes, K, n, k));
      double s = oracle_e4m3_value(scales[n * (K / 16) + k / 16]);
      float es = (float)(e * s); /* exact: at most 6 significant bits */
      W_out[n * K + k] = es * g;
    }
  }
  return ORACLE_OK;
}

/* ------------------------------------------------------------------ gemv */

static double bf16_value(uint16_t bits) {
  /* bf16 is the upper half of an IEEE binary32 */
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

int oracle_gemv(const uint8_t* codes, const uint8_t* scales, float g,
                const uint16_t* x, int64_t M, int64_t N, int64_t K,
                const int64_t* rows, int64_t n_rows, double* y, double* absdot) {
  int64_t cnt = rows ? n_rows : N, i;
  if (M < 0 || N < 0 || K < 0 || (K % 16) != 0) return ORACLE_ERR_SHAPE;
  if (rows) {
    for (i = 0; i < n_rows; ++i)
      if (rows[i] < 0 || rows[i] >= N) return ORACLE_ERR_SHAPE;
  }
#pragma omp parallel for schedule(dynamic, 16)
  for (i = 0; i < cnt; ++i) {
    const int64_t n = rows ? rows[i] : i;
    int64_t m, k;
    for (m = 0; m < M; ++m) {
      double sum = 0.0, asum = 0.0;
      for (k = 0; k < K; ++k) {
        double w = oracle_e2m1_value(code_at(codes, K, n, k)) *
                   oracle_e4m3_value(scales[n * (K / 16) + k / 16]);
        double t = w * bf16_value(x[m * K + k]);  /* exact in fp64 */
        sum += t;
        asum += fabs(t);
      }
      y[m * cnt + i] = (double)g * sum;
      if (absdot) absdot[m * cnt + i] = fabs((double)g) * asum;
    }
  }
  return ORACLE_OK;
}

/* ------------------------------------------------------------------- moe */

uint16_t oracle_bf16_from_double(double v) {
  /* One rounding from fp64 to bf16 (8 significant bits), ties to even,
     with bf16's subnormals (quantum 2^-133) and overflow to infinity. */
  double a, q;
  int ex, e;
  float f;
  uint32_t u;
  uint16_t sign = signbit(v) ? 0x8000u : 0u;
  if (isnan(v)) return 0x7FC0u;
  a = fabs(v);
  if (a == 0.0) return sign;
  if (isinf(a)) return (uint16_t)(sign | 0x7F80u);
  (void)frexp(a, &ex);
  e = ex - 1;                           /* a in [2^e, 2^(e+1)) */
  if (e < -126) e = -126;               /* subnormals share the quantum 2^-133 */
  q = ldexp(rne_int(ldexp(a, 7 - e)), e - 7);
  if (q >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80u);
  f = (float)q;                         /* exact: q has <= 8 significant bits */
  memcpy(&u, &f, 4);
  return (uint16_t)(sign | (uint16_t)((u >> 16) & 0x7FFFu));
}

/* fp64 dot of one NVFP4 row with a vector given as doubles; also |.| sum. */
static void row_dot(const uint8_t* codes, const uint8_t* scales, int64_t K,
                    int64_t n, const double* v, double* dot, double* adot) {
  double sum = 0.0, asum = 0.0;
  int64_t k;
  for (k = 0; k < K; ++k) {
    double w = oracle_e2m1_value(code_at(codes, K, n, k)) *
               oracle_e4m3_value(scales[n * (K / 16) + k / 16]);
    sum += w * v[k];
    asum += fabs(w * v[k]);
  }
  *dot = sum;
  if (adot) *adot = asum;
}

int oracle_moe(const uint8_t* w13_codes, const uint8_t* w13_scales, const float* w13_g,
               const uint8_t* w2_codes, const uint8_t* w2_scales, const float* w2_g,
               const uint16_t* x, const int32_t* ids, const float* gate_w,
               int64_t M, int64_t E, int64_t H, int64_t I, int64_t topk,
               double* y, double* bound, uint16_t* h_out) {
  int64_t m, i;
  if (M < 0 || E < 0 || H < 0 || I < 0 || topk < 0) return ORACLE_ERR_SHAPE;
  if ((H % 16) != 0 || (I % 16) != 0) return ORACLE_ERR_SHAPE;
  for (i = 0; i < M * H; ++i) {
    y[i] = 0.0;
    if (bound) bound[i] = 0.0;
  }
  if (h_out) memset(h_out, 0, (size_t)(M * topk * I) * sizeof(uint16_t));

  for (m = 0; m < M; ++m) {
    double* xv = (double*)malloc((size_t)H * sizeof(double));
    double* a = (double*)malloc((size_t)(2 * I) * sizeof(double));
    double* h = (double*)malloc((size_t)I * sizeof(double));
    int64_t j, k;
    for (k = 0; k < H; ++k) xv[k] = bf16_value(x[m * H + k]);
    for (j = 0; j < topk; ++j) {
      const int32_t e = ids[m * topk + j];
      const double gw = (double)gate_w[m * topk + j];
      const uint8_t *c13, *s13, *c2, *s2;
      int64_t r, n;
      if (e < 0 || (int64_t)e >= E) continue;  /* out-of-range slot: nothing */
      c13 = w13_codes + (int64_t)e * (2 * I) * (H / 2);
      s13 = w13_scales + (int64_t)e * (2 * I) * (H / 16);
      c2 = w2_codes + (int64_t)e * H * (I / 2);
      s2 = w2_scales + (int64_t)e * H * (I / 16);
      /* gate_up: a = g13 * W13 . x */
#pragma omp parallel for schedule(static)
      for (r = 0; r < 2 * I; ++r) {
        double d;
        row_dot(c13, s13, H, r, xv, &d, NULL);
        a[r] = (double)w13_g[e] * d;
      }
      /* SwiGLU, one rounding to bf16 */
      for (r = 0; r < I; ++r) {
        double G = a[r], U = a[I + r];
        uint16_t hb = oracle_bf16_from_double(G / (1.0 + exp(-G)) * U);
        h[r] = bf16_value(hb);
        if (h_out) h_out[(m * topk + j) * I + r] = hb;
      }
      /* down, then combine by gate weight */
#pragma omp parallel for schedule(static)
      for (n = 0; n < H; ++n) {
        double d, ad;
        row_dot(c2, s2, I, n, h, &d, &ad);
        y[m * H + n] += gw * ((double)w2_g[e] * d);
        if (bound) bound[m * H + n] += fabs(gw) * fabs((double)w2_g[e]) * ad;
      }
    }
    free(xv);
    free(a);
    free(h);
  }
  return ORACLE_OK;
}

/* One dense SwiGLU FFN (gate|up rows, bf16 activations, down) for one token,
   added to y and bound: the shared expert of oracle_moe_shared. */
static void shared_ffn_add(const uint8_t* c13, const uint8_t* s13, double g13,
                           const uint8_t* c2, const uint8_t* s2, double g2,
                           const double* xv, int64_t H, int64_t Is,
                           double* y, double* bound, uint16_t* hs_out) {
  double* a = (double*)malloc((size_t)(2 * Is) * sizeof(double));
  double* h = (double*)malloc((size_t)Is * sizeof(double));
  int64_t r, n;
#pragma omp parallel for schedule(static)
  for (r = 0; r < 2 * Is; ++r) {
    double d;
    row_dot(c13, s13, H, r, xv, &d, NULL);
    a[r] = g13 * d;
  }
  for (r = 0; r < Is; ++r) {
    double G = a[r], U = a[Is + r];
    uint16_t hb = oracle_bf16_from_double(G / (1.0 + exp(-G)) * U);
    h[r] = bf16_value(hb);
    if (hs_out) hs_out[r] = hb;
  }
#pragma omp parallel for schedule(static)
  for (n = 0; n < H; ++n) {
    double d, ad;
    row_dot(c2, s2, Is, n, h, &d, &ad);
    y[n] += 1.0 * (g2 * d);
    if (bound) bound[n] += fabs(g2) * ad;
  }
  free(a);
  free(h);
}

int oracle_moe_shared(const uint8_t* w13_codes, const uint8_t* w13_scales, const float* w13_g,
                      const uint8_t* w2_codes, const uint8_t* w2_scales, const float* w2_g,
                      const uint16_t* x, const int32_t* ids, const float* gate_w,
                      int64_t M, int64_t E, int64_t H, int64_t I, int64_t topk,
                      const uint8_t* ws13_codes, const uint8_t* ws13_scales, const float* ws13_g,
                      const uint8_t* ws2_codes, const uint8_t* ws2_scales, const float* ws2_g,
                      int64_t Is, double* y, double* bound, uint16_t* h_out, uint16_t* hs_out) {
  int64_t m, k;
  int rc;
  if (Is < 0 || (Is % 16) != 0) return ORACLE_ERR_SHAPE;
  /* the routed slots first (blend order: routed, then shared) */
  rc = oracle_moe(w13_codes, w13_scales, w13_g, w2_codes, w2_scales, w2_g, x, ids, gate_w,
                  M, E, H, I, topk, y, bound, h_out);
  if (rc != ORACLE_OK) return rc;
  for (m = 0; m < M; ++m) {
    double* xv = (double*)malloc((size_t)H * sizeof(double));
    for (k = 0; k < H; ++k) xv[k] = bf16_value(x[m * H + k]);
    shared_ffn_add(ws13_codes, ws13_scales, (double)ws13_g[0], ws2_codes, ws2_scales,
                   (double)ws2_g[0], xv, H, Is, y + m * H, bound ? bound + m * H : NULL,
                   hs_out ? hs_out + m * Is : NULL);
    free(xv);
  }
  return ORACLE_OK;
}

/* ------------------------------------------------------------------ w4a4 */

int oracle_quantize_act(const uint16_t* x, int64_t M, int64_t K, float g_x, uint8_t* codes,
                        uint8_t* scales) {
  int64_t m;
  if (M < 0 || K < 0 || (K % 16) != 0) return ORACLE_ERR_SHAPE;
  if (!(g_x > 0.0f) || !isfinite(g_x)) return ORACLE_ERR_GSCALE;
  for (m = 0; m < M * K; ++m)
    if (!isfinite(bf16_value(x[m]))) return ORACLE_ERR_NONFINITE;
  for (m = 0; m < M; ++m) {
    int64_t b;
    for (b = 0; b < K / 16; ++b) {
      float w[16];
      int j;
      for (j = 0; j < 16; ++j) w[j] = (float)bf16_value(x[m * K + b * 16 + j]);  /* exact */
      quantize_block(w, g_x, codes + m * (K / 2) + b * 8, scales + m * (K / 16) + b);
    }
  }
  return ORACLE_OK;
}

int oracle_gemv_w4a4(const uint8_t* codes_w, const uint8_t* scales_w, float g_w,
                     const uint8_t* codes_x, const uint8_t* scales_x, float g_x,
                     int64_t M, int64_t N, int64_t K, const int64_t* rows, int64_t n_rows,
                     double* y, double* absdot) {
  const int64_t cnt = rows ? n_rows : N;
  int64_t i;
  if (M < 0 || N < 0 || K < 0 || (K % 16) != 0) return ORACLE_ERR_SHAPE;
  if (rows) {
    for (i = 0; i < n_rows; ++i)
      if (rows[i] < 0 || rows[i] >= N) return ORACLE_ERR_SHAPE;
  }
#pragma omp parallel for schedule(dynamic, 16)
  for (i = 0; i < cnt; ++i) {
    const int64_t n = rows ? rows[i] : i;
    int64_t m, k;
    for (m = 0; m < M; ++m) {
      double sum = 0.0, asum = 0.0;
      for (k = 0; k < K; ++k) {
        double w = oracle_e2m1_value(code_at(codes_w, K, n, k)) *
                   oracle_e4m3_value(scales_w[n * (K / 16) + k / 16]);
        double v = oracle_e2m1_value(code_at(codes_x, K, m, k)) *
                   oracle_e4m3_value(scales_x[m * (K / 16) + k / 16]);
        double t = w * v;   /* exact in fp64 */
        sum += t;
        asum += fabs(t);
      }
      y[m * cnt + i] = (double)g_w * (double)g_x * sum;
      if (absdot) absdot[m * cnt + i] = fabs((double)g_w * (double)g_x) * asum;
    }
  }
  return ORACLE_OK;
}

/* One row of bf16 activations quantized with a static scale (as in
   oracle_quantize_act) and decoded to the exact values e2m1 * s (fp64,
   without the tensor scale). */
static void quantize_decode_row(const uint16_t* x, int64_t K, float g, uint8_t* codes,
                                uint8_t* scales, double* v) {
  int64_t b;
  for (b = 0; b < K / 16; ++b) {
    float w[16];
    int j;
    for (j = 0; j < 16; ++j) w[j] = (float)bf16_value(x[b * 16 + j]);
    quantize_block(w, g, codes + b * 8, scales + b);
  }
  for (b = 0; b < K; ++b) {
    unsigned c = (codes[b / 2] >> (4 * (b % 2))) & 15u;
    v[b] = oracle_e2m1_value(c) * oracle_e4m3_value(scales[b / 16]);
  }
}

int oracle_moe_w4a4(const uint8_t* w13_codes, const uint8_t* w13_scales, const float* w13_g,
                    const uint8_t* w2_codes, const uint8_t* w2_scales, const float* w2_g,
                    const uint16_t* x, const int32_t* ids, const float* gate_w,
                    int64_t M, int64_t E, int64_t H, int64_t I, int64_t topk,
                    float g_a13, float g_a2,
                    const uint8_t* ws13_codes, const uint8_t* ws13_scales, const float* ws13_g,
                    const uint8_t* ws2_codes, const uint8_t* ws2_scales, const float* ws2_g,
                    int64_t Is, const uint16_t* h_in, double* y, double* bound,
                    uint16_t* h_out, uint8_t* hq_codes, uint8_t* hq_scales) {
  int64_t m, i;
  if (M < 0 || E < 0 || H < 0 || I < 0 || topk < 0 || Is < 0) return ORACLE_ERR_SHAPE;
  if ((H % 16) != 0 || (I % 16) != 0 || (Is % 16) != 0) return ORACLE_ERR_SHAPE;
  if (!(g_a13 > 0.0f) || !isfinite(g_a13) || !(g_a2 > 0.0f) || !isfinite(g_a2))
    return ORACLE_ERR_GSCALE;
  for (i = 0; i < M * H; ++i)
    if (!isfinite(bf16_value(x[i]))) return ORACLE_ERR_NONFINITE;
  for (i = 0; i < M * H; ++i) {
    y[i] = 0.0;
    if (bound) bound[i] = 0.0;
  }
  if (h_out) memset(h_out, 0, (size_t)(M * topk * I) * sizeof(uint16_t));
  if (hq_codes) memset(hq_codes, 0, (size_t)(M * topk * (I / 2)));
  if (hq_scales) memset(hq_scales, 0, (size_t)(M * topk * (I / 16)));

  for (m = 0; m < M; ++m) {
    uint8_t* xc = (uint8_t*)malloc((size_t)(H / 2) + 1);
    uint8_t* xs = (uint8_t*)malloc((size_t)(H / 16) + 1);
    double* xq = (double*)malloc((size_t)H * sizeof(double) + 8);
    double* a = (double*)malloc((size_t)(2 * I) * sizeof(double) + 8);
    uint16_t* hb = (uint16_t*)malloc((size_t)I * sizeof(uint16_t) + 2);
    uint8_t* hc = (uint8_t*)malloc((size_t)(I / 2) + 1);
    uint8_t* hs = (uint8_t*)malloc((size_t)(I / 16) + 1);
    double* hq = (double*)malloc((size_t)I * sizeof(double) + 8);
    int64_t j, k;
    /* the token's activations on the NVFP4 grid of the static scale g_a13 */
    quantize_decode_row(x + m * H, H, g_a13, xc, xs, xq);
    for (j = 0; j < topk; ++j) {
      const int64_t slot = m * topk + j;
      const int32_t e = ids[slot];
      const double gw = (double)gate_w[slot];
      const uint8_t *c13, *s13, *c2, *s2;
      double g13, g2;
      int64_t r, n;
      if (e < 0 || (int64_t)e >= E) continue;  /* out-of-range slot: nothing */
      c13 = w13_codes + (int64_t)e * (2 * I) * (H / 2);
      s13 = w13_scales + (int64_t)e * (2 * I) * (H / 16);
      c2 = w2_codes + (int64_t)e * H * (I / 2);
      s2 = w2_scales + (int64_t)e * H * (I / 16);
      g13 = (double)w13_g[e] * (double)g_a13;   /* exact: two fp32 factors */
      g2 = (double)w2_g[e] * (double)g_a2;
      /* gate_up of the quantized token: a = g13 * g_a13 * W13 . xq */
#pragma omp parallel for schedule(static)
      for (r = 0; r < 2 * I; ++r) {
        double d;
        row_dot(c13, s13, H, r, xq, &d, NULL);
        a[r] = g13 * d;
      }
      /* SwiGLU, one rounding to bf16 */
      for (r = 0; r < I; ++r) {
        double G = a[r], U = a[I + r];
        hb[r] = oracle_bf16_from_double(G / (1.0 + exp(-G)) * U);
        if (h_out) h_out[slot * I + r] = hb[r];
      }
      /* h on the NVFP4 grid of the static scale g_a2 (from h_in if given) */
      quantize_decode_row(h_in ? h_in + slot * I : hb, I, g_a2, hc, hs, hq);
      if (hq_codes) memcpy(hq_codes + slot * (I / 2), hc, (size_t)(I / 2));
      if (hq_scales) memcpy(hq_scales + slot * (I / 16), hs, (size_t)(I / 16));
      /* down, then combine by gate weight */
#pragma omp parallel for schedule(static)
      for (n = 0; n < H; ++n) {
        double d, ad;
        row_dot(c2, s2, I, n, hq, &d, &ad);
        y[m * H + n] += gw * (g2 * d);
        if (bound) bound[m * H + n] += fabs(gw) * fabs(g2) * ad;
      }
    }
    /* the shared expert: W4A16 on the token's unquantized activations */
    if (Is > 0) {
      double* xv = (double*)malloc((size_t)H * sizeof(double) + 8);
      for (k = 0; k < H; ++k) xv[k] = bf16_value(x[m * H + k]);
      shared_ffn_add(ws13_codes, ws13_scales, (double)ws13_g[0], ws2_codes, ws2_scales,
                     (double)ws2_g[0], xv, H, Is, y + m * H, bound ? bound + m * H : NULL,
                     NULL);
      free(xv);
    }
    free(xc);
    free(xs);
    free(xq);
    free(a);
    free(hb);
    free(hc);
    free(hs);
    free(hq);
  }
  return ORACLE_OK;
}
