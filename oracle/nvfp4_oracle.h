/*
 * nvfp4_oracle.h -- plain CPU oracle for the NVFP4 (g16) W4A16 small-M GEMV
 * and its MoE expert-slot variant.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the package smoke check and
 * the benchmark's CPU-baseline leg may load this library. The GPU product
 * path never links, imports or calls it, and it shares no code, header or
 * table with the GPU path.
 *
 * What is computed follows the blueprint pages for GLM-5.3-Flash-NVFP4 on
 * GB10: graph.json node "l0.kda.q" (steps "act bf16", "weight
 * nvfp4/g16->bf16", "accumulate f32", "scale f32"), the blueprint page's
 * Precision table (format "nvfp4/g16": 16-element groups), card.json
 * performance[6].note ("E2M1 + UE4M3/16" weight, BF16 activation), and for the
 * MoE variant graph.json nodes "l3.moe.experts_act" (silu_mul) and
 * "l3.moe.blend" (scatter/combine in f32). The bit layouts of E2M1 and E4M3
 * are not on the pages; they are the public OCP Microscaling (MX) v1.0
 * element formats FP4 E2M1 and FP8 E4M3.
 *
 * Precision: the quantisation decisions (pack) are taken in IEEE fp32 with
 * round-to-nearest-even, the precision the GPU kernel takes them in, so that
 * codes and scales are comparable byte for byte. Dot products are exact
 * (every term is exact in fp64) and summed in fp64.
 */
#ifndef NVFP4_ORACLE_H
#define NVFP4_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes of the oracle entry points. */
#define ORACLE_OK 0
#define ORACLE_ERR_SHAPE (-1)   /* K not a multiple of 16, or a negative size */
#define ORACLE_ERR_NONFINITE (-2) /* an input weight is NaN or Inf */
#define ORACLE_ERR_GSCALE (-3)  /* tensor scale not finite and > 0 */

/* Element decoders. */
double oracle_e2m1_value(unsigned code);   /* 4-bit code -> value; code 8 is -0.0 */
double oracle_e4m3_value(unsigned byte);   /* 8-bit E4M3FN -> value; 0x7F/0xFF NaN */

/* Element encoders: nearest representable value, ties to the even code,
   saturating at the largest finite magnitude (448 for E4M3, 6 for E2M1).
   e4m3: non-positive or NaN input encodes to 0x00 (the block scale is never
   negative). e2m1: a negative input whose magnitude rounds to 0 encodes to
   +0 (0x0). */
unsigned oracle_e4m3_encode(float r);
unsigned oracle_e2m1_encode(float t);

/* Quantise fp32 W[N,K] (row-major) to NVFP4 g16:
   codes[N, K/2]: byte j of row n holds element 2j in the low nibble and
                  element 2j+1 in the high nibble;
   scales[N, K/16]: one E4M3 byte per 16 consecutive elements of a row;
   *gscale_out: the fp32 tensor scale g.
   g = max|W| / 2688 (= 6*448), or 1 for an all-zero tensor, unless
   gscale_override is non-NULL, in which case g = *gscale_override. */
int oracle_pack(const float* W, int64_t N, int64_t K, uint8_t* codes,
                uint8_t* scales, float* gscale_out, const float* gscale_override);

/* W_out[n,k] = (e2m1 * s) * g in fp32: one rounding, at the multiply by g. */
int oracle_dequant(const uint8_t* codes, const uint8_t* scales, float g,
                   int64_t N, int64_t K, float* W_out);

/* y[m, n] = g * sum_k e2m1(c[n,k]) * s[n,k/16] * x[m,k]   (fp64)
   absdot[m, n] = |g| * sum_k |e2m1 * s * x|                  (fp64, may be NULL)
   x is bf16 given as its 16 bit patterns, row-major [M,K].
   rows: if non-NULL, only the n_rows output rows listed are computed and the
   results are stored densely as y[m, i] for i < n_rows (M x n_rows). */
int oracle_gemv(const uint8_t* codes, const uint8_t* scales, float g,
                const uint16_t* x, int64_t M, int64_t N, int64_t K,
                const int64_t* rows, int64_t n_rows, double* y, double* absdot);

/* MoE expert slots (W4A16), per token m and slot j < topk:
     e = ids[m, j] (slots with e outside [0, E) contribute nothing)
     a = g13[e] * W13[e] . x[m]            (2I values, fp64)
     G = a[0:I], U = a[I:2I]
     h = bf16_rne( G / (1 + exp(-G)) * U ) (fp64, then one rounding to bf16)
     o = g2[e] * W2[e] . h                 (H values, fp64)
     y[m] += gate_w[m, j] * o              (fp64)
   bound[m, n] = sum_j |gate_w| * |g2[e]| * sum_i |e2m1 * s * h_i|.
   h_out (may be NULL): [M*topk, I] bf16 bits of h (zeros for skipped slots).
   Weights: w13 codes [E, 2I, H/2], scales [E, 2I, H/16], g13 [E];
            w2  codes [E, H, I/2],  scales [E, H, I/16],  g2  [E]. */
int oracle_moe(const uint8_t* w13_codes, const uint8_t* w13_scales, const float* w13_g,
               const uint8_t* w2_codes, const uint8_t* w2_scales, const float* w2_g,
               const uint16_t* x, const int32_t* ids, const float* gate_w,
               int64_t M, int64_t E, int64_t H, int64_t I, int64_t topk,
               double* y, double* bound, uint16_t* h_out);

/* MoE with a shared expert (graph.json nodes "l3.moe.shared_gate_up",
   "l3.moe.shared_act", "l3.moe.shared_down" and "l3.moe.blend", which takes
   the routed slots and the shared output): y is oracle_moe's y plus, for every
   token m,
     a   = gs13 * WS13 . x[m]                     (2 Is values)
     hs  = bf16( silu(a[0:Is]) * a[Is:2Is] )
     y[m] += gs2 * WS2 . hs
   added after the routed slots, with weight 1; bound grows by
   |gs2| * sum |WS2 * hs|. hs_out (may be NULL): [M, Is] bf16 bits of hs.
   Shared weights: codes [2 Is, H/2], scales [2 Is, H/16], gs13 [1];
                   codes [H, Is/2],  scales [H, Is/16],  gs2 [1]. */
int oracle_moe_shared(const uint8_t* w13_codes, const uint8_t* w13_scales, const float* w13_g,
                      const uint8_t* w2_codes, const uint8_t* w2_scales, const float* w2_g,
                      const uint16_t* x, const int32_t* ids, const float* gate_w,
                      int64_t M, int64_t E, int64_t H, int64_t I, int64_t topk,
                      const uint8_t* ws13_codes, const uint8_t* ws13_scales, const float* ws13_g,
                      const uint8_t* ws2_codes, const uint8_t* ws2_scales, const float* ws2_g,
                      int64_t Is, double* y, double* bound, uint16_t* h_out, uint16_t* hs_out);

/* W4A4 (card.json "W4A4 NVFP4 x NVFP4 (static input scale)"; graph.json node
   "l0.mlp.xn_quant", op act_quant, bf16 -> nvfp4/g16, step "compute f32").
   oracle_quantize_act: each row of bf16 x[M, K] is quantized to NVFP4 g16
   like a weight row, with the given static tensor scale g_x in place of
   max|x| / 2688 (steps 2-4 of oracle_pack on the exact fp32 values of x).
   Codes [M, K/2], scales [M, K/16].
   oracle_gemv_w4a4: y[m, n] = g_w * g_x * sum_k (e2m1_w * s_w) * (e2m1_x * s_x)
   in fp64 (every product exact); absdot the same with |.|; rows as in
   oracle_gemv. */
int oracle_quantize_act(const uint16_t* x, int64_t M, int64_t K, float g_x, uint8_t* codes,
                        uint8_t* scales);
int oracle_gemv_w4a4(const uint8_t* codes_w, const uint8_t* scales_w, float g_w,
                     const uint8_t* codes_x, const uint8_t* scales_x, float g_x,
                     int64_t M, int64_t N, int64_t K, const int64_t* rows, int64_t n_rows,
                     double* y, double* absdot);

/* W4A4 MoE (card.json performance[64] and [65]: the routed gate|up and down
   union sweeps of W4A4 experts; performance[24] and graph.json node
   "l0.mlp.xn_quant": activations quantized with a static input scale; the
   shared expert stays W4A16, card.json performance[4] and [9]). Per token m:
     xq = e2m1 * s of oracle_quantize_act(x[m], g_a13)      (exact values)
   and per valid slot j with expert e:
     a  = g13[e] * g_a13 * W13[e] . xq                       (2I values, fp64)
     h  = bf16( silu(a[0:I]) * a[I:2I] )                     (one rounding)
     hq = e2m1 * s of oracle_quantize_act(h, g_a2)            (exact values)
     y[m] += gate_w[m, j] * (g2[e] * g_a2 * W2[e] . hq)       (fp64)
   then the shared expert as in oracle_moe_shared, on the unquantized x
   (skipped when Is == 0; its pointers may then be NULL).
   h_in (may be NULL): [M*topk, I] bf16 bits used in place of h for the
   quantization and the down projection of every valid slot, so that a
   caller can take the rounding decisions on an h computed elsewhere; h_out
   still receives the h computed here. hq_codes [M*topk, I/2] and hq_scales
   [M*topk, I/16] (may be NULL) receive the quantized h (zeros for skipped
   slots). bound as in oracle_moe, with |g2[e] * g_a2| and |hq|. */
int oracle_moe_w4a4(const uint8_t* w13_codes, const uint8_t* w13_scales, const float* w13_g,
                    const uint8_t* w2_codes, const uint8_t* w2_scales, const float* w2_g,
                    const uint16_t* x, const int32_t* ids, const float* gate_w,
                    int64_t M, int64_t E, int64_t H, int64_t I, int64_t topk,
                    float g_a13, float g_a2,
                    const uint8_t* ws13_codes, const uint8_t* ws13_scales, const float* ws13_g,
                    const uint8_t* ws2_codes, const uint8_t* ws2_scales, const float* ws2_g,
                    int64_t Is, const uint16_t* h_in, double* y, double* bound,
                    uint16_t* h_out, uint8_t* hq_codes, uint8_t* hq_scales);

/* Round a double to the nearest bf16 (ties to even), returning its bits. */
uint16_t oracle_bf16_from_double(double v);

#ifdef __cplusplus
}
#endif
#endif
