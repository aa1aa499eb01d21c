/*
 * nvfp4_gemv.h -- C ABI of the MI355X (gfx950) NVFP4 g16 W4A16 small-M GEMV
 * library: weight packing, bit-exact dequantisation, the weight-streaming
 * GEMV y[M,N] = x[M,K] . W[N,K]^T for M <= 128 activation rows, and the MoE
 * expert-slot variant for M <= 8 (gather top-k experts by id, SwiGLU,
 * combine by gate weight).
 *
 * The operations are the ones the GLM-5.3-Flash-NVFP4 blueprint pages
 * describe for their decode step:
 *  - weight format "nvfp4/g16" with activation "bf16" (blueprint page,
 *    Precision table, 322 weighted nodes): E2M1 4-bit codes, one unsigned
 *    E4M3 scale per 16 consecutive weights of a row ("E2M1 + UE4M3/16",
 *    card.json performance[6].note) and one fp32 tensor scale;
 *  - per-node steps "act bf16, weight nvfp4/g16->bf16, mma bf16*bf16,
 *    accumulate f32, scale f32" (graph.json node "l0.kda.q");
 *  - the MoE slot GEMV over 8 experts (card.json performance[33],
 *    w4a16_gemv_sw_moe), the union of expert ids over the rows
 *    (performance[31], performance[64]), silu_mul to bf16 (graph.json node
 *    "l3.moe.experts_act") and the f32 combine by gate weight (graph.json node
 *    "l3.moe.blend"). The element bit layouts are OCP MX v1.0 E2M1 / E4M3.
 *
 * Conventions for every entry point:
 *  - every pointer is a DEVICE pointer of the current HIP device; arrays are
 *    row-major and contiguous; the caller owns (allocates and frees) every
 *    buffer. The library allocates no device memory. Its mutable global
 *    state: the per-thread text of nvfp4_last_error(), the fixed array of
 *    nvfp4_moe_gemv_noalloc, one fault word per device (see
 *    nvfp4_check_device_faults) and the wait bound of
 *    nvfp4_debug_set_wait_limit.
 *  - shapes are checked on the host before anything is launched; on a failed
 *    check nothing is launched, the call returns the error code and
 *    nvfp4_last_error() describes it. Device data (ids, scales, the tensor
 *    scale) is not inspected on the host.
 *  - work is enqueued on `stream` (0 = the null stream) and the call returns
 *    without synchronising. A launch failure returns NVFP4_ERR_HIP.
 *  - outputs must not overlap inputs (checked: NVFP4_ERR_ALIAS).
 *  - results are deterministic: no floating-point atomics, fixed reduction
 *    order for a given shape.
 *
 * NVFP4 g16 storage of a weight matrix W[N, K] (N output rows, K inputs;
 * K % 32 == 0 for the GEMV, K % 16 == 0 for pack/dequant):
 *  - codes  uint8[N, K/2]:  byte j of row n holds element 2j in bits 3..0
 *                           and element 2j+1 in bits 7..4 (E2M1, sign in
 *                           the nibble's bit 3);
 *  - scales uint8[N, K/16]: E4M3 (sign bit 0) scale of elements
 *                           16b .. 16b+15 of the row;
 *  - gscale float[1]:       fp32 tensor scale g.
 *  The dequantised weight is w[n,k] = e2m1(code) * e4m3(scale) * g.
 */
#ifndef NVFP4_GEMV_H
#define NVFP4_GEMV_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NVFP4_ABI_VERSION 9

/* Largest number of activation rows (tokens) one dense GEMV call takes (the
   blueprint's "multi_seq" plan arm: 2 to 128 rows). */
#define NVFP4_MAX_M 128
/* Largest number of tokens one MoE call takes. */
#define NVFP4_MOE_MAX_M 8
/* Largest number of expert slots per token in the MoE call. */
#define NVFP4_MAX_TOPK 16
/* Largest MoE intermediate size I (down-projection row length) per call. */
#define NVFP4_MOE_MAX_I (1 << 24)
/* Largest number of output rows N of one dense GEMV call (of all segments
   together): every launch grid then stays within 32-bit work-item counts. */
#define NVFP4_MAX_N (1LL << 30)
/* Largest MoE hidden size H per call. */
#define NVFP4_MOE_MAX_H (1 << 24)
/* Largest K (inputs per row) of one dense or W4A4 GEMV call: the many-token
   kernel addresses a token block's x and a row tile's codes with 32-bit
   offsets. */
#define NVFP4_MAX_K (1LL << 20)

typedef enum nvfp4_status {
  NVFP4_OK = 0,
  NVFP4_ERR_NULL = 1,        /* a required pointer is NULL */
  NVFP4_ERR_SHAPE = 2,       /* negative size or a divisibility rule broken */
  NVFP4_ERR_ALIGN = 3,       /* a pointer is not aligned as documented */
  NVFP4_ERR_UNSUPPORTED = 4, /* a size above its NVFP4_MAX_* / NVFP4_MOE_MAX_* limit */
  NVFP4_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than required */
  NVFP4_ERR_HIP = 6,         /* a HIP call or kernel launch failed */
  NVFP4_ERR_ALIAS = 7        /* an output overlaps an input */
} nvfp4_status;

/* NVFP4_ABI_VERSION of the loaded library. */
int nvfp4_abi_version(void);

/* Static text for a status code (never NULL). */
const char* nvfp4_status_string(int status);

/* Detail of the last failing call on the calling thread ("" if none). The
   text stays valid until the next library call on the same thread. */
const char* nvfp4_last_error(void);

/*
 * nvfp4_pack -- quantise fp32 W[N, K] to NVFP4 g16 (blueprint page Precision
 * table "nvfp4/g16"; card.json performance[6].note "E2M1 + UE4M3/16"), with
 * the two-level recipe of the workload: tensor scale g = max|W| / (6 * 448)
 * (g = 1 for an all-zero W), block scale = E4M3(amax_block / (6 g)), element
 * code = E2M1(w / (s g)). Both encodings round to nearest, ties to the even
 * code, and saturate (448 and 6); negative values that round to 0 become +0.
 * All arithmetic is IEEE fp32 (correctly rounded divisions, no contraction),
 * so the result is bit-for-bit reproducible on any IEEE host.
 *
 *   W              float[N, K], 16-byte aligned. Finite values required; the
 *                  result for NaN/Inf input is unspecified (no fault).
 *   N, K           N >= 0, K >= 0, K % 16 == 0.
 *   codes          uint8[N, K/2] out, 8-byte aligned.
 *   scales         uint8[N, K/16] out.
 *   gscale         float[1] out: g.
 *   gscale_override NULL, or a device float[1] holding g to use instead of
 *                  max|W| / 2688 (must be finite and > 0; not checked).
 *   stream         HIP stream.
 * Errors: NULL, SHAPE, ALIGN, ALIAS, HIP.
 */
nvfp4_status nvfp4_pack(const float* W, int64_t N, int64_t K, uint8_t* codes,
                        uint8_t* scales, float* gscale, const float* gscale_override,
                        hipStream_t stream);

/*
 * nvfp4_dequant -- W_out[n, k] = (e2m1 * s) * g in fp32: the product e2m1 * s
 * is exact and the only rounding is the multiply by g ("weight
 * nvfp4/g16->bf16" step of graph.json node "l0.kda.q", here to fp32).
 *
 *   codes   uint8[N, K/2], 16-byte aligned;  scales uint8[N, K/16];
 *   gscale  float[1];  N >= 0, K >= 0, K % 32 == 0;
 *   W_out   float[N, K] out, 16-byte aligned.
 * Errors: NULL, SHAPE, ALIGN, ALIAS, HIP.
 */
nvfp4_status nvfp4_dequant(const uint8_t* codes, const uint8_t* scales,
                           const float* gscale, int64_t N, int64_t K, float* W_out,
                           hipStream_t stream);

/*
 * nvfp4_gemv -- the W4A16 small-M GEMV of graph.json node "l0.kda.q" (steps
 * act bf16 / weight nvfp4/g16->bf16 / mma / accumulate f32 / scale f32):
 *
 *   y[m, n] = g * sum_k e2m1(c[n,k]) * e4m3(s[n, k/16]) * x[m, k]
 *
 * with fp32 accumulation and the tensor scale applied once at the end.
 * Accuracy: |y - y_exact| <= 1e-3 * sum_k |w * x| + 1e-6.
 *
 *   codes   uint8[N, K/2], 16-byte aligned;  scales uint8[N, K/16], 2-byte
 *           aligned;  gscale float[1];
 *   x       bf16[M, K] given as uint16 bit patterns, 16-byte aligned;
 *   M       0 <= M <= NVFP4_MAX_M;  0 <= N <= NVFP4_MAX_N;  K >= 0, K % 32 == 0;
 *   y       float[M, N] out, 4-byte aligned (M == 0 or N == 0: nothing is
 *           launched; K == 0: y is set to zero).
 * M <= 2 runs on the vector ALUs (and 3 <= M <= 5 when N <= 1024 and K =
 * 4096), 3 <= M <= 8 otherwise on the matrix cores with eight tokens per
 * block half of each MFMA, 9 <= M <= 128 on the matrix cores with
 * the block scale folded into the decoded weights (blueprint "Plan arms":
 * multi_seq 2..128 rows; "Planner settings": w4a16_tc=on).
 * Errors: NULL, SHAPE, ALIGN, UNSUPPORTED (M > NVFP4_MAX_M or N > NVFP4_MAX_N),
 * ALIAS, HIP.
 */
nvfp4_status nvfp4_gemv(const uint8_t* codes, const uint8_t* scales,
                        const float* gscale, const uint16_t* x, int64_t M,
                        int64_t N, int64_t K, float* y, hipStream_t stream);

/* Largest number of matrices one nvfp4_gemv_segments call takes. */
#define NVFP4_MAX_SEGMENTS 8

/* One matrix of a fused multi-projection GEMV (device pointers). */
typedef struct nvfp4_gemv_segment {
  const uint8_t* codes;    /* uint8[N, K/2], 16-byte aligned */
  const uint8_t* scales;   /* uint8[N, K/16], 2-byte aligned */
  const float* gscale;     /* float[1], 4-byte aligned */
  float* y;                /* float[M, N] out, 4-byte aligned */
  int64_t N;               /* rows of this matrix, >= 0 (0: skipped) */
} nvfp4_gemv_segment;

/*
 * nvfp4_gemv_segments -- several NVFP4 matrices that read the same
 * activations (q|k|v, gate|up), in one launch: for every segment s,
 *
 *   y_s[m, n] = g_s * sum_k decode(W_s)[n, k] * x[m, k]
 *
 * exactly as n_segments separate nvfp4_gemv calls would compute it, but the
 * work units of all matrices share one grid, so small matrices no longer leave
 * most of the GPU idle (blueprint card.json performance[6], the segmented
 * W4A16 GEMV, N = 8726 in one launch; plan flag glm_w4a16_gemv_seg).
 *
 *   segs        host array of n_segments descriptors (read during the call
 *               only); the pointers inside are device pointers;
 *   n_segments  0 .. NVFP4_MAX_SEGMENTS;
 *   x           bf16[M, K] shared by every segment, 16-byte aligned;
 *   M, K        as for nvfp4_gemv (M <= NVFP4_MAX_M, K % 32 == 0); the
 *               segments' N together at most NVFP4_MAX_N.
 * No output may overlap any input or another output.
 * Errors: NULL, SHAPE, ALIGN, UNSUPPORTED (n_segments, M or the total N too
 * large), ALIAS, HIP.
 */
nvfp4_status nvfp4_gemv_segments(const nvfp4_gemv_segment* segs, int64_t n_segments,
                                 const uint16_t* x, int64_t M, int64_t K,
                                 hipStream_t stream);

/*
 * nvfp4_moe_workspace_bytes -- device workspace that nvfp4_moe_gemv needs for
 * the given sizes: the bf16 SwiGLU activations h[M*topk, I] (slot-major, at
 * offset 0), rounded up to 256 bytes. Slots whose id is invalid leave their
 * row of h untouched.
 */
size_t nvfp4_moe_workspace_bytes(int64_t M, int64_t H, int64_t I, int64_t topk);

/*
 * nvfp4_moe_gemv -- MoE expert slots, W4A16 (card.json performance[33]
 * w4a16_gemv_sw_moe; performance[31] row union; graph.json nodes
 * "l3.moe.experts_act" and "l3.moe.blend"). For token m and slot j < topk:
 *
 *   e  = expert_ids[m, j]            (an id outside [0, E) adds nothing)
 *   a  = g13[e] * W13[e] . x[m]      (2I values, fp32 accumulation)
 *   h  = bf16( silu(a[0:I]) * a[I:2I] ),  silu(v) = v / (1 + exp(-v))
 *   y[m] += gate_w[m, j] * ( g2[e] * W2[e] . h )
 *
 * Each distinct expert's gate|up rows are streamed once for all slots routed
 * to it (the union of ids over the M rows is found on the device, no host
 * sync). The down projection and the combine are one pass: y[m] is a single
 * dot product over the token's valid slots, reduced in a fixed order
 * (deterministic, no atomics).
 *
 *   w13_codes  uint8[E, 2I, H/2] (rows 0..I-1 gate, I..2I-1 up), 16-byte
 *              aligned; w13_scales uint8[E, 2I, H/16], 2-byte aligned;
 *              w13_gscale float[E];
 *   w2_codes   uint8[E, H, I/2], 16-byte aligned; w2_scales uint8[E, H, I/16],
 *              2-byte aligned; w2_gscale float[E];
 *   x          bf16[M, H] (uint16 bits), 16-byte aligned;
 *   expert_ids int32[M, topk];  gate_w float[M, topk];
 *   M          0 <= M <= NVFP4_MOE_MAX_M; 1 <= topk <= NVFP4_MAX_TOPK; E >= 1;
 *              I <= NVFP4_MOE_MAX_I; H <= NVFP4_MOE_MAX_H;
 *              H % 32 == 0, I % 32 == 0, H > 0, I > 0;
 *   y          float[M, H] out, 16-byte aligned;
 *   workspace  device buffer of at least nvfp4_moe_workspace_bytes(M, H, I,
 *              topk) bytes, 256-byte aligned; overwritten; must not be shared
 *              by calls that may run concurrently.
 * Errors: NULL, SHAPE, ALIGN, UNSUPPORTED, WORKSPACE, ALIAS, HIP.
 */
nvfp4_status nvfp4_moe_gemv(const uint8_t* w13_codes, const uint8_t* w13_scales,
                            const float* w13_gscale, const uint8_t* w2_codes,
                            const uint8_t* w2_scales, const float* w2_gscale,
                            const uint16_t* x, const int32_t* expert_ids,
                            const float* gate_w, int64_t M, int64_t E, int64_t H,
                            int64_t I, int64_t topk, float* y, void* workspace,
                            size_t workspace_bytes, hipStream_t stream);

/*
 * nvfp4_quantize_act -- NVFP4 activations with a static input scale (card.json
 * "W4A4 NVFP4 x NVFP4 (static input scale)"; graph.json node
 * "l0.mlp.xn_quant", op act_quant, bf16 -> nvfp4/g16). Each row of x is
 * quantized like a weight row by nvfp4_pack, with *gscale_x in place of
 * max|x| / 2688:
 *   s = E4M3(amax_block / (6 g_x)),  code = E2M1(x / (s g_x))   (IEEE fp32)
 *
 *   x         bf16[M, K] (uint16 bits), 16-byte aligned, finite;
 *   gscale_x  float[1], > 0 (the static input scale), 4-byte aligned;
 *   codes_x   uint8[M, K/2] out, 8-byte aligned; scales_x uint8[M, K/16] out;
 *   K % 32 == 0.
 * Errors: NULL, SHAPE, ALIGN, ALIAS, HIP.
 */
nvfp4_status nvfp4_quantize_act(const uint16_t* x, int64_t M, int64_t K, const float* gscale_x,
                                uint8_t* codes_x, uint8_t* scales_x, hipStream_t stream);

/*
 * nvfp4_gemv_w4a4_workspace_bytes -- device workspace of nvfp4_gemv_w4a4: the
 * decoded activations (bf16[M, K]) and one float, 256-byte aligned.
 */
size_t nvfp4_gemv_w4a4_workspace_bytes(int64_t M, int64_t K);

/*
 * nvfp4_gemv_w4a4 -- y[M, N] (fp32) = g_w * g_x * decode(W) . decode(x)^T, both
 * operands NVFP4 g16 (card.json performance[20], [24]: the W4A4 dense FFN).
 * M <= 2: one launch; the activation codes are decoded in registers and each
 * 16-block's sum of e2m1_w * e2m1_x, times s_w * s_x, is exact, so fp32
 * accumulation is the only rounding. M >= 3: the activation values
 * e2m1_x * s_x (exact in bf16) are decoded once into the workspace and
 * multiplied by the weight stream as in nvfp4_gemv. Either way g_w * g_x
 * (rounded once to fp32) scales the fp32 sum. The workspace is required for
 * every M (unused when M <= 2).
 *
 *   codes_w, scales_w, gscale_w  the weight, as in nvfp4_gemv;
 *   codes_x   uint8[M, K/2], 16-byte aligned; scales_x uint8[M, K/16], 2-byte
 *             aligned; gscale_x float[1] (from nvfp4_quantize_act);
 *   M         0 <= M <= NVFP4_MAX_M; 0 <= N <= NVFP4_MAX_N; K % 32 == 0;
 *   y         float[M, N] out;
 *   workspace at least nvfp4_gemv_w4a4_workspace_bytes(M, K) bytes,
 *             256-byte aligned; overwritten; must not be shared by calls that
 *             may run concurrently.
 * Errors: NULL, SHAPE, ALIGN, UNSUPPORTED, WORKSPACE, ALIAS, HIP.
 */
nvfp4_status nvfp4_gemv_w4a4(const uint8_t* codes_w, const uint8_t* scales_w,
                             const float* gscale_w, const uint8_t* codes_x,
                             const uint8_t* scales_x, const float* gscale_x, int64_t M,
                             int64_t N, int64_t K, float* y, void* workspace,
                             size_t workspace_bytes, hipStream_t stream);

/*
 * nvfp4_gemv_w4a4_segments -- several NVFP4 weight matrices on the same NVFP4
 * activations (gate|up of the W4A4 dense FFN, card.json performance[20],
 * [24]), in one launch at M <= 2 (two at M >= 3): for every segment s,
 *
 *   y_s = g_s * g_x * decode(W_s) . decode(x)^T
 *
 * exactly as n_segments nvfp4_gemv_w4a4 calls would compute it.
 *
 *   segs        host array of n_segments descriptors, as for
 *               nvfp4_gemv_segments (read during the call only);
 *   n_segments  0 .. NVFP4_MAX_SEGMENTS;
 *   codes_x, scales_x, gscale_x  the activations, as for nvfp4_gemv_w4a4;
 *   M, K        0 <= M <= NVFP4_MAX_M, K % 32 == 0; the segments' N together
 *               at most NVFP4_MAX_N;
 *   workspace   at least nvfp4_gemv_w4a4_workspace_bytes(M, K) bytes,
 *               256-byte aligned; overwritten; must not be shared by calls
 *               that may run concurrently (not needed when K == 0).
 * No output or the workspace may overlap any input, another output or each
 * other.
 * Errors: NULL, SHAPE, ALIGN, UNSUPPORTED, WORKSPACE, ALIAS, HIP.
 */
nvfp4_status nvfp4_gemv_w4a4_segments(const nvfp4_gemv_segment* segs, int64_t n_segments,
                                      const uint8_t* codes_x, const uint8_t* scales_x,
                                      const float* gscale_x, int64_t M, int64_t K,
                                      void* workspace, size_t workspace_bytes,
                                      hipStream_t stream);

/*
 * nvfp4_moe_shared -- the shared expert of a MoE layer: a dense SwiGLU FFN
 * of width Is that every token passes through (graph.json nodes
 * "l3.moe.shared_gate_up", "l3.moe.shared_act", "l3.moe.shared_down"; card.json
 * performance[4] and [9] give gate|up N = 768 + 768, K = 4096 and down
 * N = 4096, K = 768).
 *
 *   w13_codes  uint8[2Is, H/2] (rows 0..Is-1 gate, Is..2Is-1 up), 16-byte
 *              aligned; w13_scales uint8[2Is, H/16], 2-byte aligned;
 *              w13_gscale float[1];
 *   w2_codes   uint8[H, Is/2], 16-byte aligned; w2_scales uint8[H, Is/16],
 *              2-byte aligned; w2_gscale float[1];
 *   I          Is, > 0, a multiple of 32, <= NVFP4_MOE_MAX_I.
 * The structure is read on the host during the call; the arrays are device
 * memory read by the kernels.
 */
typedef struct nvfp4_moe_shared {
  const uint8_t* w13_codes;
  const uint8_t* w13_scales;
  const float* w13_gscale;
  const uint8_t* w2_codes;
  const uint8_t* w2_scales;
  const float* w2_gscale;
  int64_t I;
} nvfp4_moe_shared;

/*
 * nvfp4_moe_shared_workspace_bytes -- device workspace that
 * nvfp4_moe_shared_gemv needs: the routed h[M * topk, I] and the shared
 * hs[M, I_shared] bf16 activations, each 256-byte aligned. 0 for negative
 * sizes.
 */
size_t nvfp4_moe_shared_workspace_bytes(int64_t M, int64_t H, int64_t I, int64_t topk,
                                        int64_t I_shared);

/*
 * nvfp4_moe_shared_gemv -- nvfp4_moe_gemv plus a shared expert, blended as
 * "routed slots + shared" (graph.json node "l3.moe.blend"): for token m,
 *
 *   y[m] = (nvfp4_moe_gemv's y[m])
 *        + gs2 * WS2 . bf16( silu(a[0:Is]) * a[Is:2Is] ),  a = gs13 * WS13 . x[m]
 *
 * with the shared term added after the routed slots (weight 1). The shared
 * expert runs inside the same two launches as the routed slots: its gate|up
 * rows are streamed once for all M tokens, and its down rows join each
 * token's down-and-combine dot product. Deterministic, no atomics.
 *
 * Arguments as nvfp4_moe_gemv, plus
 *   shared     the shared expert (must not be NULL);
 *   workspace  at least nvfp4_moe_shared_workspace_bytes(M, H, I, topk,
 *              shared->I) bytes, 256-byte aligned; overwritten; must not be
 *              shared by calls that may run concurrently.
 * y and the workspace must not overlap any input, the shared arrays included.
 * Errors: NULL, SHAPE, ALIGN, UNSUPPORTED, WORKSPACE, ALIAS, HIP.
 */
nvfp4_status nvfp4_moe_shared_gemv(const uint8_t* w13_codes, const uint8_t* w13_scales,
                                   const float* w13_gscale, const uint8_t* w2_codes,
                                   const uint8_t* w2_scales, const float* w2_gscale,
                                   const uint16_t* x, const int32_t* expert_ids,
                                   const float* gate_w, int64_t M, int64_t E, int64_t H,
                                   int64_t I, int64_t topk, const nvfp4_moe_shared* shared,
                                   float* y, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream);

/*
 * nvfp4_moe_w4a4_workspace_bytes -- device workspace that nvfp4_moe_w4a4_gemv
 * needs: h[M * topk, I] (bf16, offset 0), the shared hs[M, I_shared], then
 * h and x on the NVFP4 grid (bf16 e2m1 * s, [M * topk, I] and [M, H]), each
 * 256-byte aligned. 0 for negative sizes.
 */
size_t nvfp4_moe_w4a4_workspace_bytes(int64_t M, int64_t H, int64_t I, int64_t topk,
                                      int64_t I_shared);

/*
 * nvfp4_moe_w4a4_gemv -- MoE expert slots with W4A4 routed experts (card.json
 * performance[64] and [65]: the gate|up and down union sweeps of NVFP4
 * experts on NVFP4 activations; performance[24]: activations quantized with
 * a static input scale) and an optional W4A16 shared expert (performance[4]
 * and [9]). For token m:
 *
 *   xq = Q(x[m], g_x)                            (NVFP4 g16, static scale g_x)
 *   per valid slot j, e = expert_ids[m, j]:
 *     a  = g13[e] * g_x * W13[e] . xq
 *     h  = bf16( silu(a[0:I]) * a[I:2I] )
 *     y[m] += gate_w[m, j] * ( g2[e] * g_h * W2[e] . Q(h, g_h) )
 *   y[m] += the shared expert's term of nvfp4_moe_shared_gemv on x[m]
 *
 * where Q(v, g) is the quantization of nvfp4_quantize_act (each 16-block:
 * s = E4M3(amax / (6 g)), code = E2M1(v / (s g))) taken back to the values
 * e2m1 * s, which are exact in bf16. Launches on the stream: quantize x,
 * gate|up (shared expert included), quantize h, down and combine; at M == 1
 * gate|up quantizes h itself (three launches).
 *
 * Arguments as nvfp4_moe_gemv, plus
 *   gscale_x   float[1], > 0 and finite: the static input scale of x,
 *              4-byte aligned (device memory);
 *   gscale_h   float[1], > 0 and finite: the static input scale of h;
 *   shared     the shared expert, or NULL for none;
 *   workspace  at least nvfp4_moe_w4a4_workspace_bytes(M, H, I, topk,
 *              shared ? shared->I : 0) bytes, 256-byte aligned; overwritten;
 *              must not be shared by calls that may run concurrently.
 * The static scales are device data and are not checked; other values give
 * unspecified (but memory-safe) results.
 * Errors: NULL, SHAPE, ALIGN, UNSUPPORTED, WORKSPACE, ALIAS, HIP.
 */
nvfp4_status nvfp4_moe_w4a4_gemv(const uint8_t* w13_codes, const uint8_t* w13_scales,
                                 const float* w13_gscale, const uint8_t* w2_codes,
                                 const uint8_t* w2_scales, const float* w2_gscale,
                                 const uint16_t* x, const float* gscale_x, const float* gscale_h,
                                 const int32_t* expert_ids, const float* gate_w, int64_t M,
                                 int64_t E, int64_t H, int64_t I, int64_t topk,
                                 const nvfp4_moe_shared* shared, float* y, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream);

/* Size of the device array that nvfp4_moe_gemv_noalloc keeps its SwiGLU
   activations in (one copy per device, held until the process ends). */
#define NVFP4_NOALLOC_SCRATCH_BYTES (4 << 20)

/*
 * nvfp4_moe_gemv_noalloc -- nvfp4_moe_gemv for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same computation and kernels, with the bf16
 * SwiGLU activations h[M * topk, I] kept in a library-owned device array of
 * NVFP4_NOALLOC_SCRATCH_BYTES bytes (a file-scope __device__ array, one per
 * device) instead of a caller workspace. Nothing is allocated by the call.
 *
 * Arguments as nvfp4_moe_gemv without the workspace. The activations must
 * fit: nvfp4_moe_workspace_bytes(M, H, I, topk) <= NVFP4_NOALLOC_SCRATCH_BYTES
 * (else NVFP4_ERR_UNSUPPORTED, nothing launched). Every call on a device
 * shares that device's array: calls that may overlap on one device (other
 * streams, other host threads) race on it and must be serialised by the
 * caller. The array is overwritten by every call; nothing in it needs to
 * start at zero.
 * Errors: NULL, SHAPE, ALIGN, UNSUPPORTED, ALIAS, HIP.
 */
nvfp4_status nvfp4_moe_gemv_noalloc(const uint8_t* w13_codes, const uint8_t* w13_scales,
                                    const float* w13_gscale, const uint8_t* w2_codes,
                                    const uint8_t* w2_scales, const float* w2_gscale,
                                    const uint16_t* x, const int32_t* expert_ids,
                                    const float* gate_w, int64_t M, int64_t E, int64_t H,
                                    int64_t I, int64_t topk, float* y, hipStream_t stream);

/*
 * nvfp4_stream_read -- measurement aid, not part of the product path: reads
 * `bytes` of device memory once with the 128-bit non-temporal loads and the
 * launch shape of the M = 1 GEMV (one wavefront per 4 KiB) and discards the
 * data. Its throughput is the read bandwidth this device reaches on a pure
 * stream, the ceiling the weight-streaming kernels are reported against, as
 * the blueprint's card.json prices each kernel floor at a measured read
 * bandwidth (performance[*].floor_us at 249 GB/s) next to the nominal one
 * (hardware.memory_bandwidth_gbps, 273).
 *
 *   buf    device memory, 16-byte aligned;  bytes  a multiple of 16;
 *   sink   uint32[1] device memory, 4-byte aligned: written only when the
 *          XOR of all words read equals 0x9E3779B9 (it keeps the loads
 *          alive; the value is of no use), must not overlap buf.
 * Errors: NULL, SHAPE, ALIGN, ALIAS, HIP.
 */
nvfp4_status nvfp4_stream_read(const void* buf, size_t bytes, uint32_t* sink,
                               hipStream_t stream);

/*
 * nvfp4_check_device_faults -- diagnostic: waits for `stream`, then reads and
 * clears the current device's fault word. A kernel sets it when it gives up
 * a bounded internal wait: the split-K GEMV (3 <= M <= 8, K a multiple of 256
 * that the 16-wavefront kernel cannot split) sums a tile's partials once all
 * wavefronts of its workgroup have delivered them, and a wavefront that is
 * four tiles ahead waits for a free slot; after about 4M polls it records
 * the fault and delivers a NaN partial. The results of a call that set the
 * fault are invalid (tiles summed from that partial hold NaN; others may be
 * wrong without showing it). Not seen in normal operation. Synchronises
 * the stream; not for use under graph capture.
 * Returns NVFP4_OK, or NVFP4_ERR_HIP (also on a HIP failure) with
 * nvfp4_last_error() naming the fault.
 */
nvfp4_status nvfp4_check_device_faults(hipStream_t stream);

/*
 * nvfp4_debug_set_wait_limit -- test hook: the number of polls after which
 * the split-K slot wait gives up (0 restores the default of 1 << 22; a
 * negative value makes every tile give up at once, to exercise the fault
 * path). Process-wide and not synchronised with other host threads; applies
 * to launches made after the call.
 */
void nvfp4_debug_set_wait_limit(int polls);

#ifdef __cplusplus
}
#endif
#endif /* NVFP4_GEMV_H */
