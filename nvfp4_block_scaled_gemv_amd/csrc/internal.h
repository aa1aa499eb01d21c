// internal.h -- launchers shared between the kernels and the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "segments.h"

// Limits of one call (the public header exports the same values).
#define NVFP4_MAX_M_INTERNAL 128
#define NVFP4_MOE_MAX_M_INTERNAL 8
#define NVFP4_MAX_TOPK_INTERNAL 16
// The largest M of the vector-ALU and the eight-token matrix-core kernels;
// above it the many-token kernel (gemv_mt.hip) runs.
#define NVFP4_MAX_M_SMALL 8

namespace nvfp4 {

hipError_t launch_pack(const float* W, int64_t N, int64_t K, uint8_t* codes,
                       uint8_t* scales, float* gscale, const float* override_g,
                       hipStream_t stream);

hipError_t launch_dequant(const uint8_t* codes, const uint8_t* scales, const float* gscale,
                          int64_t N, int64_t K, float* out, hipStream_t stream);

hipError_t launch_gemv(const uint8_t* codes, const uint8_t* scales, const float* gscale,
                       const uint16_t* x, int M, int64_t N, int64_t K, float* y,
                       hipStream_t stream);

// One launch over n <= kMaxSegments matrices sharing x[M, K] (all N > 0).
hipError_t launch_gemv_segments(const SegDesc* d, int n, const uint16_t* x, int M, int64_t K,
                                hipStream_t stream);

// Matrix-core paths, 2 <= M <= 8 (gemv_mfma.hip routes K % 256 == 0 to
// gemv_g8r.hip, gemv_g8.hip or gemv_splitk.hip; M = 2 only where those two
// apply), and 9 <= M <= 128 (gemv_mt.hip).
bool mt_applicable(int M);
// 2 <= M <= 16 (groups of 8 tokens), K % 256 == 0 and K / 256 splitting
// evenly over at most 16 wavefronts of up to 4 slices (gemv_g8.hip): one
// launch shape per row count and K (g8_shape), or an explicit one
bool g8_applicable(int M, int64_t K);
// 9 <= M <= 16: the same kernel in two groups of 8 tokens (below 2^17 rows)
bool g8_groups_applicable(const SegDesc* d, int n, int M, int64_t K);
void g8_shape(int64_t rows, int64_t K, int M, int* TW, int* S, int* W);
hipError_t launch_gemv_g8(const SegDesc* d, int n, const uint16_t* x, int M, int64_t K,
                          hipStream_t stream);
hipError_t launch_gemv_g8_shape(const SegDesc* d, int n, const uint16_t* x, int M, int64_t K,
                                int TW, int S, hipStream_t stream);
// 2 <= M <= 8 on one very tall matrix (2^17 rows and more, K % 256 == 0,
// K <= 4096; gemv_g8r.hip): wavefronts split the rows, x held once per
// workgroup in LDS
bool g8r_applicable(int M, int n, int64_t N, int64_t K);
hipError_t launch_gemv_g8r(const SegDesc& d, const uint16_t* x, int M, int64_t K,
                           hipStream_t stream);
// 9 <= M <= 128 (gemv_mt.hip): G token groups of 32 per workgroup in
// `tblocks` token blocks, R row wavefronts of 32 rows sharing staged x, W
// k-groups splitting K; mt_shape picks one from the rows, M and K.
struct MtShape {
  int G, tblocks, R, W;
};
MtShape mt_shape(const SegDesc* d, int n, int M, int64_t K);
int64_t mt_lds_bytes(const MtShape& sh);
hipError_t launch_gemv_mt(const SegDesc* d, int n, const uint16_t* x, int M, int64_t K,
                          hipStream_t stream);
hipError_t launch_gemv_mt_shape(const SegDesc* d, int n, const uint16_t* x, int M, int64_t K,
                                const MtShape& sh, hipStream_t stream);
hipError_t launch_gemv_mfma(const SegDesc* d, int n, const uint16_t* x, int M, int64_t K,
                            hipStream_t stream);
bool splitk_applicable(int M, int64_t K);
// the slot-wait bound of later split-K launches (0: the default; negative:
// give up at once) and the read-and-clear of this device's fault word
void splitk_set_spin_limit(int limit);
hipError_t splitk_take_fault(hipStream_t stream, uint32_t* fault);
void splitk_default_shape(int64_t K, int* KS, int* XS, int* D);
hipError_t launch_gemv_splitk(const SegDesc* d, int n, const uint16_t* x, int M, int64_t K,
                              hipStream_t stream);
hipError_t launch_gemv_splitk_shape(const SegDesc* d, int n, const uint16_t* x, int M,
                                    int64_t K, int KS, int XS, int D, int64_t grid,
                                    hipStream_t stream);

// W4A4: activation quantization with a static input scale, and the GEMV on
// quantized activations (workspace: the exact bf16 activations, then the
// product of the two tensor scales).
struct W4a4Layout {
  size_t x_off;   // uint16 bf16 x~[M, K]
  size_t g_off;   // float g_w * g_x, one per matrix (up to kMaxSegments)
  size_t total;   // rounded up to 256 bytes
};
W4a4Layout w4a4_layout(int64_t M, int64_t K);
hipError_t launch_quantize_act(const uint16_t* x, int64_t M, int64_t K, const float* gscale_x,
                               uint8_t* codes, uint8_t* scales, hipStream_t stream);
hipError_t launch_gemv_w4a4(const uint8_t* codes_w, const uint8_t* scales_w,
                            const float* gscale_w, const uint8_t* codes_x,
                            const uint8_t* scales_x, const float* gscale_x, int M, int64_t N,
                            int64_t K, float* y, void* workspace, hipStream_t stream);
// The same over n <= kMaxSegments matrices (all N > 0) sharing the activations;
// the workspace holds up to kMaxSegments tensor-scale products after x~.
hipError_t launch_gemv_w4a4_segments(const SegDesc* d, int n, const uint8_t* codes_x,
                                     const uint8_t* scales_x, const float* gscale_x, int M,
                                     int64_t K, void* workspace, hipStream_t stream);
// W4A4 GEMV at M <= 2 on the vector ALUs, activations read as NVFP4.
hipError_t launch_gemv_w4a4_valu(const SegDesc* d, int n, const uint8_t* codes_x,
                                 const uint8_t* scales_x, const float* gscale_x, int M,
                                 int64_t K, hipStream_t stream);
// bf16 rows [rows, K] quantized with the static scale *gscale and written
// back as the exact bf16 values e2m1 * s (the tensor scale left out). With
// ids, row r is skipped (not written) when ids[r] is outside [0, E).
hipError_t launch_quantize_decode(const uint16_t* x, int64_t rows, int64_t K,
                                  const float* gscale, const int32_t* ids, int64_t E,
                                  uint16_t* out, hipStream_t stream);

hipError_t launch_fill_zero(float* y, size_t n, hipStream_t stream);

// Read `bytes` (a multiple of 16) from buf once; the measurement ceiling.
hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink,
                              hipStream_t stream);

// MoE workspace layout (byte offsets from the workspace base).
struct MoeLayout {
  size_t h_off;       // uint16 bf16 SwiGLU activations h[M * topk, I]
  size_t hs_off;      // the shared expert's hs[M, Is] (empty when Is = 0)
  size_t hq_off;      // W4A4: h on the NVFP4 grid, e2m1 * s as bf16 [M * topk, I]
  size_t xq_off;      // W4A4: x on the NVFP4 grid, e2m1 * s as bf16 [M, H]
  size_t total;       // rounded up to 256 bytes
};
MoeLayout moe_layout(int64_t M, int64_t H, int64_t I, int64_t topk, int64_t Is, bool w4a4);

// The shared expert of a MoE call (I = 0: none). h is set by the launcher.
struct MoeShared {
  const uint8_t* c13;   // codes [2 Is, H/2]
  const uint8_t* s13;   // scales [2 Is, H/16]
  const float* g13;     // [1]
  const uint8_t* c2;    // codes [H, Is/2]
  const uint8_t* s2;    // scales [H, Is/16]
  const float* g2;      // [1]
  int64_t I;            // Is
  uint16_t* h;          // hs [M, Is] in the workspace
};

// W4A4 routed experts: the static input scales of x (gate|up) and of h (down),
// device fp32 [1] each. The shared expert stays W4A16.
struct MoeW4a4 {
  const float* ga13;
  const float* ga2;
};

hipError_t launch_moe(const uint8_t* w13_codes, const uint8_t* w13_scales,
                      const float* w13_gscale, const uint8_t* w2_codes,
                      const uint8_t* w2_scales, const float* w2_gscale, const uint16_t* x,
                      const int32_t* ids, const float* gate_w, int M, int64_t E, int64_t H,
                      int64_t I, int topk, const MoeShared* shared, const MoeW4a4* w4a4,
                      float* y, void* workspace, hipStream_t stream);

}  // namespace nvfp4
