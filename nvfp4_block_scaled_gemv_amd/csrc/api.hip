// api.hip -- the extern "C" boundary: host-side argument checks, then the
// launches on the caller's stream. No allocation, no synchronisation.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "nvfp4_gemv.h"
#include "internal.h"

static_assert(NVFP4_MAX_M == NVFP4_MAX_M_INTERNAL, "M limit mismatch");
static_assert(NVFP4_MOE_MAX_M == NVFP4_MOE_MAX_M_INTERNAL, "MoE M limit mismatch");
static_assert(NVFP4_MAX_TOPK == NVFP4_MAX_TOPK_INTERNAL, "topk limit mismatch");

namespace {

thread_local char g_last_error[512] = "";

nvfp4_status fail(nvfp4_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

void clear_error() { g_last_error[0] = '\0'; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// [a, a + na) and [b, b + nb) share a byte.
bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

nvfp4_status hip_result(hipError_t e, const char* what) {
  if (e != hipSuccess)
    return fail(NVFP4_ERR_HIP, "%s: %s (%s)", what, hipGetErrorName(e), hipGetErrorString(e));
  return NVFP4_OK;
}

}  // namespace

static_assert(NVFP4_MAX_SEGMENTS == nvfp4::kMaxSegments, "segment limit mismatch");

extern "C" {

int nvfp4_abi_version(void) { return NVFP4_ABI_VERSION; }

const char* nvfp4_status_string(int status) {
  switch (status) {
    case NVFP4_OK: return "ok";
    case NVFP4_ERR_NULL: return "null pointer";
    case NVFP4_ERR_SHAPE: return "invalid shape";
    case NVFP4_ERR_ALIGN: return "misaligned pointer";
    case NVFP4_ERR_UNSUPPORTED: return "unsupported size";
    case NVFP4_ERR_WORKSPACE: return "workspace too small";
    case NVFP4_ERR_HIP: return "HIP error";
    case NVFP4_ERR_ALIAS: return "output overlaps an input";
    default: return "unknown status";
  }
}

const char* nvfp4_last_error(void) { return g_last_error; }

nvfp4_status nvfp4_pack(const float* W, int64_t N, int64_t K, uint8_t* codes,
                        uint8_t* scales, float* gscale, const float* gscale_override,
                        hipStream_t stream) {
  clear_error();
  if (N < 0 || K < 0 || (K % 16) != 0)
    return fail(NVFP4_ERR_SHAPE, "nvfp4_pack: need N >= 0, K >= 0, K %% 16 == 0 (N=%lld K=%lld)",
                (long long)N, (long long)K);
  const size_t numel = (size_t)N * (size_t)K;
  if (!gscale || (numel && (!W || !codes || !scales)))
    return fail(NVFP4_ERR_NULL, "nvfp4_pack: W, codes, scales and gscale must be non-NULL");
  if (!aligned(W, 16) || !aligned(codes, 8) || !aligned(gscale, 4) ||
      (gscale_override && !aligned(gscale_override, 4)))
    return fail(NVFP4_ERR_ALIGN, "nvfp4_pack: W must be 16-byte, codes 8-byte, gscale 4-byte aligned");
  const size_t wb = numel * 4, cb = numel / 2, sb = numel / 16;
  if (overlap(codes, cb, W, wb) || overlap(scales, sb, W, wb) || overlap(gscale, 4, W, wb) ||
      overlap(codes, cb, scales, sb) || overlap(codes, cb, gscale, 4) ||
      overlap(scales, sb, gscale, 4) || overlap(gscale, 4, gscale_override, 4))
    return fail(NVFP4_ERR_ALIAS, "nvfp4_pack: outputs overlap each other or an input");
  return hip_result(nvfp4::launch_pack(W, N, K, codes, scales, gscale, gscale_override, stream),
                    "nvfp4_pack launch");
}

nvfp4_status nvfp4_dequant(const uint8_t* codes, const uint8_t* scales, const float* gscale,
                           int64_t N, int64_t K, float* W_out, hipStream_t stream) {
  clear_error();
  if (N < 0 || K < 0 || (K % 32) != 0)
    return fail(NVFP4_ERR_SHAPE, "nvfp4_dequant: need N >= 0, K >= 0, K %% 32 == 0 (N=%lld K=%lld)",
                (long long)N, (long long)K);
  const size_t numel = (size_t)N * (size_t)K;
  if (numel == 0) return NVFP4_OK;
  if (!codes || !scales || !gscale || !W_out)
    return fail(NVFP4_ERR_NULL, "nvfp4_dequant: NULL pointer");
  if (!aligned(codes, 16) || !aligned(W_out, 16) || !aligned(gscale, 4))
    return fail(NVFP4_ERR_ALIGN, "nvfp4_dequant: codes and W_out must be 16-byte aligned");
  if (overlap(W_out, numel * 4, codes, numel / 2) || overlap(W_out, numel * 4, scales, numel / 16) ||
      overlap(W_out, numel * 4, gscale, 4))
    return fail(NVFP4_ERR_ALIAS, "nvfp4_dequant: W_out overlaps an input");
  return hip_result(nvfp4::launch_dequant(codes, scales, gscale, N, K, W_out, stream),
                    "nvfp4_dequant launch");
}

nvfp4_status nvfp4_gemv(const uint8_t* codes, const uint8_t* scales, const float* gscale,
                        const uint16_t* x, int64_t M, int64_t N, int64_t K, float* y,
                        hipStream_t stream) {
  clear_error();
  if (M < 0 || N < 0 || K < 0 || (K % 32) != 0)
    return fail(NVFP4_ERR_SHAPE, "nvfp4_gemv: need M, N, K >= 0 and K %% 32 == 0 (M=%lld N=%lld K=%lld)",
                (long long)M, (long long)N, (long long)K);
  if (M > NVFP4_MAX_M || N > NVFP4_MAX_N || K > NVFP4_MAX_K)
    return fail(NVFP4_ERR_UNSUPPORTED,
                "nvfp4_gemv: M=%lld (max %d), N=%lld (max %lld), K=%lld (max %lld)",
                (long long)M, NVFP4_MAX_M, (long long)N, (long long)NVFP4_MAX_N, (long long)K,
                (long long)NVFP4_MAX_K);
  if (M == 0 || N == 0) return NVFP4_OK;
  if (!y) return fail(NVFP4_ERR_NULL, "nvfp4_gemv: y is NULL");
  if (!aligned(y, 4)) return fail(NVFP4_ERR_ALIGN, "nvfp4_gemv: y must be 4-byte aligned");
  const size_t yb = (size_t)M * (size_t)N * 4;
  if (K == 0) return hip_result(nvfp4::launch_fill_zero(y, (size_t)M * (size_t)N, stream),
                                "nvfp4_gemv zero fill");
  if (!codes || !scales || !gscale || !x) return fail(NVFP4_ERR_NULL, "nvfp4_gemv: NULL input");
  if (!aligned(codes, 16) || !aligned(scales, 2) || !aligned(x, 16) || !aligned(gscale, 4))
    return fail(NVFP4_ERR_ALIGN,
                "nvfp4_gemv: codes and x must be 16-byte, scales 2-byte, gscale 4-byte aligned");
  const size_t nk = (size_t)N * (size_t)K;
  if (overlap(y, yb, codes, nk / 2) || overlap(y, yb, scales, nk / 16) ||
      overlap(y, yb, gscale, 4) || overlap(y, yb, x, (size_t)M * (size_t)K * 2))
    return fail(NVFP4_ERR_ALIAS, "nvfp4_gemv: y overlaps an input");
  return hip_result(nvfp4::launch_gemv(codes, scales, gscale, x, (int)M, N, K, y, stream),
                    "nvfp4_gemv launch");
}

nvfp4_status nvfp4_gemv_segments(const nvfp4_gemv_segment* segs, int64_t n_segments,
                                 const uint16_t* x, int64_t M, int64_t K, hipStream_t stream) {
  clear_error();
  if (n_segments < 0 || M < 0 || K < 0 || (K % 32) != 0)
    return fail(NVFP4_ERR_SHAPE,
                "nvfp4_gemv_segments: need n_segments, M, K >= 0 and K %% 32 == 0 "
                "(n=%lld M=%lld K=%lld)",
                (long long)n_segments, (long long)M, (long long)K);
  if (n_segments > NVFP4_MAX_SEGMENTS || M > NVFP4_MAX_M || K > NVFP4_MAX_K)
    return fail(NVFP4_ERR_UNSUPPORTED,
                "nvfp4_gemv_segments: n_segments=%lld (max %d), M=%lld (max %d), K=%lld (max %lld)",
                (long long)n_segments, NVFP4_MAX_SEGMENTS, (long long)M, NVFP4_MAX_M,
                (long long)K, (long long)NVFP4_MAX_K);
  if (n_segments == 0 || M == 0) return NVFP4_OK;
  if (!segs) return fail(NVFP4_ERR_NULL, "nvfp4_gemv_segments: segs is NULL");
  nvfp4::SegDesc d[NVFP4_MAX_SEGMENTS];
  int n = 0;
  int64_t total_n = 0;
  for (int64_t s = 0; s < n_segments; ++s) {
    const nvfp4_gemv_segment& g = segs[s];
    if (g.N < 0)
      return fail(NVFP4_ERR_SHAPE, "nvfp4_gemv_segments: segment %lld has N=%lld < 0",
                  (long long)s, (long long)g.N);
    if (g.N > NVFP4_MAX_N - total_n)
      return fail(NVFP4_ERR_UNSUPPORTED, "nvfp4_gemv_segments: the segments' N exceed %lld",
                  (long long)NVFP4_MAX_N);
    total_n += g.N;
    if (g.N == 0) continue;
    if (!g.y) return fail(NVFP4_ERR_NULL, "nvfp4_gemv_segments: segment %lld y is NULL", (long long)s);
    if (!aligned(g.y, 4))
      return fail(NVFP4_ERR_ALIGN, "nvfp4_gemv_segments: segment %lld y must be 4-byte aligned",
                  (long long)s);
    if (K > 0) {
      if (!g.codes || !g.scales || !g.gscale || !x)
        return fail(NVFP4_ERR_NULL, "nvfp4_gemv_segments: segment %lld has a NULL input",
                    (long long)s);
      if (!aligned(g.codes, 16) || !aligned(g.scales, 2) || !aligned(g.gscale, 4) ||
          !aligned(x, 16))
        return fail(NVFP4_ERR_ALIGN,
                    "nvfp4_gemv_segments: segment %lld: codes and x must be 16-byte, scales "
                    "2-byte, gscale 4-byte aligned", (long long)s);
    }
    d[n++] = {g.codes, g.scales, g.gscale, g.y, g.N};
  }
  if (n == 0) return NVFP4_OK;
  // no output may overlap any input or another output
  for (int a = 0; a < n; ++a) {
    const size_t ya = (size_t)M * (size_t)d[a].N * 4;
    if (K > 0 && overlap(d[a].y, ya, x, (size_t)M * (size_t)K * 2))
      return fail(NVFP4_ERR_ALIAS, "nvfp4_gemv_segments: an output overlaps x");
    for (int b = 0; b < n; ++b) {
      const size_t nk = (size_t)d[b].N * (size_t)K;
      if (K > 0 && (overlap(d[a].y, ya, d[b].codes, nk / 2) ||
                    overlap(d[a].y, ya, d[b].scales, nk / 16) ||
                    overlap(d[a].y, ya, d[b].gscale, 4)))
        return fail(NVFP4_ERR_ALIAS, "nvfp4_gemv_segments: an output overlaps an input");
      if (b != a && overlap(d[a].y, ya, d[b].y, (size_t)M * (size_t)d[b].N * 4))
        return fail(NVFP4_ERR_ALIAS, "nvfp4_gemv_segments: two outputs overlap");
    }
  }
  if (K == 0) {
    for (int a = 0; a < n; ++a) {
      const nvfp4_status st =
          hip_result(nvfp4::launch_fill_zero(d[a].y, (size_t)M * (size_t)d[a].N, stream),
                     "nvfp4_gemv_segments zero fill");
      if (st != NVFP4_OK) return st;
    }
    return NVFP4_OK;
  }
  return hip_result(nvfp4::launch_gemv_segments(d, n, x, (int)M, K, stream),
                    "nvfp4_gemv_segments launch");
}

nvfp4_status nvfp4_quantize_act(const uint16_t* x, int64_t M, int64_t K, const float* gscale_x,
                                uint8_t* codes_x, uint8_t* scales_x, hipStream_t stream) {
  clear_error();
  if (M < 0 || K < 0 || (K % 32) != 0)
    return fail(NVFP4_ERR_SHAPE,
                "nvfp4_quantize_act: need M, K >= 0 and K %% 32 == 0 (M=%lld K=%lld)",
                (long long)M, (long long)K);
  const size_t numel = (size_t)M * (size_t)K;
  if (numel == 0) return NVFP4_OK;
  if (!x || !gscale_x || !codes_x || !scales_x)
    return fail(NVFP4_ERR_NULL, "nvfp4_quantize_act: NULL pointer");
  if (!aligned(x, 16) || !aligned(codes_x, 8) || !aligned(gscale_x, 4))
    return fail(NVFP4_ERR_ALIGN,
                "nvfp4_quantize_act: x must be 16-byte, codes 8-byte, gscale_x 4-byte aligned");
  const size_t xb = numel * 2, cb = numel / 2, sb = numel / 16;
  if (overlap(codes_x, cb, x, xb) || overlap(scales_x, sb, x, xb) ||
      overlap(codes_x, cb, gscale_x, 4) || overlap(scales_x, sb, gscale_x, 4) ||
      overlap(codes_x, cb, scales_x, sb))
    return fail(NVFP4_ERR_ALIAS, "nvfp4_quantize_act: outputs overlap each other or an input");
  return hip_result(nvfp4::launch_quantize_act(x, M, K, gscale_x, codes_x, scales_x, stream),
                    "nvfp4_quantize_act launch");
}

size_t nvfp4_gemv_w4a4_workspace_bytes(int64_t M, int64_t K) {
  if (M < 0 || K < 0) return 0;
  return nvfp4::w4a4_layout(M, K).total;
}

nvfp4_status nvfp4_gemv_w4a4(const uint8_t* codes_w, const uint8_t* scales_w,
                             const float* gscale_w, const uint8_t* codes_x,
                             const uint8_t* scales_x, const float* gscale_x, int64_t M,
                             int64_t N, int64_t K, float* y, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  clear_error();
  if (M < 0 || N < 0 || K < 0 || (K % 32) != 0)
    return fail(NVFP4_ERR_SHAPE,
                "nvfp4_gemv_w4a4: need M, N, K >= 0 and K %% 32 == 0 (M=%lld N=%lld K=%lld)",
                (long long)M, (long long)N, (long long)K);
  if (M > NVFP4_MAX_M || N > NVFP4_MAX_N || K > NVFP4_MAX_K)
    return fail(NVFP4_ERR_UNSUPPORTED,
                "nvfp4_gemv_w4a4: M=%lld (max %d), N=%lld (max %lld), K=%lld (max %lld)",
                (long long)M, NVFP4_MAX_M, (long long)N, (long long)NVFP4_MAX_N, (long long)K,
                (long long)NVFP4_MAX_K);
  if (M == 0 || N == 0) return NVFP4_OK;
  if (!y) return fail(NVFP4_ERR_NULL, "nvfp4_gemv_w4a4: y is NULL");
  if (!aligned(y, 4)) return fail(NVFP4_ERR_ALIGN, "nvfp4_gemv_w4a4: y must be 4-byte aligned");
  const size_t yb = (size_t)M * (size_t)N * 4;
  if (K == 0) return hip_result(nvfp4::launch_fill_zero(y, (size_t)M * (size_t)N, stream),
                                "nvfp4_gemv_w4a4 zero fill");
  if (!codes_w || !scales_w || !gscale_w || !codes_x || !scales_x || !gscale_x)
    return fail(NVFP4_ERR_NULL, "nvfp4_gemv_w4a4: NULL input");
  const size_t need = nvfp4::w4a4_layout(M, K).total;
  if (!workspace || workspace_bytes < need)
    return fail(NVFP4_ERR_WORKSPACE, "nvfp4_gemv_w4a4: workspace of %zu bytes needed, %zu given",
                need, workspace ? workspace_bytes : (size_t)0);
  if (!aligned(codes_w, 16) || !aligned(scales_w, 2) || !aligned(gscale_w, 4) ||
      !aligned(codes_x, 16) || !aligned(scales_x, 2) || !aligned(gscale_x, 4) ||
      !aligned(workspace, 256))
    return fail(NVFP4_ERR_ALIGN,
                "nvfp4_gemv_w4a4: codes 16-byte, scales 2-byte, scales of the tensors 4-byte, "
                "workspace 256-byte aligned");
  const size_t nk = (size_t)N * (size_t)K, mk = (size_t)M * (size_t)K;
  const void* ins[] = {codes_w, scales_w, gscale_w, codes_x, scales_x, gscale_x};
  const size_t insz[] = {nk / 2, nk / 16, 4, mk / 2, mk / 16, 4};
  for (int i = 0; i < 6; ++i)
    if (overlap(y, yb, ins[i], insz[i]) || overlap(workspace, need, ins[i], insz[i]))
      return fail(NVFP4_ERR_ALIAS, "nvfp4_gemv_w4a4: y or workspace overlaps input %d", i);
  if (overlap(y, yb, workspace, need))
    return fail(NVFP4_ERR_ALIAS, "nvfp4_gemv_w4a4: y overlaps the workspace");
  return hip_result(nvfp4::launch_gemv_w4a4(codes_w, scales_w, gscale_w, codes_x, scales_x,
                                            gscale_x, (int)M, N, K, y, workspace, stream),
                    "nvfp4_gemv_w4a4 launch");
}

nvfp4_status nvfp4_gemv_w4a4_segments(const nvfp4_gemv_segment* segs, int64_t n_segments,
                                      const uint8_t* codes_x, const uint8_t* scales_x,
                                      const float* gscale_x, int64_t M, int64_t K,
                                      void* workspace, size_t workspace_bytes,
                                      hipStream_t stream) {
  clear_error();
  const char* fn = "nvfp4_gemv_w4a4_segments";
  if (n_segments < 0 || M < 0 || K < 0 || (K % 32) != 0)
    return fail(NVFP4_ERR_SHAPE, "%s: need n_segments, M, K >= 0 and K %% 32 == 0 "
                "(n=%lld M=%lld K=%lld)", fn, (long long)n_segments, (long long)M, (long long)K);
  if (n_segments > NVFP4_MAX_SEGMENTS || M > NVFP4_MAX_M || K > NVFP4_MAX_K)
    return fail(NVFP4_ERR_UNSUPPORTED, "%s: n_segments=%lld (max %d), M=%lld (max %d), K=%lld (max %lld)",
                fn, (long long)n_segments, NVFP4_MAX_SEGMENTS, (long long)M, NVFP4_MAX_M,
                (long long)K, (long long)NVFP4_MAX_K);
  if (n_segments == 0 || M == 0) return NVFP4_OK;
  if (!segs) return fail(NVFP4_ERR_NULL, "%s: segs is NULL", fn);
  nvfp4::SegDesc d[NVFP4_MAX_SEGMENTS];
  int n = 0;
  int64_t total_n = 0;
  for (int64_t s = 0; s < n_segments; ++s) {
    const nvfp4_gemv_segment& g = segs[s];
    if (g.N < 0)
      return fail(NVFP4_ERR_SHAPE, "%s: segment %lld has N=%lld < 0", fn, (long long)s,
                  (long long)g.N);
    if (g.N > NVFP4_MAX_N - total_n)
      return fail(NVFP4_ERR_UNSUPPORTED, "%s: the segments' N exceed %lld", fn,
                  (long long)NVFP4_MAX_N);
    total_n += g.N;
    if (g.N == 0) continue;
    if (!g.y) return fail(NVFP4_ERR_NULL, "%s: segment %lld y is NULL", fn, (long long)s);
    if (!aligned(g.y, 4))
      return fail(NVFP4_ERR_ALIGN, "%s: segment %lld y must be 4-byte aligned", fn,
                  (long long)s);
    if (K > 0) {
      if (!g.codes || !g.scales || !g.gscale)
        return fail(NVFP4_ERR_NULL, "%s: segment %lld has a NULL input", fn, (long long)s);
      if (!aligned(g.codes, 16) || !aligned(g.scales, 2) || !aligned(g.gscale, 4))
        return fail(NVFP4_ERR_ALIGN, "%s: segment %lld: codes must be 16-byte, scales 2-byte, "
                    "gscale 4-byte aligned", fn, (long long)s);
    }
    d[n++] = {g.codes, g.scales, g.gscale, g.y, g.N};
  }
  if (n == 0) return NVFP4_OK;
  if (K > 0) {
    if (!codes_x || !scales_x || !gscale_x)
      return fail(NVFP4_ERR_NULL, "%s: NULL activation input", fn);
    if (!aligned(codes_x, 16) || !aligned(scales_x, 2) || !aligned(gscale_x, 4))
      return fail(NVFP4_ERR_ALIGN, "%s: codes_x 16-byte, scales_x 2-byte, gscale_x 4-byte "
                  "aligned", fn);
  }
  const size_t need = nvfp4::w4a4_layout(M, K).total;
  if (K > 0) {
    if (!workspace || workspace_bytes < need)
      return fail(NVFP4_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                  workspace ? workspace_bytes : (size_t)0);
    if (!aligned(workspace, 256))
      return fail(NVFP4_ERR_ALIGN, "%s: workspace must be 256-byte aligned", fn);
  }
  // no output (or the workspace) may overlap any input, another output or the workspace
  const size_t mk = (size_t)M * (size_t)K;
  for (int a = 0; a < n; ++a) {
    const size_t ya = (size_t)M * (size_t)d[a].N * 4;
    if (K > 0 && (overlap(d[a].y, ya, codes_x, mk / 2) || overlap(d[a].y, ya, scales_x, mk / 16) ||
                  overlap(d[a].y, ya, gscale_x, 4) || overlap(d[a].y, ya, workspace, need)))
      return fail(NVFP4_ERR_ALIAS, "%s: an output overlaps the activations or the workspace", fn);
    for (int b = 0; b < n; ++b) {
      const size_t nk = (size_t)d[b].N * (size_t)K;
      if (K > 0 && (overlap(d[a].y, ya, d[b].codes, nk / 2) ||
                    overlap(d[a].y, ya, d[b].scales, nk / 16) ||
                    overlap(d[a].y, ya, d[b].gscale, 4)))
        return fail(NVFP4_ERR_ALIAS, "%s: an output overlaps an input", fn);
      if (K > 0 && (overlap(workspace, need, d[b].codes, nk / 2) ||
                    overlap(workspace, need, d[b].scales, nk / 16) ||
                    overlap(workspace, need, d[b].gscale, 4)))
        return fail(NVFP4_ERR_ALIAS, "%s: the workspace overlaps an input", fn);
      if (b != a && overlap(d[a].y, ya, d[b].y, (size_t)M * (size_t)d[b].N * 4))
        return fail(NVFP4_ERR_ALIAS, "%s: two outputs overlap", fn);
    }
  }
  if (K > 0 && (overlap(workspace, need, codes_x, mk / 2) ||
                overlap(workspace, need, scales_x, mk / 16) || overlap(workspace, need, gscale_x, 4)))
    return fail(NVFP4_ERR_ALIAS, "%s: the workspace overlaps the activations", fn);
  if (K == 0) {
    for (int a = 0; a < n; ++a) {
      const nvfp4_status st =
          hip_result(nvfp4::launch_fill_zero(d[a].y, (size_t)M * (size_t)d[a].N, stream),
                     "nvfp4_gemv_w4a4_segments zero fill");
      if (st != NVFP4_OK) return st;
    }
    return NVFP4_OK;
  }
  return hip_result(nvfp4::launch_gemv_w4a4_segments(d, n, codes_x, scales_x, gscale_x, (int)M,
                                                     K, workspace, stream),
                    "nvfp4_gemv_w4a4_segments launch");
}

nvfp4_status nvfp4_stream_read(const void* buf, size_t bytes, uint32_t* sink,
                               hipStream_t stream) {
  clear_error();
  if (bytes % 16 != 0)
    return fail(NVFP4_ERR_SHAPE, "nvfp4_stream_read: bytes=%zu is not a multiple of 16", bytes);
  if (bytes == 0) return NVFP4_OK;
  if (!buf || !sink) return fail(NVFP4_ERR_NULL, "nvfp4_stream_read: NULL pointer");
  if (!aligned(buf, 16) || !aligned(sink, 4))
    return fail(NVFP4_ERR_ALIGN, "nvfp4_stream_read: buf must be 16-byte, sink 4-byte aligned");
  if (overlap(sink, 4, buf, bytes))
    return fail(NVFP4_ERR_ALIAS, "nvfp4_stream_read: sink overlaps buf");
  return hip_result(nvfp4::launch_stream_read(buf, bytes, sink, stream),
                    "nvfp4_stream_read launch");
}

nvfp4_status nvfp4_check_device_faults(hipStream_t stream) {
  clear_error();
  uint32_t fault = 0u;
  const hipError_t e = nvfp4::splitk_take_fault(stream, &fault);
  if (e != hipSuccess)
    return fail(NVFP4_ERR_HIP, "nvfp4_check_device_faults: %s (%s)", hipGetErrorName(e),
                hipGetErrorString(e));
  if (fault != 0u)
    return fail(NVFP4_ERR_HIP,
                "nvfp4_check_device_faults: a split-K GEMV slot wait gave up (fault word %#x); "
                "the tiles concerned hold NaN",
                fault);
  return NVFP4_OK;
}

void nvfp4_debug_set_wait_limit(int polls) { nvfp4::splitk_set_spin_limit(polls); }

size_t nvfp4_moe_workspace_bytes(int64_t M, int64_t H, int64_t I, int64_t topk) {
  if (M < 0 || H < 0 || I < 0 || topk < 0) return 0;
  return nvfp4::moe_layout(M, H, I, topk, 0, false).total;
}

size_t nvfp4_moe_shared_workspace_bytes(int64_t M, int64_t H, int64_t I, int64_t topk,
                                        int64_t I_shared) {
  if (M < 0 || H < 0 || I < 0 || topk < 0 || I_shared < 0) return 0;
  return nvfp4::moe_layout(M, H, I, topk, I_shared, false).total;
}

size_t nvfp4_moe_w4a4_workspace_bytes(int64_t M, int64_t H, int64_t I, int64_t topk,
                                      int64_t I_shared) {
  if (M < 0 || H < 0 || I < 0 || topk < 0 || I_shared < 0) return 0;
  return nvfp4::moe_layout(M, H, I, topk, I_shared, true).total;
}

}  // extern "C"

namespace {

// The current device's scratch array of nvfp4_moe_gemv_noalloc (defined at
// the end of this file), or NULL with the error text set.
void* device_scratch(const char* fn);

// Checks and launch shared by nvfp4_moe_gemv, nvfp4_moe_shared_gemv,
// nvfp4_moe_w4a4_gemv and nvfp4_moe_gemv_noalloc (shared == NULL: no shared
// expert; w4a4: the routed experts take NVFP4 activations with the static
// scales ga13 and ga2; own_ws: the workspace is the library's scratch array,
// looked up after every host-side check, just before the launch).
nvfp4_status moe_checked(const char* fn, const uint8_t* w13_codes, const uint8_t* w13_scales,
                         const float* w13_gscale, const uint8_t* w2_codes,
                         const uint8_t* w2_scales, const float* w2_gscale, const uint16_t* x,
                         const int32_t* expert_ids, const float* gate_w, int64_t M, int64_t E,
                         int64_t H, int64_t I, int64_t topk, const nvfp4_moe_shared* shared,
                         bool w4a4, const float* ga13, const float* ga2, float* y,
                         void* workspace, size_t workspace_bytes, hipStream_t stream,
                         bool own_ws = false) {
  clear_error();
  if (M < 0 || E < 1 || H <= 0 || I <= 0 || topk < 1 || (H % 32) != 0 || (I % 32) != 0)
    return fail(NVFP4_ERR_SHAPE,
                "%s: need M >= 0, E >= 1, topk >= 1, H, I > 0 and multiples of 32 "
                "(M=%lld E=%lld H=%lld I=%lld topk=%lld)",
                fn, (long long)M, (long long)E, (long long)H, (long long)I, (long long)topk);
  const int64_t Is = shared ? shared->I : 0;
  if (shared && (Is <= 0 || (Is % 32) != 0))
    return fail(NVFP4_ERR_SHAPE, "%s: shared expert width I=%lld must be > 0 and a multiple of 32",
                fn, (long long)Is);
  if (M > NVFP4_MOE_MAX_M || topk > NVFP4_MAX_TOPK || I > NVFP4_MOE_MAX_I || Is > NVFP4_MOE_MAX_I ||
      H > NVFP4_MOE_MAX_H)
    return fail(NVFP4_ERR_UNSUPPORTED,
                "%s: M=%lld (max %d), topk=%lld (max %d), I=%lld, shared I=%lld (max %d), "
                "H=%lld (max %d)", fn,
                (long long)M, NVFP4_MOE_MAX_M, (long long)topk, NVFP4_MAX_TOPK, (long long)I,
                (long long)Is, NVFP4_MOE_MAX_I, (long long)H, NVFP4_MOE_MAX_H);
  if (M == 0) return NVFP4_OK;
  if (!w13_codes || !w13_scales || !w13_gscale || !w2_codes || !w2_scales || !w2_gscale || !x ||
      !expert_ids || !gate_w || !y)
    return fail(NVFP4_ERR_NULL, "%s: NULL pointer", fn);
  if (shared && (!shared->w13_codes || !shared->w13_scales || !shared->w13_gscale ||
                 !shared->w2_codes || !shared->w2_scales || !shared->w2_gscale))
    return fail(NVFP4_ERR_NULL, "%s: NULL pointer in the shared expert", fn);
  if (w4a4 && (!ga13 || !ga2)) return fail(NVFP4_ERR_NULL, "%s: NULL static input scale", fn);
  const size_t need = nvfp4::moe_layout(M, H, I, topk, Is, w4a4).total;
  if (own_ws && need > (size_t)NVFP4_NOALLOC_SCRATCH_BYTES)
    return fail(NVFP4_ERR_UNSUPPORTED,
                "%s: M * topk * I * 2 = %zu bytes of activations exceed the %d-byte scratch "
                "array (use nvfp4_moe_gemv with a workspace)",
                fn, need, NVFP4_NOALLOC_SCRATCH_BYTES);
  if (!own_ws && (!workspace || workspace_bytes < need))
    return fail(NVFP4_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned(w13_codes, 16) || !aligned(w2_codes, 16) || !aligned(w13_scales, 2) ||
      !aligned(w2_scales, 2) || !aligned(x, 16) || !aligned(y, 16) ||
      (!own_ws && !aligned(workspace, 256)) ||
      !aligned(expert_ids, 4) || !aligned(gate_w, 4) || !aligned(w13_gscale, 4) ||
      !aligned(w2_gscale, 4))
    return fail(NVFP4_ERR_ALIGN, "%s: alignment rule broken (see nvfp4_gemv.h)", fn);
  if (shared && (!aligned(shared->w13_codes, 16) || !aligned(shared->w2_codes, 16) ||
                 !aligned(shared->w13_scales, 2) || !aligned(shared->w2_scales, 2) ||
                 !aligned(shared->w13_gscale, 4) || !aligned(shared->w2_gscale, 4)))
    return fail(NVFP4_ERR_ALIGN, "%s: alignment rule broken in the shared expert", fn);
  if (w4a4 && (!aligned(ga13, 4) || !aligned(ga2, 4)))
    return fail(NVFP4_ERR_ALIGN, "%s: static input scales must be 4-byte aligned", fn);
  const size_t e13 = (size_t)E * 2 * (size_t)I * (size_t)H, e2 = (size_t)E * (size_t)H * (size_t)I;
  const size_t s13 = 2 * (size_t)Is * (size_t)H, s2 = (size_t)H * (size_t)Is;
  const size_t yb = (size_t)M * (size_t)H * 4, S = (size_t)(M * topk);
  const void* ins[] = {w13_codes, w13_scales, w13_gscale, w2_codes, w2_scales, w2_gscale, x,
                       expert_ids, gate_w,
                       shared ? shared->w13_codes : nullptr, shared ? shared->w13_scales : nullptr,
                       shared ? shared->w13_gscale : nullptr, shared ? shared->w2_codes : nullptr,
                       shared ? shared->w2_scales : nullptr, shared ? shared->w2_gscale : nullptr,
                       w4a4 ? ga13 : nullptr, w4a4 ? ga2 : nullptr};
  const size_t insz[] = {e13 / 2, e13 / 16, (size_t)E * 4, e2 / 2, e2 / 16, (size_t)E * 4,
                         (size_t)M * (size_t)H * 2, S * 4, S * 4,
                         s13 / 2, s13 / 16, 4, s2 / 2, s2 / 16, 4, 4, 4};
  // (the library's own scratch array cannot overlap a caller buffer)
  for (int i = 0; i < 17; ++i) {
    if (overlap(y, yb, ins[i], insz[i]) ||
        (!own_ws && overlap(workspace, need, ins[i], insz[i])))
      return fail(NVFP4_ERR_ALIAS, "%s: y or workspace overlaps input %d", fn, i);
  }
  if (!own_ws && overlap(y, yb, workspace, need))
    return fail(NVFP4_ERR_ALIAS, "%s: y overlaps the workspace", fn);
  if (own_ws) {
    workspace = device_scratch(fn);
    if (!workspace) return NVFP4_ERR_HIP;
  }
  nvfp4::MoeShared sh = {};
  if (shared) {
    sh.c13 = shared->w13_codes;
    sh.s13 = shared->w13_scales;
    sh.g13 = shared->w13_gscale;
    sh.c2 = shared->w2_codes;
    sh.s2 = shared->w2_scales;
    sh.g2 = shared->w2_gscale;
    sh.I = Is;
  }
  const nvfp4::MoeW4a4 q = {ga13, ga2};
  return hip_result(nvfp4::launch_moe(w13_codes, w13_scales, w13_gscale, w2_codes, w2_scales,
                                      w2_gscale, x, expert_ids, gate_w, (int)M, E, H, I,
                                      (int)topk, shared ? &sh : nullptr, w4a4 ? &q : nullptr, y,
                                      workspace, stream),
                    fn);
}

}  // namespace

extern "C" {

nvfp4_status nvfp4_moe_gemv(const uint8_t* w13_codes, const uint8_t* w13_scales,
                            const float* w13_gscale, const uint8_t* w2_codes,
                            const uint8_t* w2_scales, const float* w2_gscale, const uint16_t* x,
                            const int32_t* expert_ids, const float* gate_w, int64_t M, int64_t E,
                            int64_t H, int64_t I, int64_t topk, float* y, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  return moe_checked("nvfp4_moe_gemv", w13_codes, w13_scales, w13_gscale, w2_codes, w2_scales,
                     w2_gscale, x, expert_ids, gate_w, M, E, H, I, topk, nullptr, false, nullptr,
                     nullptr, y, workspace, workspace_bytes, stream);
}

nvfp4_status nvfp4_moe_shared_gemv(const uint8_t* w13_codes, const uint8_t* w13_scales,
                                   const float* w13_gscale, const uint8_t* w2_codes,
                                   const uint8_t* w2_scales, const float* w2_gscale,
                                   const uint16_t* x, const int32_t* expert_ids,
                                   const float* gate_w, int64_t M, int64_t E, int64_t H,
                                   int64_t I, int64_t topk, const nvfp4_moe_shared* shared,
                                   float* y, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream) {
  if (!shared) {
    clear_error();
    return fail(NVFP4_ERR_NULL, "nvfp4_moe_shared_gemv: NULL shared expert");
  }
  return moe_checked("nvfp4_moe_shared_gemv", w13_codes, w13_scales, w13_gscale, w2_codes,
                     w2_scales, w2_gscale, x, expert_ids, gate_w, M, E, H, I, topk, shared, false,
                     nullptr, nullptr, y, workspace, workspace_bytes, stream);
}

nvfp4_status nvfp4_moe_w4a4_gemv(const uint8_t* w13_codes, const uint8_t* w13_scales,
                                 const float* w13_gscale, const uint8_t* w2_codes,
                                 const uint8_t* w2_scales, const float* w2_gscale,
                                 const uint16_t* x, const float* gscale_x, const float* gscale_h,
                                 const int32_t* expert_ids, const float* gate_w, int64_t M,
                                 int64_t E, int64_t H, int64_t I, int64_t topk,
                                 const nvfp4_moe_shared* shared, float* y, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
  return moe_checked("nvfp4_moe_w4a4_gemv", w13_codes, w13_scales, w13_gscale, w2_codes,
                     w2_scales, w2_gscale, x, expert_ids, gate_w, M, E, H, I, topk, shared, true,
                     gscale_x, gscale_h, y, workspace, workspace_bytes, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// nvfp4_moe_gemv_noalloc: nvfp4_moe_gemv with its workspace (the bf16 SwiGLU
// activations h) in a file-scope device array instead of caller memory, for
// callers that cannot allocate. Each device the library runs on holds its own
// copy of the array until the process ends. In host code `scratch` only names
// the symbol: its device address is looked up once per device with
// hipGetSymbolAddress (with that device current) and that address is what
// the kernels receive.

namespace {

static __device__ __align__(256) unsigned char scratch[NVFP4_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch` (looked up on the first call on
// that device), or NULL with the error text set.
void* device_scratch(const char* fn) {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    fail(NVFP4_ERR_HIP, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    fail(NVFP4_ERR_UNSUPPORTED, "%s: device %d is past the %d devices this entry point serves",
         fn, dev, kMaxDevices);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t r = hipGetSymbolAddress((void**)&ptr, HIP_SYMBOL(scratch));
    if (r != hipSuccess || !ptr) {
      fail(NVFP4_ERR_HIP, "%s: hipGetSymbolAddress(scratch) on device %d: %s", fn, dev,
           hipGetErrorString(r));
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

nvfp4_status nvfp4_moe_gemv_noalloc(const uint8_t* w13_codes, const uint8_t* w13_scales,
                                    const float* w13_gscale, const uint8_t* w2_codes,
                                    const uint8_t* w2_scales, const float* w2_gscale,
                                    const uint16_t* x, const int32_t* expert_ids,
                                    const float* gate_w, int64_t M, int64_t E, int64_t H,
                                    int64_t I, int64_t topk, float* y, hipStream_t stream) {
  return moe_checked("nvfp4_moe_gemv_noalloc", w13_codes, w13_scales, w13_gscale, w2_codes,
                     w2_scales, w2_gscale, x, expert_ids, gate_w, M, E, H, I, topk, nullptr,
                     false, nullptr, nullptr, y, nullptr, 0, stream, /*own_ws=*/true);
}

}  // extern "C"
