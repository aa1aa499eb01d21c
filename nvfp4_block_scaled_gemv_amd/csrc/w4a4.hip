// w4a4.hip -- NVFP4 activations (W4A4) on gfx950.
//
// The pages' W4A4 path (card.json "W4A4 NVFP4 x NVFP4 (static input scale)",
// performance[20], [24], [64], [65]; graph.json node "l0.mlp.xn_quant", op
// act_quant, bf16 -> nvfp4/g16):
//   k_quantize_act: each row of bf16 x[M, K] is quantized like a weight row,
//     with the caller's static tensor scale g_x: s = E4M3(amax / (6 g_x)),
//     code = E2M1(x / (s g_x)), in IEEE fp32 (the same encoders as pack).
//   nvfp4_gemv_w4a4: y = g_w g_x sum_k (e2m1_w s_w)(e2m1_x s_x). At M <= 2
//     the vector-ALU kernel k_gemv_w4a4 (gemv.hip) decodes both operands in
//     registers. At M >= 3 the activation values e2m1_x s_x (at most 6
//     significant bits in [2^-10, 2688], so exact in bf16) are written to the
//     workspace by k_w4a4_prep with the product scale g_w g_x (one fp32
//     rounding), and the bf16 MFMA GEMV kernels do the rest; x is at most
//     8 x K values, so the extra pass moves kilobytes.
//   k_quantize_decode: the same quantization, written back as the decoded
//     bf16 values, for the W4A4 MoE (its x before gate|up, its h before down).
#include "device.h"
#include "internal.h"
#include "quant.h"

namespace nvfp4 {

static inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

W4a4Layout w4a4_layout(int64_t M, int64_t K) {
  W4a4Layout L;
  L.x_off = 0;
  L.g_off = align256((size_t)M * (size_t)K * sizeof(uint16_t));
  L.total = align256(L.g_off + kMaxSegments * sizeof(float));
  return L;
}

// Eight lanes per 16-element block, two elements (one code byte) per lane:
// the block amax by a max over the 8 lanes (DPP within quads and half-rows;
// exact and order-free), then the same scale and element encoders as pack.
// Lane 0 of each group writes the scale byte. n (code bytes) is a multiple
// of 8, so the lanes of a block stay or leave together.
__global__ __launch_bounds__(256) void k_quantize_act(const uint16_t* __restrict__ x, size_t n,
                                                      const float* __restrict__ gscale_x,
                                                      uint8_t* __restrict__ codes,
                                                      uint8_t* __restrict__ scales) {
  const size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n) return;
  const float g = *gscale_x;
  const uint32_t u = reinterpret_cast<const uint32_t*>(x)[t];
  const float w0 = __uint_as_float(u << 16), w1 = __uint_as_float(u & 0xFFFF0000u);
  float ab = fmaxf(fabsf(w0), fabsf(w1));
  ab = fmaxf(ab, dpp_f32<0xB1>(ab));    // quad_perm [1,0,3,2]
  ab = fmaxf(ab, dpp_f32<0x4E>(ab));    // quad_perm [2,3,0,1]
  ab = fmaxf(ab, dpp_f32<0x141>(ab));   // row_half_mirror: the other quad of the 8
  const uint32_t sc = e4m3_encode(ab / (6.0f * g));
  const float s = e4m3_to_f32<0>(sc);
  uint32_t byte = 0u;
  if (s != 0.0f) {
    const float dn = s * g;
    byte = e2m1_encode(w0 / dn) | (e2m1_encode(w1 / dn) << 4);
  }
  codes[t] = (uint8_t)byte;
  if ((t & 7) == 0) scales[t >> 3] = (uint8_t)sc;
}

// The tensor scales g_w of up to kMaxSegments matrices.
struct W4a4Scales {
  const float* g[kMaxSegments];
  int n;
};

// One thread per 32 activation elements (16 code bytes, two blocks): the
// exact bf16 values e2m1 * s; thread s < n also writes g_w[s] * g_x.
__global__ __launch_bounds__(256) void k_w4a4_prep(const uint8_t* __restrict__ codes_x,
                                                   const uint8_t* __restrict__ scales_x,
                                                   size_t nchunks, const W4a4Scales gw,
                                                   const float* __restrict__ g_x,
                                                   uint16_t* __restrict__ xt,
                                                   float* __restrict__ g_prod) {
  const size_t c = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c < (size_t)gw.n) g_prod[c] = *gw.g[c] * *g_x;
  if (c >= nchunks) return;
  const uint4 q = *reinterpret_cast<const uint4*>(codes_x + c * 16);
  const uint32_t sw = (uint32_t)scales_x[2 * c] | ((uint32_t)scales_x[2 * c + 1] << 8);
  const float s0 = e4m3_to_f32<0>(sw), s1 = e4m3_to_f32<1>(sw);
  const uint32_t words[4] = {q.x, q.y, q.z, q.w};
  uint4* o = reinterpret_cast<uint4*>(xt + c * 32);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float s = (i < 2) ? s0 : s1;
    uint32_t out[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const float2_t v = p == 0 ? e2m1x2_to_f32<0>(words[i]) : p == 1 ? e2m1x2_to_f32<1>(words[i])
                       : p == 2 ? e2m1x2_to_f32<2>(words[i]) : e2m1x2_to_f32<3>(words[i]);
      // e2m1 * s is exact in fp32 and has at most 6 significant bits: its
      // upper 16 bits are the exact bf16
      out[p] = (__float_as_uint(v.x * s) >> 16) | (__float_as_uint(v.y * s) & 0xFFFF0000u);
    }
    o[i] = make_uint4(out[0], out[1], out[2], out[3]);
  }
}

// One lane per element, 16 lanes per block (a DPP row): quantize like
// k_quantize_act (block amax by a max over the row, exact and order-free),
// then write the decoded value e2m1 * s as bf16 (exact: at most 6
// significant bits) in place of the code. Row r = element / K is skipped when ids names no expert
// in [0, E) for it. n and K are multiples of 16, so the lanes of a block
// stay or leave together.
__global__ __launch_bounds__(256) void k_quantize_decode(const uint16_t* __restrict__ x,
                                                         size_t n, int64_t K,
                                                         const float* __restrict__ gscale,
                                                         const int32_t* __restrict__ ids,
                                                         int64_t E,
                                                         uint16_t* __restrict__ out) {
  const size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n) return;
  // the element, the scale and the row's id load together (the element's
  // address does not depend on the id, which only decides the write)
  const float g = *gscale;
  const float w = __uint_as_float((uint32_t)x[t] << 16);   // bf16 -> fp32 is exact
  if (ids) {
    const int32_t e = ids[t / (size_t)K];
    if (e < 0 || (int64_t)e >= E) return;
  }
  out[t] = quantize_decode_lane(w, g);
}

hipError_t launch_quantize_decode(const uint16_t* x, int64_t rows, int64_t K,
                                  const float* gscale, const int32_t* ids, int64_t E,
                                  uint16_t* out, hipStream_t stream) {
  const size_t n = (size_t)rows * (size_t)K;
  if (n > 0xFFFFFF00u) return hipErrorInvalidConfiguration;   // a grid counts < 2^32 lanes
  if (n)
    hipLaunchKernelGGL(k_quantize_decode, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                       stream, x, n, K, gscale, ids, E, out);
  return hipGetLastError();
}

hipError_t launch_quantize_act(const uint16_t* x, int64_t M, int64_t K, const float* gscale_x,
                               uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  const size_t n = (size_t)M * (size_t)K / 2;
  if (n > 0xFFFFFF00u) return hipErrorInvalidConfiguration;   // a grid counts < 2^32 lanes
  if (n)
    hipLaunchKernelGGL(k_quantize_act, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                       stream, x, n, gscale_x, codes, scales);
  return hipGetLastError();
}

hipError_t launch_gemv_w4a4_segments(const SegDesc* d, int n, const uint8_t* codes_x,
                                     const uint8_t* scales_x, const float* gscale_x, int M,
                                     int64_t K, void* workspace, hipStream_t stream) {
  if (n < 1 || n > kMaxSegments) return hipErrorInvalidValue;
  if (M <= 2)   // the vector-ALU kernel reads the NVFP4 activations directly
    return launch_gemv_w4a4_valu(d, n, codes_x, scales_x, gscale_x, M, K, stream);
  const W4a4Layout L = w4a4_layout(M, K);
  uint16_t* xt = reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) + L.x_off);
  float* gp = reinterpret_cast<float*>(static_cast<char*>(workspace) + L.g_off);
  W4a4Scales gw = {};
  gw.n = n;
  SegDesc dd[kMaxSegments];
  for (int s = 0; s < n; ++s) {
    gw.g[s] = d[s].gscale;
    dd[s] = d[s];
    dd[s].gscale = gp + s;   // g_w[s] * g_x, written by the prep pass
  }
  const size_t nchunks = (size_t)M * (size_t)K / 32;
  const size_t threads = nchunks > (size_t)n ? nchunks : (size_t)n;
  hipLaunchKernelGGL(k_w4a4_prep, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream,
                     codes_x, scales_x, nchunks, gw, gscale_x, xt, gp);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // the matrix-core kernels at every row count (not the dense route's
  // vector-ALU kernel for small matrices), so that one segments call and
  // separate calls sum in the same order
  if (M > NVFP4_MAX_M_SMALL && !g8_groups_applicable(dd, n, M, K))
    return launch_gemv_mt(dd, n, xt, M, K, stream);
  return launch_gemv_mfma(dd, n, xt, M, K, stream);
}

hipError_t launch_gemv_w4a4(const uint8_t* codes_w, const uint8_t* scales_w,
                            const float* gscale_w, const uint8_t* codes_x,
                            const uint8_t* scales_x, const float* gscale_x, int M, int64_t N,
                            int64_t K, float* y, void* workspace, hipStream_t stream) {
  const SegDesc d = {codes_w, scales_w, gscale_w, y, N};
  return launch_gemv_w4a4_segments(&d, 1, codes_x, scales_x, gscale_x, M, K, workspace, stream);
}

}  // namespace nvfp4
