// gemv_core.h -- the wavefront-level NVFP4 g16 dot-product engine used by the
// vector-ALU dense GEMV (bf16 activations, and NVFP4 activations for W4A4)
// and by the MoE gate|up sweep.
//
// Layout of the work: one wavefront owns R weight rows at a time. The K axis
// of a row is cut into 32-element chunks (16 code bytes = one 128-bit load,
// plus 2 scale bytes); lane l takes chunks l, l+64, l+128, ... so that each
// wavefront load instruction reads 1 KiB of contiguous codes. A chunk is
// decoded once (v_cvt_scalef32_pk_bf16_fp4, exact) and reused for every
// activation row; per 16-element block and activation row, 8 bf16 pair dots
// (v_dot2_f32_bf16) give a block partial that is multiplied by the block's
// E4M3 scale and accumulated in fp32. Lanes are summed at the end
// (wave_sum: DPP within 16-lane rows, v_readlane across them).
#pragma once

#include "device.h"

namespace nvfp4 {

// Activations staged in LDS (kernels where every wavefront of a workgroup
// reads the same rows of x): 16-byte unit u holds x[8u .. 8u+7] of the
// row-major [M, K] array; chunk c (32 elements) is units 4c .. 4c+3, its
// quarter q stored at unit 4c + (q ^ ((c >> 2) & 3)). A lane reads one
// chunk per 128-bit load pair and 16 lanes read 16 consecutive chunks, which
// the swizzle puts on distinct banks (K a multiple of 512 keeps the pattern
// the same in every row).
__device__ __forceinline__ int x1x_unit(int u) {
  const int c = u >> 2;
  return 4 * c + ((u & 3) ^ ((c >> 2) & 3));
}

// the nu units of x, UPT per thread of NT (surplus threads repeat the last):
// loaded into registers first, so that other loads can be issued before the
// LDS stores wait for them
template <int NT, int UPT>
__device__ __forceinline__ void x1x_load(const uint16_t* __restrict__ xs, int nu,
                                         u32x4_t (&xv)[UPT]) {
#pragma unroll
  for (int k = 0; k < UPT; ++k) {
    const int u0 = (int)threadIdx.x + NT * k;
    xv[k] = reinterpret_cast<const u32x4_t*>(xs)[u0 < nu ? u0 : nu - 1];
  }
}
template <int NT, int UPT>
__device__ __forceinline__ void x1x_store(u32x4_t* xl, int nu, const u32x4_t (&xv)[UPT]) {
#pragma unroll
  for (int k = 0; k < UPT; ++k) {
    const int u0 = (int)threadIdx.x + NT * k;
    xl[x1x_unit(u0 < nu ? u0 : nu - 1)] = xv[k];
  }
}

// out[r][m] = sum_k e2m1(c[row_r, k]) * s[row_r, k/16] * x_m[k]  (no tensor
// scale), for r < R and m < ns (ns <= MS; entries m >= ns are left at 0).
// Every lane of the wavefront receives the totals. `rows[r]` must be valid
// row indices (callers clamp ragged tails and drop the duplicate results).
template <int MS, int R>
__device__ __forceinline__ void wave_row_dots(const uint8_t* __restrict__ codes,
                                              const uint8_t* __restrict__ scales,
                                              int64_t K, const int64_t (&rows)[R],
                                              const uint16_t* const (&xs)[MS], int ns,
                                              float (&out)[R][MS]) {
  const int lane = threadIdx.x & 63;
  const int64_t C = K >> 5;        // chunks per row
  const int64_t cb = K >> 1;       // code bytes per row
  const int64_t sb = K >> 4;       // scale bytes per row
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MS; ++m) out[r][m] = 0.0f;

  for (int64_t c = lane; c < C; c += 64) {
    u32x4_t q[R];
    uint32_t sw[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      q[r] = load_stream(codes + rows[r] * cb + c * 16);
      sw[r] = *reinterpret_cast<const uint16_t*>(scales + rows[r] * sb + c * 2);
    }
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      bf16x2_t wd[R][8];
      float s[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const uint32_t w0 = b ? q[r].z : q[r].x;
        const uint32_t w1 = b ? q[r].w : q[r].y;
        wd[r][0] = e2m1x2_to_bf16<0>(w0);
        wd[r][1] = e2m1x2_to_bf16<1>(w0);
        wd[r][2] = e2m1x2_to_bf16<2>(w0);
        wd[r][3] = e2m1x2_to_bf16<3>(w0);
        wd[r][4] = e2m1x2_to_bf16<0>(w1);
        wd[r][5] = e2m1x2_to_bf16<1>(w1);
        wd[r][6] = e2m1x2_to_bf16<2>(w1);
        wd[r][7] = e2m1x2_to_bf16<3>(w1);
        s[r] = b ? e4m3_to_f32<1>(sw[r]) : e4m3_to_f32<0>(sw[r]);
      }
#pragma unroll
      for (int m = 0; m < MS; ++m) {
        if (m < ns) {
          const uint4* xp = reinterpret_cast<const uint4*>(xs[m] + c * 32 + b * 16);
          const uint4 xa = xp[0], xb = xp[1];
          const bf16x2_t xv[8] = {as_bf16x2(xa.x), as_bf16x2(xa.y), as_bf16x2(xa.z),
                                  as_bf16x2(xa.w), as_bf16x2(xb.x), as_bf16x2(xb.y),
                                  as_bf16x2(xb.z), as_bf16x2(xb.w)};
#pragma unroll
          for (int r = 0; r < R; ++r) {
            float p = 0.0f;
#pragma unroll
            for (int j = 0; j < 8; ++j) p = dot2(wd[r][j], xv[j], p);
            out[r][m] = __builtin_fmaf(p, s[r], out[r][m]);
          }
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MS; ++m)
      if (m < ns) out[r][m] = wave_sum(out[r][m]);
}

// The same with NVFP4 activations (W4A4): activation row m is codes xc[m]
// (two E2M1 per byte) and E4M3 scales xsc[m], one per 16 elements. Per
// 16-element block, the 16 products e2m1_w * e2m1_x (exact in bf16 inputs)
// are summed exactly (each is a multiple of 1/4 below 36), and the block sum
// times s_w * s_x (a product of two E4M3 values, exact in fp32) is exact too:
// accumulation is the only rounding.
template <int MS, int R>
__device__ __forceinline__ void wave_row_dots_q(const uint8_t* __restrict__ codes,
                                                const uint8_t* __restrict__ scales,
                                                int64_t K, const int64_t (&rows)[R],
                                                const uint8_t* const (&xc)[MS],
                                                const uint8_t* const (&xsc)[MS],
                                                float (&out)[R][MS]) {
  const int lane = threadIdx.x & 63;
  const int64_t C = K >> 5, cb = K >> 1, sb = K >> 4;
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MS; ++m) out[r][m] = 0.0f;

  for (int64_t c = lane; c < C; c += 64) {
    u32x4_t q[R], qx[MS];
    uint32_t sw[R], swx[MS];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      q[r] = load_stream(codes + rows[r] * cb + c * 16);
      sw[r] = *reinterpret_cast<const uint16_t*>(scales + rows[r] * sb + c * 2);
    }
#pragma unroll
    for (int m = 0; m < MS; ++m) {
      qx[m] = *reinterpret_cast<const u32x4_t*>(xc[m] + c * 16);
      swx[m] = *reinterpret_cast<const uint16_t*>(xsc[m] + c * 2);
    }
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      bf16x2_t wd[R][8];
      float s[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const uint32_t w0 = b ? q[r].z : q[r].x;
        const uint32_t w1 = b ? q[r].w : q[r].y;
        wd[r][0] = e2m1x2_to_bf16<0>(w0);
        wd[r][1] = e2m1x2_to_bf16<1>(w0);
        wd[r][2] = e2m1x2_to_bf16<2>(w0);
        wd[r][3] = e2m1x2_to_bf16<3>(w0);
        wd[r][4] = e2m1x2_to_bf16<0>(w1);
        wd[r][5] = e2m1x2_to_bf16<1>(w1);
        wd[r][6] = e2m1x2_to_bf16<2>(w1);
        wd[r][7] = e2m1x2_to_bf16<3>(w1);
        s[r] = b ? e4m3_to_f32<1>(sw[r]) : e4m3_to_f32<0>(sw[r]);
      }
#pragma unroll
      for (int m = 0; m < MS; ++m) {
        const uint32_t v0 = b ? qx[m].z : qx[m].x;
        const uint32_t v1 = b ? qx[m].w : qx[m].y;
        const bf16x2_t xv[8] = {e2m1x2_to_bf16<0>(v0), e2m1x2_to_bf16<1>(v0),
                                e2m1x2_to_bf16<2>(v0), e2m1x2_to_bf16<3>(v0),
                                e2m1x2_to_bf16<0>(v1), e2m1x2_to_bf16<1>(v1),
                                e2m1x2_to_bf16<2>(v1), e2m1x2_to_bf16<3>(v1)};
        const float sx = b ? e4m3_to_f32<1>(swx[m]) : e4m3_to_f32<0>(swx[m]);
#pragma unroll
        for (int r = 0; r < R; ++r) {
          float p = 0.0f;
#pragma unroll
          for (int j = 0; j < 8; ++j) p = dot2(wd[r][j], xv[j], p);
          out[r][m] = __builtin_fmaf(p, s[r] * sx, out[r][m]);
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MS; ++m) out[r][m] = wave_sum(out[r][m]);
}

}  // namespace nvfp4
