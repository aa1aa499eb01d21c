// g8_ops.h -- pieces shared by the eight-token matrix-core GEMV kernels
// (gemv_g8.hip: workgroups split K; gemv_g8r.hip: wavefronts split rows):
// the E2M1 decode of an MFMA B fragment, the DPP row rotation that builds the
// second A operand of a window, and the merge of the two blocks' halves of a
// tile partial. The MFMA layout and the x arrangement they assume are
// described in gemv_g8.hip.
#pragma once

#include "device.h"

namespace nvfp4 {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

constexpr int kG8Slice = 256;                      // k per slice
constexpr int kG8Pitch = 144;                      // staged code row: 128 bytes + 16 (bank skew)
constexpr int kG8StageBytes = 16 * kG8Pitch + 16 * 16;   // codes, then scales

__device__ __forceinline__ bf16x8_t g8_e2m1x8(uint32_t w) {
  const bf16x2_t b0 = e2m1x2_to_bf16<0>(w);
  const bf16x2_t b1 = e2m1x2_to_bf16<1>(w);
  const bf16x2_t b2 = e2m1x2_to_bf16<2>(w);
  const bf16x2_t b3 = e2m1x2_to_bf16<3>(w);
  bf16x8_t r;
  r[0] = b0[0]; r[1] = b0[1]; r[2] = b1[0]; r[3] = b1[1];
  r[4] = b2[0]; r[5] = b2[1]; r[6] = b3[0]; r[7] = b3[1];
  return r;
}

__device__ __forceinline__ bf16x8_t g8_bf16x8(u32x4_t v) {
  bf16x8_t r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

// v of lane l ^ 8 (the other half of the lane's 16-lane row)
__device__ __forceinline__ uint32_t g8_row_ror8(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, true);   // row_ror:8
}

// The two blocks' halves of a tile partial added: lanes l and l + 32 hold the
// same (token, row) for the two blocks of each MFMA. One half-wave exchange
// per pair of registers: lanes < 32 receive registers 0 and 2 (tokens
// 4 g + 0, 4 g + 2), lanes >= 32 registers 1 and 3 (tokens 4 (g - 2) + 1,
// 4 (g - 2) + 3); each sum is (first block) + (second block).
__device__ __forceinline__ f32x2_t g8_merge_halves(f32x4_t v) {
  f32x2_t r;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[2 * k]),
                                                    __float_as_uint(v[2 * k + 1]), false, false);
    // p[0] = {v[2k] of lanes 0..31, v[2k+1] of lanes 0..31},
    // p[1] = {v[2k] of lanes 32..63, v[2k+1] of lanes 32..63}
    r[k] = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  }
  return r;
}

}  // namespace nvfp4
