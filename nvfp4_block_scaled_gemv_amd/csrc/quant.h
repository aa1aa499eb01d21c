// quant.h -- activation quantization with a static scale on gfx950 (W4A4:
// card.json "W4A4 NVFP4 x NVFP4 (static input scale)"; graph.json node
// "l0.mlp.xn_quant", op act_quant, bf16 -> nvfp4/g16).
#pragma once

#include "device.h"

namespace nvfp4 {

// Activation quantization with a static scale g, one lane per element: the
// 16 lanes of the calling lane's DPP row hold one 16-element block and must
// all be active. The block amax is a max over the row (exact and
// order-free); then s = E4M3(amax / (6 g)) and code = E2M1(w / (s g)) with
// the encoders of the weight pack, in IEEE fp32. Returns the decoded value
// e2m1 * s as bf16 bits, which is exact (at most 6 significant bits).
__device__ __forceinline__ uint16_t quantize_decode_lane(float w, float g) {
  float ab = fabsf(w);
  ab = fmaxf(ab, dpp_f32<0xB1>(ab));    // quad_perm [1,0,3,2]
  ab = fmaxf(ab, dpp_f32<0x4E>(ab));    // quad_perm [2,3,0,1]
  ab = fmaxf(ab, dpp_f32<0x141>(ab));   // row_half_mirror
  ab = fmaxf(ab, dpp_f32<0x140>(ab));   // row_mirror: the 16-lane row
  const float r = ab / (6.0f * g);
  const float s = e4m3_to_f32<0>(e4m3_encode(r));
  const uint32_t code = s != 0.0f ? e2m1_encode(w / (s * g)) : 0u;
  const float v = e2m1x2_to_f32<0>(code).x * s;
  return (uint16_t)(__float_as_uint(v) >> 16);
}

}  // namespace nvfp4
