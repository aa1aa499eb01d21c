// device.h -- gfx950 device helpers for NVFP4 g16: element decode through the
// CDNA4 conversion instructions, fp32 encoders for the pack kernel, and
// wavefront reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// 128-bit load with the non-temporal hint: streamed weights are read once.
__device__ __forceinline__ u32x4_t load_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}

// Buffer loads with a byte bound (raw buffer resource, no stride): a lane
// whose offset lies past the bound reads zeros and touches no memory. Kernels
// send masked lanes to kBufOob, past every bound used here, instead of
// clamping addresses or selecting after the load (a select right after a
// load makes the wavefront wait for it). AUX is the cache policy: kBufNt for
// streamed weights, 0 for data that other workgroups read again.
constexpr int kBufOob = 0x7FFFFFF0;
constexpr uint32_t kBufMaxRecords = 0x7FFFFF00u;
constexpr int kBufNt = 2;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* p, int64_t bytes) {
  const int64_t n =
      bytes <= 0 ? 0 : (bytes < (int64_t)kBufMaxRecords ? bytes : (int64_t)kBufMaxRecords);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)n, 0x00020000);
}
template <int AUX>
__device__ __forceinline__ u32x4_t buf_load16(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX));
}
template <int AUX>
__device__ __forceinline__ uint32_t buf_load4(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, AUX);
}

// ------------------------------------------------------------------ decode

// Two E2M1 codes (byte `sel` of `word`; low nibble -> .x) to bf16. The scale
// operand of v_cvt_scalef32_pk_bf16_fp4 only contributes its exponent, so it
// is always 1.0 here and block scales are applied to fp32 partial sums.
template <int SEL>
__device__ __forceinline__ bf16x2_t e2m1x2_to_bf16(uint32_t word) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, 1.0f, SEL);
}

template <int SEL>
__device__ __forceinline__ float2_t e2m1x2_to_f32(uint32_t word) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, SEL);
}

// UE4M3 scale byte `sel` of `word` to fp32 (v_cvt_f32_fp8 decodes the OCP
// E4M3FN format on gfx950; exact for every byte).
template <int SEL>
__device__ __forceinline__ float e4m3_to_f32(uint32_t word) {
  return __builtin_amdgcn_cvt_f32_fp8(word, SEL);
}

// bf16 dot of two pairs accumulated into fp32: a.x*b.x + a.y*b.y + c.
__device__ __forceinline__ float dot2(bf16x2_t a, bf16x2_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(a, b, c, false);
}

__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t u) {
  bf16x2_t r;
  __builtin_memcpy(&r, &u, 4);
  return r;
}

// ------------------------------------------------------------------ encode
// Round-to-nearest-even onto the E4M3 grid by integer manipulation of the
// fp32 bit pattern, saturating at 448 (0x7E). Non-positive and NaN inputs
// give 0x00 (a block scale is never negative).
__device__ __forceinline__ uint32_t e4m3_encode(float r) {
  if (!(r > 0.0f)) return 0u;
  if (r > 448.0f) return 0x7Eu;
  const uint32_t u = __float_as_uint(r);
  const int exp = (int)(u >> 23) - 127;   // unbiased exponent of r
  const uint32_t man = u & 0x7FFFFFu;
  if (exp < -6) {
    // E4M3 subnormal range: integer multiple of 2^-9. r = (2^23 + man) *
    // 2^(exp - 23), so r * 2^9 = (2^23 + man) >> (14 - exp) with RNE.
    if (exp < -10) return 0u;              // below 2^-10: rounds to zero
    const uint32_t sig = man | 0x800000u;  // exp >= -10: r is an fp32 normal
    const int sh = 14 - exp;               // 21 .. 24
    const uint32_t q = sig >> sh;
    const uint32_t rem = sig & ((1u << sh) - 1u);
    const uint32_t half = 1u << (sh - 1);
    return q + ((rem > half || (rem == half && (q & 1u))) ? 1u : 0u);
  }
  // normal range: keep 3 mantissa bits with RNE; a carry bumps the exponent
  const uint32_t keep = man >> 20;
  const uint32_t rem = man & 0xFFFFFu;
  const uint32_t up = (rem > 0x80000u || (rem == 0x80000u && (keep & 1u))) ? 1u : 0u;
  const uint32_t code = ((uint32_t)(exp + 7) << 3) + keep + up;
  return code > 0x7Eu ? 0x7Eu : code;
}

// E2M1 code of t by comparison with the decision points between adjacent
// magnitudes (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5); a point exactly on a
// boundary goes to the neighbour with the even code. Magnitudes above 5 give
// 6 (saturating). A negative t whose magnitude rounds to 0 gives +0.
__device__ __forceinline__ uint32_t e2m1_encode(float t) {
  const float a = fabsf(t);
  uint32_t mag;
  if (a <= 0.25f) mag = 0u;
  else if (a < 0.75f) mag = 1u;
  else if (a <= 1.25f) mag = 2u;
  else if (a < 1.75f) mag = 3u;
  else if (a <= 2.5f) mag = 4u;
  else if (a < 3.5f) mag = 5u;
  else if (a <= 5.0f) mag = 6u;
  else mag = 7u;
  return (t < 0.0f && mag != 0u) ? (mag | 8u) : mag;
}

// One 16-element block with tensor scale g: s = E4M3(amax / (6 g)), then
// codes E2M1(w / (s g)) (all-zero codes when s is 0). Returns the scale byte;
// lo holds elements 0..7 and hi elements 8..15, element i in nibble i % 8.
__device__ __forceinline__ uint32_t encode_block16(const float (&w)[16], float g,
                                                   uint32_t& lo, uint32_t& hi) {
  float ab = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) ab = fmaxf(ab, fabsf(w[i]));
  const float d6 = 6.0f * g;
  const float r = ab / d6;
  const uint32_t sc = e4m3_encode(r);
  const float s = e4m3_to_f32<0>(sc);
  lo = 0u;
  hi = 0u;
  if (s != 0.0f) {
    const float dn = s * g;
#pragma unroll
    for (int i = 0; i < 8; ++i) lo |= e2m1_encode(w[i] / dn) << (4 * i);
#pragma unroll
    for (int i = 0; i < 8; ++i) hi |= e2m1_encode(w[8 + i] / dn) << (4 * i);
  }
  return sc;
}

// --------------------------------------------------------------- reductions

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

// Sum over the 64 lanes of a wavefront; every lane receives the total. All
// 64 lanes must be active. Within each 16-lane row the partial sums travel
// by DPP (quad permutations [1,0,3,2] and [2,3,0,1], then the half-row and
// row mirrors), so each lane ends with its row's sum; the four row sums are
// then read out with v_readlane and added in a fixed order. No LDS traffic,
// and the same result on every lane.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f32<0xB1>(v);    // quad_perm [1,0,3,2]
  v += dpp_f32<0x4E>(v);    // quad_perm [2,3,0,1]
  v += dpp_f32<0x141>(v);   // row_half_mirror
  v += dpp_f32<0x140>(v);   // row_mirror
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return (r0 + r1) + (r2 + r3);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    uint32_t o = __shfl_xor(v, off, 64);
    v = o > v ? o : v;
  }
  return v;
}

}  // namespace nvfp4
