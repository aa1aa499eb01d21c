// moe.hip -- NVFP4 g16 W4A16 MoE expert slots on gfx950.
//
// The pages' MoE decode path (graph.json nodes "l3.moe.experts_gate_up",
// "l3.moe.experts_act", "l3.moe.experts_down", "l3.moe.blend"; card.json
// performance[31] row union, performance[33] W4A16 slot GEMV, performance[64]
// union sweep) becomes four launches, all on the caller's stream and with no
// host synchronisation:
//   1. k_moe_union:   distinct valid expert ids of the batch (the "row union").
//   2. k_moe_gate_up: per distinct expert, stream its gate|up rows once, dot
//                     them with x of every slot routed to it, and write
//                     h = bf16(silu(gate) * up) per slot (SwiGLU fused).
//   3. k_moe_down:    per distinct expert, stream its down rows once and write
//                     the fp32 output of every slot routed to it.
//   4. k_moe_combine: y[m] = sum_j gate_w[m, j] * o[m, j] in slot order.
// Steps 2 and 3 launch one grid row per possible distinct expert (M * topk);
// rows past the device-side count exit at once.
#include "gemv_core.h"
#include "internal.h"

namespace nvfp4 {

constexpr int kMaxSlots = NVFP4_MAX_M_INTERNAL * NVFP4_MAX_TOPK_INTERNAL;  // 128
constexpr int kSlotPass = 8;   // slots of one expert handled per pass
constexpr int kMoeWaves = 4;

static inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

MoeLayout moe_layout(int64_t M, int64_t H, int64_t I, int64_t topk) {
  MoeLayout L;
  const size_t S = (size_t)(M * topk);
  L.union_off = 0;
  L.h_off = align256(L.union_off + (S + 1) * sizeof(int32_t));
  L.o_off = align256(L.h_off + S * (size_t)I * sizeof(uint16_t));
  L.total = align256(L.o_off + S * (size_t)H * sizeof(float));
  return L;
}

// One workgroup of kMaxSlots threads. uni[0] = number of distinct valid ids,
// uni[1 + u] = the u-th distinct id in order of first appearance.
__global__ __launch_bounds__(kMaxSlots) void k_moe_union(const int32_t* __restrict__ ids,
                                                         int S, int64_t E,
                                                         int32_t* __restrict__ uni) {
  __shared__ int32_t sid[kMaxSlots];
  __shared__ int32_t first[kMaxSlots];
  const int i = threadIdx.x;
  const int32_t id = (i < S) ? ids[i] : -1;
  sid[i] = id;
  __syncthreads();
  bool f = (i < S) && id >= 0 && (int64_t)id < E;
  for (int j = 0; j < i && f; ++j)
    if (sid[j] == id) f = false;
  first[i] = f ? 1 : 0;
  __syncthreads();
  if (f) {
    int rank = 0;
    for (int j = 0; j < i; ++j) rank += first[j];
    uni[1 + rank] = id;
  }
  if (i == 0) {
    int cnt = 0;
    for (int j = 0; j < S; ++j) cnt += first[j];
    uni[0] = cnt;
  }
}

// Slots (in increasing order) whose id equals e, from position `start` on;
// returns how many were written to slot[] (at most kSlotPass) and the next
// start position. Uniform across the wavefront.
__device__ __forceinline__ int next_slots(const int32_t* __restrict__ ids, int S, int32_t e,
                                          int& start, int (&slot)[kSlotPass]) {
  int n = 0;
  while (start < S && n < kSlotPass) {
    if (ids[start] == e) slot[n++] = start;
    ++start;
  }
  return n;
}

__device__ __forceinline__ uint16_t bf16_rne(float v) {
  const uint32_t u = __float_as_uint(v);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);  // NaN
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// gate|up sweep: grid (M*topk, Y). A wavefront takes 2 consecutive outputs
// r, r+1 and streams the 4 weight rows r, r+1 (gate) and I+r, I+r+1 (up).
__global__ __launch_bounds__(256) void k_moe_gate_up(
    const uint8_t* __restrict__ w13_codes, const uint8_t* __restrict__ w13_scales,
    const float* __restrict__ w13_gscale, const uint16_t* __restrict__ x,
    const int32_t* __restrict__ ids, const int32_t* __restrict__ uni, int S, int topk,
    int64_t H, int64_t I, uint16_t* __restrict__ h) {
  const int u = blockIdx.x;
  if (u >= uni[0]) return;
  const int32_t e = uni[1 + u];
  const int lane = threadIdx.x & 63;
  const uint8_t* codes = w13_codes + (int64_t)e * (2 * I) * (H / 2);
  const uint8_t* scales = w13_scales + (int64_t)e * (2 * I) * (H / 16);
  const float g = w13_gscale[e];
  const int64_t wave =
      (int64_t)blockIdx.y * kMoeWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.y * kMoeWaves;

  int start = 0;
  int slot[kSlotPass];
  int ns;
  while ((ns = next_slots(ids, S, e, start, slot)) > 0) {
    const uint16_t* xs[kSlotPass];
#pragma unroll
    for (int m = 0; m < kSlotPass; ++m) xs[m] = x + (int64_t)(slot[m < ns ? m : 0] / topk) * H;
    for (int64_t r0 = wave * 2; r0 < I; r0 += nwaves * 2) {
      const int64_t r1 = (r0 + 1 < I) ? r0 + 1 : r0;
      const int64_t rows[4] = {r0, r1, I + r0, I + r1};
      float acc[4][kSlotPass];
      wave_row_dots<kSlotPass, 4>(codes, scales, H, rows, xs, ns, acc);
#pragma unroll
      for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int m = 0; m < kSlotPass; ++m)
          if (lane == p * kSlotPass + m && m < ns && r0 + p < I) {
            const float G = g * acc[p][m], U = g * acc[2 + p][m];
            const float act = G / (1.0f + expf(-G)) * U;
            h[(int64_t)slot[m] * I + r0 + p] = bf16_rne(act);
          }
    }
  }
}

// down sweep: grid (M*topk, Y). A wavefront takes 4 consecutive output rows.
__global__ __launch_bounds__(256) void k_moe_down(
    const uint8_t* __restrict__ w2_codes, const uint8_t* __restrict__ w2_scales,
    const float* __restrict__ w2_gscale, const uint16_t* __restrict__ h,
    const int32_t* __restrict__ ids, const int32_t* __restrict__ uni, int S, int64_t H,
    int64_t I, float* __restrict__ o) {
  const int u = blockIdx.x;
  if (u >= uni[0]) return;
  const int32_t e = uni[1 + u];
  const int lane = threadIdx.x & 63;
  const uint8_t* codes = w2_codes + (int64_t)e * H * (I / 2);
  const uint8_t* scales = w2_scales + (int64_t)e * H * (I / 16);
  const float g = w2_gscale[e];
  const int64_t wave =
      (int64_t)blockIdx.y * kMoeWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.y * kMoeWaves;

  int start = 0;
  int slot[kSlotPass];
  int ns;
  while ((ns = next_slots(ids, S, e, start, slot)) > 0) {
    const uint16_t* xs[kSlotPass];
#pragma unroll
    for (int m = 0; m < kSlotPass; ++m) xs[m] = h + (int64_t)slot[m < ns ? m : 0] * I;
    for (int64_t n0 = wave * 4; n0 < H; n0 += nwaves * 4) {
      int64_t rows[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) rows[r] = (n0 + r < H) ? n0 + r : H - 1;
      float acc[4][kSlotPass];
      wave_row_dots<kSlotPass, 4>(codes, scales, I, rows, xs, ns, acc);
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int m = 0; m < kSlotPass; ++m)
          if (lane == r * kSlotPass + m && m < ns && n0 + r < H)
            o[(int64_t)slot[m] * H + n0 + r] = g * acc[r][m];
    }
  }
}

// y[m, n] = sum_j gate_w[m, j] * o[m*topk + j, n] over valid slots, j in order.
__global__ __launch_bounds__(256) void k_moe_combine(const float* __restrict__ o,
                                                     const int32_t* __restrict__ ids,
                                                     const float* __restrict__ gate_w,
                                                     int M, int topk, int64_t E, int64_t H,
                                                     float* __restrict__ y) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)M * H) return;
  const int64_t m = i / H, n = i - m * H;
  float acc = 0.0f;
  for (int j = 0; j < topk; ++j) {
    const int32_t e = ids[m * topk + j];
    if (e >= 0 && (int64_t)e < E)
      acc = __builtin_fmaf(gate_w[m * topk + j], o[(m * topk + j) * H + n], acc);
  }
  y[i] = acc;
}

hipError_t launch_moe(const uint8_t* w13_codes, const uint8_t* w13_scales,
                      const float* w13_gscale, const uint8_t* w2_codes,
                      const uint8_t* w2_scales, const float* w2_gscale, const uint16_t* x,
                      const int32_t* ids, const float* gate_w, int M, int64_t E, int64_t H,
                      int64_t I, int topk, float* y, void* workspace, hipStream_t stream) {
  const MoeLayout L = moe_layout(M, H, I, topk);
  char* ws = static_cast<char*>(workspace);
  int32_t* uni = reinterpret_cast<int32_t*>(ws + L.union_off);
  uint16_t* h = reinterpret_cast<uint16_t*>(ws + L.h_off);
  float* o = reinterpret_cast<float*>(ws + L.o_off);
  const int S = M * topk;
  hipLaunchKernelGGL(k_moe_union, dim3(1), dim3(kMaxSlots), 0, stream, ids, S, E, uni);
  // gate|up: one wavefront per 2 outputs, up to 64 workgroups per expert
  {
    const int64_t groups = (I + 1) / 2;
    int64_t yb = (groups + kMoeWaves - 1) / kMoeWaves;
    if (yb > 64) yb = 64;
    hipLaunchKernelGGL(k_moe_gate_up, dim3(S, (unsigned)yb), dim3(256), 0, stream, w13_codes,
                       w13_scales, w13_gscale, x, ids, uni, S, topk, H, I, h);
  }
  {
    const int64_t groups = (H + 3) / 4;
    int64_t yb = (groups + kMoeWaves - 1) / kMoeWaves;
    if (yb > 64) yb = 64;
    hipLaunchKernelGGL(k_moe_down, dim3(S, (unsigned)yb), dim3(256), 0, stream, w2_codes,
                       w2_scales, w2_gscale, h, ids, uni, S, H, I, o);
  }
  {
    const int64_t n = (int64_t)M * H;
    hipLaunchKernelGGL(k_moe_combine, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                       o, ids, gate_w, M, topk, E, H, y);
  }
  return hipGetLastError();
}

}  // namespace nvfp4
