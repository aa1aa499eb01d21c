// moe.hip -- NVFP4 g16 MoE expert slots on gfx950.
//
// The pages' MoE decode path (graph.json nodes "l3.moe.experts_gate_up",
// "l3.moe.experts_act", "l3.moe.experts_down", "l3.moe.blend"; card.json
// performance[31] row union, performance[33] W4A16 slot GEMV, performance[64]
// union sweep) runs as two launches on the caller's stream, with no host
// synchronisation and no atomics:
//   1. k_moe_gate_up: grid (row block, slot j). The workgroup of the first
//      slot that names an expert streams that expert's gate|up rows once and
//      dots them with x of every slot routed to it (the row union, found with
//      wavefront ballots over the ids); it writes h = bf16(silu(gate) * up)
//      per slot. Workgroups of later slots with the same id, and of invalid
//      ids, exit at once.
//   2. The down projection and the gate-weighted combine in one pass. For
//      output row n and token m,
//        y[m, n] = sum_j gate_w[m, j] * g2[e_j] * W2[e_j][n, :] . h_j
//      is one dot product over the token's valid slots laid end to end (a
//      K axis of (valid slots) x I), walked in (slot, 32-element chunk)
//      pairs with all 64 lanes busy whatever I is. At M = 1 a wavefront owns
//      R output rows (k_moe_down); at M >= 2 the pairs of all tokens are
//      split over the wavefronts of a workgroup (k_moe_down_split). Sums run
//      in a fixed order: deterministic, no per-slot output buffer, no
//      separate combine launch.
// An optional shared expert (graph.json nodes "l3.moe.shared_gate_up",
// "l3.moe.shared_act", "l3.moe.shared_down"; "l3.moe.blend" takes the routed
// slots and the shared output) rides in the same two launches: one more
// gate|up grid row streams its rows once for all M tokens, and each token's
// down dot product runs on over the shared expert's chunks after its routed
// slots, with coefficient g2s (gate weight 1).
// W4A4 routed experts (card.json performance[64], [65]) use the same kernels
// on activations put on the NVFP4 grid by k_quantize_decode (w4a4.hip), with
// the static scales folded into the weight scale and the combine weight. At
// M = 1, k_moe_gate_up_w4a4_1 takes the place of gate|up and of h's
// quantization pass.
#include "gemv_core.h"
#include "internal.h"
#include "quant.h"

namespace nvfp4 {

constexpr int kMoeWaves = 4;     // wavefronts per workgroup
constexpr int kDownRows = 2;     // output rows per wavefront in the down pass
constexpr int kDownUnroll = 2;   // (slot, chunk) pairs in flight per lane
constexpr int kGateUpSlots = 2;  // slots per pass over an expert's gate|up rows, M >= 2
// wavefronts that six per SIMD hold at once on the 256 CUs of an MI355X
constexpr int64_t kOneRoundWaves6 = 6 * 4 * 256;

static inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

MoeLayout moe_layout(int64_t M, int64_t H, int64_t I, int64_t topk, int64_t Is, bool w4a4) {
  MoeLayout L;
  const size_t hbytes = (size_t)(M * topk) * (size_t)I * sizeof(uint16_t);
  L.h_off = 0;
  L.hs_off = align256(hbytes);
  L.hq_off = align256(L.hs_off + (size_t)M * (size_t)Is * sizeof(uint16_t));
  L.xq_off = L.hq_off;
  L.total = L.hq_off;
  if (w4a4) {
    L.xq_off = align256(L.hq_off + hbytes);
    L.total = align256(L.xq_off + (size_t)M * (size_t)H * sizeof(uint16_t));
  }
  return L;
}

__device__ __forceinline__ uint16_t bf16_rne(float v) {
  const uint32_t u = __float_as_uint(v);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);  // NaN
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// One wavefront: gate rows r0, r0+1 and up rows I+r0, I+r0+1 of one expert
// against x of up to MS slots; writes h[slot, r0 .. r0+1].
// The token of slot s is s / xdiv (topk for routed slots, 1 for the shared
// expert, whose slots are the tokens).
template <int MS>
__device__ __forceinline__ void gate_up_rows(const uint8_t* __restrict__ codes,
                                             const uint8_t* __restrict__ scales, float g,
                                             const uint16_t* __restrict__ x, int64_t H,
                                             int64_t I, int64_t r0, int xdiv,
                                             const int (&slot)[MS], int ns,
                                             uint16_t* __restrict__ h) {
  const int lane = threadIdx.x & 63;
  const int64_t r1 = (r0 + 1 < I) ? r0 + 1 : r0;
  const int64_t rows[4] = {r0, r1, I + r0, I + r1};
  const uint16_t* xs[MS];
#pragma unroll
  for (int m = 0; m < MS; ++m) xs[m] = x + (int64_t)(slot[m] / xdiv) * H;
  float acc[4][MS];
  wave_row_dots<MS, 4>(codes, scales, H, rows, xs, ns, acc);
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int m = 0; m < MS; ++m)
      if (lane == p * MS + m && m < ns && r0 + p < I) {
        const float G = g * acc[p][m], U = g * acc[2 + p][m];
        const float act = G / (1.0f + expf(-G)) * U;
        h[(int64_t)slot[m] * I + r0 + p] = bf16_rne(act);
      }
}

// grid (ceil(ceil(max(I, Is)/2) / kMoeWaves), S [+ 1 for the shared expert, row 0]);
// a wavefront owns one gate/up row pair. Row blocks are the fast grid axis:
// workgroups are dealt to the 8 XCDs round robin in linear order, so each
// expert's rows spread over all XCDs (with the slot as the fast axis, every
// row block of a slot's expert landed on the XCD of slot mod 8).
// Routed slots read xr with weight scale w13_gscale[e] * *ga (xr = x and
// ga = NULL for W4A16; the W4A4 activations on the NVFP4 grid and their
// static scale otherwise); the shared expert always reads x.
// The shared expert and a routed expert take the same path once their
// weights, activation rows and slot set are chosen, so the dot-product engine
// is inlined once per slot-group width: MSX slots per pass over the rows
// (one pass per slot at MSX = 1, which the launcher uses at M = 1; it keeps
// the kernel at the register count of one slot and so at 6 wavefronts per
// SIMD, against 3 when a 4-slot group and a separate shared-expert path were
// inlined side by side).
// W7 caps the registers for seven wavefronts per SIMD. The launcher takes it
// at M = 1 when the grid holds more wavefronts than six per SIMD run in one
// round (the 768-wide shared expert's grid row makes 6912 for 6144 places):
// with the shared expert, 25.7 -> 24.2 us; without it (exactly one round at
// six) the uncapped kernel stays faster, 21.5 against 21.9 us.
template <int MSX, bool W7>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(W7 ? 7 : 1))) void k_moe_gate_up(
    const uint8_t* __restrict__ w13_codes, const uint8_t* __restrict__ w13_scales,
    const float* __restrict__ w13_gscale, const uint16_t* __restrict__ x,
    const uint16_t* __restrict__ xr, const float* __restrict__ ga,
    const int32_t* __restrict__ ids, int S, int topk, int64_t E, int64_t H, int64_t I,
    uint16_t* __restrict__ h, const MoeShared sh, int M) {
  // the shared expert (when there is one) is grid row 0, so that its
  // workgroups, which serve every token, start first
  const bool shared_row = sh.I > 0 && blockIdx.y == 0;
  const int j = sh.I > 0 ? (int)blockIdx.y - 1 : (int)blockIdx.y;   // routed slot
  const int lane = threadIdx.x & 63;
  const int64_t pair =
      (int64_t)blockIdx.x * kMoeWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t r0 = pair * 2;
  const uint8_t* codes;
  const uint8_t* scales;
  const uint16_t* xs;   // activation rows; slot s reads row s / xdiv
  uint16_t* hd;         // h rows; slot s writes row s
  float g;
  int64_t Iv;
  int xdiv;
  uint64_t m0, m1;      // the slots to serve: bit s of m0, bit s - 64 of m1
  if (shared_row) {
    // the shared expert: its rows once, for all M tokens (its slots)
    if (r0 >= sh.I) return;
    codes = sh.c13;
    scales = sh.s13;
    g = *sh.g13;
    xs = x;
    hd = sh.h;
    Iv = sh.I;
    xdiv = 1;
    m0 = (M >= 64) ? ~0ull : ((1ull << M) - 1ull);
    m1 = 0;
  } else {
    if (r0 >= I) return;
    const int32_t e = ids[j];
    if (e < 0 || (int64_t)e >= E) return;
    if constexpr (MSX == 1) {
      // one token (M = 1): each slot streams its own expert's rows. A
      // token's top-k names distinct experts; a repeated id is streamed once
      // per slot, which is still correct.
      m0 = 1ull << (j & 63);
      m1 = 0;
    } else {
      // lane l looks at slots l and l + 64 (S <= 128)
      const int32_t a = lane < S ? ids[lane] : -1;
      const int32_t b = lane + 64 < S ? ids[lane + 64] : -1;
      const uint64_t earlier =
          __ballot(a == e && lane < j) | __ballot(b == e && lane + 64 < j);
      if (earlier) return;   // the workgroup of an earlier slot streams this expert
      m0 = __ballot(a == e);   // all >= j, j included
      m1 = __ballot(b == e);
    }
    codes = w13_codes + (int64_t)e * (2 * I) * (H / 2);
    scales = w13_scales + (int64_t)e * (2 * I) * (H / 16);
    g = ga ? w13_gscale[e] * *ga : w13_gscale[e];
    xs = xr;
    hd = h;
    Iv = I;
    xdiv = topk;
  }
  if (MSX == 1 || __popcll(m0) + __popcll(m1) == 1) {   // one slot
    const int slot[1] = {MSX == 1 ? (shared_row ? 0 : j)
                                  : (m0 ? __builtin_ctzll(m0) : 64 + __builtin_ctzll(m1))};
    gate_up_rows<1>(codes, scales, g, xs, H, Iv, r0, xdiv, slot, 1, hd);
    return;
  }
  while (m0 | m1) {
    int slot[MSX];
    int ns = 0;
#pragma unroll
    for (int q = 0; q < MSX; ++q) {
      if (m0) {
        slot[q] = __builtin_ctzll(m0);
        m0 &= m0 - 1;
        ++ns;
      } else if (m1) {
        slot[q] = 64 + __builtin_ctzll(m1);
        m1 &= m1 - 1;
        ++ns;
      } else {
        slot[q] = slot[0];   // unused column (q >= ns): any served slot
      }
    }
    gate_up_rows<MSX>(codes, scales, g, xs, H, Iv, r0, xdiv, slot, ns, hd);
  }
}

// Gate|up pieces for H = 2048 CL, launched for H = 4096 (CL = 2: more
// chunks per lane would spill, and one chunk per lane was slower in the
// dense GEMV's version of this staging). They compute the rows of
// wave_row_dots<1, 4> in the same per-lane order of (chunk, block)
// products, so the same h bit for bit, with two changes to the memory side:
//  - the activation row is staged once per workgroup in LDS (8 KB at H =
//    4096, x1x_unit layout of gemv_core.h) instead of every wavefront
//    reading all of it through the L1;
//  - each lane issues the loads of all CL of its chunks before the first
//    product, so a wavefront waits for one HBM round trip, not CL.

// the codes and scales of rows[0..3] at the lane's CL chunks
template <int CL>
__device__ __forceinline__ void gate_up_loads_1x(const uint8_t* __restrict__ codes,
                                                 const uint8_t* __restrict__ scales, int64_t H,
                                                 const int64_t (&rows)[4], u32x4_t (&q)[CL][4],
                                                 uint32_t (&sw)[CL][4]) {
  const int lane = threadIdx.x & 63;
  const int64_t cb = H >> 1, sbytes = H >> 4;
#pragma unroll
  for (int cl = 0; cl < CL; ++cl)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t c = lane + 64 * cl;
      q[cl][r] = load_stream(codes + rows[r] * cb + c * 16);
      sw[cl][r] = *reinterpret_cast<const uint16_t*>(scales + rows[r] * sbytes + c * 2);
    }
}

// acc[r] = the wavefront's dot of row r with the staged x (every lane)
template <int CL>
__device__ __forceinline__ void gate_up_dots_1x(const u32x4_t (&q)[CL][4],
                                                const uint32_t (&sw)[CL][4],
                                                const u32x4_t* xl, float (&acc)[4]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int r = 0; r < 4; ++r) acc[r] = 0.0f;
#pragma unroll
  for (int cl = 0; cl < CL; ++cl) {
    const int c = lane + 64 * cl;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const u32x4_t xa = xl[x1x_unit(4 * c + 2 * b)];
      const u32x4_t xb = xl[x1x_unit(4 * c + 2 * b + 1)];
      const bf16x2_t xq[8] = {as_bf16x2(xa.x), as_bf16x2(xa.y), as_bf16x2(xa.z),
                              as_bf16x2(xa.w), as_bf16x2(xb.x), as_bf16x2(xb.y),
                              as_bf16x2(xb.z), as_bf16x2(xb.w)};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t w0 = b ? q[cl][r].z : q[cl][r].x;
        const uint32_t w1 = b ? q[cl][r].w : q[cl][r].y;
        const bf16x2_t wd[8] = {e2m1x2_to_bf16<0>(w0), e2m1x2_to_bf16<1>(w0),
                                e2m1x2_to_bf16<2>(w0), e2m1x2_to_bf16<3>(w0),
                                e2m1x2_to_bf16<0>(w1), e2m1x2_to_bf16<1>(w1),
                                e2m1x2_to_bf16<2>(w1), e2m1x2_to_bf16<3>(w1)};
        const float sc = b ? e4m3_to_f32<1>(sw[cl][r]) : e4m3_to_f32<0>(sw[cl][r]);
        float p = 0.0f;
#pragma unroll
        for (int t = 0; t < 8; ++t) p = dot2(wd[t], xq[t], p);
        acc[r] = __builtin_fmaf(p, sc, acc[r]);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) acc[r] = wave_sum(acc[r]);
}

// Gate|up at one token (M = 1) with the pieces above: every slot multiplies
// the same activation row, which each workgroup stages once. Grid and
// outputs as k_moe_gate_up<1, W7>, dynamic LDS 2 H bytes; same-process A/B
// (288 experts, top-8, with the one-token down pass below): routed 21.4 ->
// 20.0 us, with the shared expert 24.1 -> 21.1 us.
template <int CL, bool W7>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(W7 ? 7 : 6))) void k_moe_gate_up_1x(
    const uint8_t* __restrict__ w13_codes, const uint8_t* __restrict__ w13_scales,
    const float* __restrict__ w13_gscale, const uint16_t* __restrict__ x,
    const uint16_t* __restrict__ xr, const float* __restrict__ ga,
    const int32_t* __restrict__ ids, int64_t E, int64_t H, int64_t I,
    uint16_t* __restrict__ h, const MoeShared sh) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  u32x4_t* const xl = reinterpret_cast<u32x4_t*>(lds);
  const bool shared_row = sh.I > 0 && blockIdx.y == 0;
  const int j = sh.I > 0 ? (int)blockIdx.y - 1 : (int)blockIdx.y;   // routed slot
  const int lane = threadIdx.x & 63;
  const int64_t r0 =
      ((int64_t)blockIdx.x * kMoeWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6)) * 2;
  int32_t e = 0;
  bool ok = true;
  const uint8_t* codes = sh.c13;
  const uint8_t* scales = sh.s13;
  const uint16_t* xs = x;
  uint16_t* hd = sh.h;
  int64_t Iv = sh.I;
  if (!shared_row) {
    e = ids[j];
    ok = e >= 0 && (int64_t)e < E;
    codes = w13_codes + (int64_t)(ok ? e : 0) * (2 * I) * (H / 2);
    scales = w13_scales + (int64_t)(ok ? e : 0) * (2 * I) * (H / 16);
    xs = xr;
    hd = h + (int64_t)j * I;
    Iv = I;
  }
  const bool act = ok && r0 < Iv;   // the whole wavefront
  u32x4_t xv[CL];
  x1x_load<256, CL>(xs, (int)(H >> 3), xv);
  const int64_t r1 = (r0 + 1 < Iv) ? r0 + 1 : r0;
  const int64_t rows[4] = {r0, r1, Iv + r0, Iv + r1};
  u32x4_t q[CL][4];
  uint32_t sw[CL][4];
  if (act) gate_up_loads_1x<CL>(codes, scales, H, rows, q, sw);
  x1x_store<256, CL>(xl, (int)(H >> 3), xv);
  __syncthreads();
  if (!act) return;
  float acc[4];
  gate_up_dots_1x<CL>(q, sw, xl, acc);
  const float g = shared_row ? *sh.g13 : (ga ? w13_gscale[e] * *ga : w13_gscale[e]);
#pragma unroll
  for (int p = 0; p < 2; ++p)
    if (lane == p && r0 + p < Iv) {
      const float G = g * acc[p], U = g * acc[2 + p];
      const float a = G / (1.0f + expf(-G)) * U;
      hd[r0 + p] = bf16_rne(a);
    }
}

// Two or more tokens, H = 4096 (CL = 2 chunks per lane): the slot groups
// of k_moe_gate_up<MSX> (two slots per pass, in slot order) and its
// per-lane order of products, so the same h bit for bit, with the memory
// side of k_moe_gate_up_1x: a wavefront loads the codes
// and scales of its rows once, before its first pass (k_moe_gate_up<MSX>
// streams them again for every pass), and each pass's two activation rows
// are staged once per workgroup in LDS (x1x_unit layout, one row per half)
// instead of every wavefront reading them through the L1. Every wavefront
// of a workgroup serves the same slot, so all take the same passes and
// barriers. A pass with one slot stages its row twice and computes both
// halves (skipping the second measured slower: more registers). 288
// experts, top-8, M = 8, same-process A/B: uniform routing 114.7 -> 115.0
// us, one expert named by all tokens 113.2 -> 111.2 us, all tokens on the
// same 8 experts 102.0 -> 74.5 us (their weights are read once, not once
// per pass).
template <int CL>
__global__ __launch_bounds__(256) void k_moe_gate_up_mx(
    const uint8_t* __restrict__ w13_codes, const uint8_t* __restrict__ w13_scales,
    const float* __restrict__ w13_gscale, const uint16_t* __restrict__ x,
    const uint16_t* __restrict__ xr, const float* __restrict__ ga,
    const int32_t* __restrict__ ids, int S, int topk, int64_t E, int64_t H, int64_t I,
    uint16_t* __restrict__ h, const MoeShared sh, int M) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  u32x4_t* const xl = reinterpret_cast<u32x4_t*>(lds);
  const bool shared_row = sh.I > 0 && blockIdx.y == 0;
  const int j = sh.I > 0 ? (int)blockIdx.y - 1 : (int)blockIdx.y;   // routed slot
  const int lane = threadIdx.x & 63;
  const int64_t r0 =
      ((int64_t)blockIdx.x * kMoeWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6)) * 2;
  const uint8_t* codes;
  const uint8_t* scales;
  const uint16_t* xs;
  uint16_t* hd;
  float g;
  int64_t Iv;
  int xdiv;
  uint64_t m0, m1;
  if (shared_row) {
    codes = sh.c13;
    scales = sh.s13;
    g = *sh.g13;
    xs = x;
    hd = sh.h;
    Iv = sh.I;
    xdiv = 1;
    m0 = (M >= 64) ? ~0ull : ((1ull << M) - 1ull);
    m1 = 0;
  } else {
    const int32_t e = ids[j];
    if (e < 0 || (int64_t)e >= E) return;   // the whole workgroup
    const int32_t a = lane < S ? ids[lane] : -1;
    const int32_t b = lane + 64 < S ? ids[lane + 64] : -1;
    const uint64_t earlier =
        __ballot(a == e && lane < j) | __ballot(b == e && lane + 64 < j);
    if (earlier) return;   // the whole workgroup: an earlier slot streams this expert
    m0 = __ballot(a == e);
    m1 = __ballot(b == e);
    codes = w13_codes + (int64_t)e * (2 * I) * (H / 2);
    scales = w13_scales + (int64_t)e * (2 * I) * (H / 16);
    g = ga ? w13_gscale[e] * *ga : w13_gscale[e];
    xs = xr;
    hd = h;
    Iv = I;
    xdiv = topk;
  }
  const bool act = r0 < Iv;   // the whole wavefront
  const int64_t r1 = (r0 + 1 < Iv) ? r0 + 1 : r0;
  const int64_t rows[4] = {r0, r1, Iv + r0, Iv + r1};
  u32x4_t q[CL][4];
  uint32_t sw[CL][4];
  if (act) gate_up_loads_1x<CL>(codes, scales, H, rows, q, sw);
  constexpr int nu = 256 * CL;   // units per activation row (H = 2048 CL)
  while (m0 | m1) {
    int slot[2];
    int ns = 0;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if (m0) {
        slot[t] = __builtin_ctzll(m0);
        m0 &= m0 - 1;
        ++ns;
      } else if (m1) {
        slot[t] = 64 + __builtin_ctzll(m1);
        m1 &= m1 - 1;
        ++ns;
      } else {
        slot[t] = slot[0];
      }
    }
    // the two activation rows into LDS (a lone slot's row twice)
    u32x4_t xv[2 * CL];
    const u32x4_t* const xrow[2] = {
        reinterpret_cast<const u32x4_t*>(xs + (int64_t)(slot[0] / xdiv) * H),
        reinterpret_cast<const u32x4_t*>(xs + (int64_t)(slot[1] / xdiv) * H)};
#pragma unroll
    for (int k = 0; k < 2 * CL; ++k) {
      const int t = k / CL;   // 256 threads, nu = 256 CL units per row
      xv[k] = xrow[t][(int)threadIdx.x + 256 * (k - t * CL)];
    }
#pragma unroll
    for (int k = 0; k < 2 * CL; ++k) {
      const int t = k / CL;
      xl[t * nu + x1x_unit((int)threadIdx.x + 256 * (k - t * CL))] = xv[k];
    }
    __syncthreads();
    if (act) {
      float acc[4][2];
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r][0] = acc[r][1] = 0.0f;
#pragma unroll
      for (int cl = 0; cl < CL; ++cl) {
        const int c = lane + 64 * cl;
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          // one (chunk, block) step at a time: without the fence the
          // scheduler hoists later steps' LDS reads and decodes (125 VGPRs,
          // four wavefronts per SIMD instead of five; M = 8 uniform routing
          // 120.1 -> 125.8 us)
          __builtin_amdgcn_sched_barrier(0);
          bf16x2_t xq[2][8];
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const u32x4_t xa = xl[t * nu + x1x_unit(4 * c + 2 * b)];
            const u32x4_t xb = xl[t * nu + x1x_unit(4 * c + 2 * b + 1)];
            xq[t][0] = as_bf16x2(xa.x); xq[t][1] = as_bf16x2(xa.y);
            xq[t][2] = as_bf16x2(xa.z); xq[t][3] = as_bf16x2(xa.w);
            xq[t][4] = as_bf16x2(xb.x); xq[t][5] = as_bf16x2(xb.y);
            xq[t][6] = as_bf16x2(xb.z); xq[t][7] = as_bf16x2(xb.w);
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const uint32_t w0 = b ? q[cl][r].z : q[cl][r].x;
            const uint32_t w1 = b ? q[cl][r].w : q[cl][r].y;
            const bf16x2_t wd[8] = {e2m1x2_to_bf16<0>(w0), e2m1x2_to_bf16<1>(w0),
                                    e2m1x2_to_bf16<2>(w0), e2m1x2_to_bf16<3>(w0),
                                    e2m1x2_to_bf16<0>(w1), e2m1x2_to_bf16<1>(w1),
                                    e2m1x2_to_bf16<2>(w1), e2m1x2_to_bf16<3>(w1)};
            const float sc = b ? e4m3_to_f32<1>(sw[cl][r]) : e4m3_to_f32<0>(sw[cl][r]);
#pragma unroll
            for (int t = 0; t < 2; ++t) {
              float p = 0.0f;
#pragma unroll
              for (int z = 0; z < 8; ++z) p = dot2(wd[z], xq[t][z], p);
              acc[r][t] = __builtin_fmaf(p, sc, acc[r][t]);
            }
          }
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        acc[r][0] = wave_sum(acc[r][0]);
        acc[r][1] = wave_sum(acc[r][1]);
      }
#pragma unroll
      for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int t = 0; t < 2; ++t)
          if (lane == p * 2 + t && t < ns && r0 + p < Iv) {
            const float G = g * acc[p][t], U = g * acc[2 + p][t];
            const float a = G / (1.0f + expf(-G)) * U;
            hd[(int64_t)slot[t] * Iv + r0 + p] = bf16_rne(a);
          }
    }
    __syncthreads();   // every wavefront has read this pass's rows
  }
}

constexpr int kW4Waves = 8;   // k_moe_gate_up_w4a4_1: 16 gate|up rows per workgroup

// W4A4 at M = 1: gate|up with the quantization of h folded in (three
// launches per call instead of four). grid (ceil(max(I, Is) / 16), topk
// [+ 1 for the shared expert, row 0]), kW4Waves wavefronts of one row pair
// each, so a workgroup holds 16 consecutive rows of one slot's h -- exactly
// one 16-block, as I is a multiple of 32.
//   - A routed workgroup streams its 16 rows against x on the NVFP4 grid of
//     *ga13 (xq, from k_quantize_decode) with weight scale g13[e] * *ga13,
//     writes their h, and puts the 16 values on the grid of *ga2 (hq) in
//     wavefront 0, one lane per value, as k_quantize_decode would.
//   - The shared expert's workgroups (W4A16) read x itself and write hs.
// A routed workgroup whose id is invalid returns as a whole before the
// barrier; every other one takes it whole.
// (Quantizing x inside each workgroup instead, into LDS, measured slower:
// 30.2 against 27.8 us at 288 experts, top-8, shared expert 768. The
// quantization sits in front of every workgroup's first weight load.)
// At most 80 VGPRs (six wavefronts per SIMD): three workgroups per CU, so
// the M = 1 grid runs in about one round (83 unbounded: two per CU); W7
// caps them for seven, taken when the grid holds more wavefronts than one
// round at six (the shared expert's grid row), as for k_moe_gate_up.
template <bool W7>
__global__ __launch_bounds__(64 * kW4Waves) __attribute__((amdgpu_waves_per_eu(W7 ? 7 : 6)))
void k_moe_gate_up_w4a4_1(
    const uint8_t* __restrict__ w13_codes, const uint8_t* __restrict__ w13_scales,
    const float* __restrict__ w13_gscale, const uint16_t* __restrict__ x,
    const uint16_t* __restrict__ xq, const float* __restrict__ ga13,
    const float* __restrict__ ga2, const int32_t* __restrict__ ids, int topk, int64_t E,
    int64_t H, int64_t I, uint16_t* __restrict__ h, uint16_t* __restrict__ hq,
    const MoeShared sh) {
  __shared__ uint16_t s_hb[2 * kW4Waves];   // the workgroup's 16 h values
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t r0 = ((int64_t)blockIdx.x * kW4Waves + w) * 2;
  if (sh.I > 0 && blockIdx.y == 0) {
    // the shared expert: W4A16, its rows once for the token
    if (r0 < sh.I) {
      const int slot[1] = {0};
      gate_up_rows<1>(sh.c13, sh.s13, *sh.g13, x, H, sh.I, r0, 1, slot, 1, sh.h);
    }
    return;
  }
  const int j = sh.I > 0 ? (int)blockIdx.y - 1 : (int)blockIdx.y;
  if ((int64_t)blockIdx.x * 2 * kW4Waves >= I) return;   // the whole workgroup
  const int32_t e = ids[j];
  if (e < 0 || (int64_t)e >= E) return;                   // the whole workgroup
  // this wavefront's gate rows r0, r0 + 1 and up rows I + r0, I + r0 + 1 (the
  // workgroup's 16 rows lie below I)
  {
    const float g = w13_gscale[e] * *ga13;
    const int64_t rows[4] = {r0, r0 + 1, I + r0, I + r0 + 1};
    const uint16_t* xs[1] = {xq};
    float acc[4][1];
    wave_row_dots<1, 4>(w13_codes + (int64_t)e * (2 * I) * (H / 2),
                        w13_scales + (int64_t)e * (2 * I) * (H / 16), H, rows, xs, 1, acc);
    if (lane < 2) {
      const float G = g * (lane == 0 ? acc[0][0] : acc[1][0]);
      const float U = g * (lane == 0 ? acc[2][0] : acc[3][0]);
      const float act = G / (1.0f + expf(-G)) * U;
      const uint16_t hb = bf16_rne(act);
      h[(int64_t)j * I + r0 + lane] = hb;
      s_hb[2 * w + lane] = hb;
    }
  }
  __syncthreads();
  // the 16 h values on the grid of g_h: wavefront 0, one lane per value (all
  // 64 lanes run the row reductions; lanes 0..15 hold the block)
  if (w == 0) {
    const uint16_t q =
        quantize_decode_lane(__uint_as_float((uint32_t)s_hb[lane & 15] << 16), *ga2);
    if (lane < 16) hq[(int64_t)j * I + (int64_t)blockIdx.x * 2 * kW4Waves + lane] = q;
  }
}

// M = 1. grid ceil(H / (R * kMoeWaves)); a wavefront owns output rows n0 .. n0+R-1
// for every token. Routed slots read h with coefficient gate_w * g2[e] * *ga
// (ga = NULL for W4A16; for W4A4, h holds the activations on the NVFP4 grid
// and ga their static scale).
template <int R, int U>
__global__ __launch_bounds__(256) void k_moe_down(
    const uint8_t* __restrict__ w2_codes, const uint8_t* __restrict__ w2_scales,
    const float* __restrict__ w2_gscale, const uint16_t* __restrict__ h,
    const float* __restrict__ ga, const int32_t* __restrict__ ids,
    const float* __restrict__ gate_w, int M, int topk, int64_t E, int64_t H, int64_t I,
    float* __restrict__ y, const MoeShared sh) {
  const int lane = threadIdx.x & 63;
  const int64_t n0 =
      ((int64_t)blockIdx.x * kMoeWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6)) * R;
  if (n0 >= H) return;
  const int C = (int)(I >> 5);        // 32-element chunks per expert row
  const int64_t cb = I >> 1, sb = I >> 4;
  const int64_t ecb = H * cb, esb = H * sb;
  const float invC = 1.0f / (float)C;
  // the shared expert's chunks follow each token's routed slots
  const int Cs = (int)(sh.I >> 5);
  const int64_t cbs = sh.I >> 1, sbs = sh.I >> 4;
  const float gs2 = Cs > 0 ? *sh.g2 : 0.0f;
  const float gah = ga ? *ga : 1.0f;
  int64_t rows[R];
#pragma unroll
  for (int r = 0; r < R; ++r) rows[r] = (n0 + r < H) ? n0 + r : H - 1;

  for (int m = 0; m < M; ++m) {
    // compact the token's valid slots into lanes 0 .. nv-1, in slot order
    const int jl = m * topk + lane;
    const int32_t ev = lane < topk ? ids[jl] : -1;
    const bool valid = lane < topk && ev >= 0 && (int64_t)ev < E;
    const uint64_t vm = __ballot(valid);
    const int nv = __popcll(vm);
    float coef = 0.0f;
    if (valid) coef = ga ? gate_w[jl] * w2_gscale[ev] * gah : gate_w[jl] * w2_gscale[ev];
    const int q = __builtin_amdgcn_mbcnt_hi((uint32_t)(vm >> 32),
                                            __builtin_amdgcn_mbcnt_lo((uint32_t)vm, 0u));
    const int dst = (valid ? q : 63) * 4;    // lane 63 is never read (nv <= 16)
    const int e_c = __builtin_amdgcn_ds_permute(dst, ev);
    const int j_c = __builtin_amdgcn_ds_permute(dst, jl);
    const int f_c = __builtin_amdgcn_ds_permute(dst, __float_as_int(coef));

    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.0f;
    const int PR = nv * C;   // (slot, chunk) pairs of this token's routed slots
    const int P = PR + Cs;   // then the shared expert's chunks
    for (int p0 = 0; p0 < P; p0 += 64 * U) {
      u32x4_t qv[U][R];
      uint32_t sw[U][R];
      u32x4_t hv[U][4];
      float cf[U];
      bool live[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int p = p0 + lane + 64 * u;
        live[u] = p < P;
        const int pc = live[u] ? p : P - 1;
        const bool shp = pc >= PR;   // a shared-expert chunk
        const int pr = shp ? 0 : pc;
        int qi = (int)(((float)pr + 0.5f) * invC);
        if (qi * C > pr) --qi;
        if ((qi + 1) * C <= pr) ++qi;
        const int c = shp ? pc - PR : pr - qi * C;
        const int ee = __shfl(e_c, qi, 64);
        const int jj = __shfl(j_c, qi, 64);
        const float fr = __int_as_float(__shfl(f_c, qi, 64));
        cf[u] = shp ? gs2 : fr;
        const uint8_t* cbase = shp ? sh.c2 + (int64_t)c * 16
                                   : w2_codes + (int64_t)ee * ecb + (int64_t)c * 16;
        const uint8_t* sbase = shp ? sh.s2 + (int64_t)c * 2
                                   : w2_scales + (int64_t)ee * esb + (int64_t)c * 2;
        const int64_t rcb = shp ? cbs : cb, rsb = shp ? sbs : sb;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          qv[u][r] = load_stream(cbase + rows[r] * rcb);
          sw[u][r] = *reinterpret_cast<const uint16_t*>(sbase + rows[r] * rsb);
        }
        const uint16_t* hrow = shp ? sh.h + (int64_t)m * sh.I : h + (int64_t)jj * I;
        const u32x4_t* hp = reinterpret_cast<const u32x4_t*>(hrow + c * 32);
#pragma unroll
        for (int t = 0; t < 4; ++t) hv[u][t] = hp[t];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int b2 = 0; b2 < 2; ++b2) {
          const u32x4_t xa = hv[u][2 * b2], xb = hv[u][2 * b2 + 1];
          const bf16x2_t xv[8] = {as_bf16x2(xa.x), as_bf16x2(xa.y), as_bf16x2(xa.z),
                                  as_bf16x2(xa.w), as_bf16x2(xb.x), as_bf16x2(xb.y),
                                  as_bf16x2(xb.z), as_bf16x2(xb.w)};
#pragma unroll
          for (int r = 0; r < R; ++r) {
            const uint32_t w0 = b2 ? qv[u][r].z : qv[u][r].x;
            const uint32_t w1 = b2 ? qv[u][r].w : qv[u][r].y;
            float p = 0.0f;
            p = dot2(e2m1x2_to_bf16<0>(w0), xv[0], p);
            p = dot2(e2m1x2_to_bf16<1>(w0), xv[1], p);
            p = dot2(e2m1x2_to_bf16<2>(w0), xv[2], p);
            p = dot2(e2m1x2_to_bf16<3>(w0), xv[3], p);
            p = dot2(e2m1x2_to_bf16<0>(w1), xv[4], p);
            p = dot2(e2m1x2_to_bf16<1>(w1), xv[5], p);
            p = dot2(e2m1x2_to_bf16<2>(w1), xv[6], p);
            p = dot2(e2m1x2_to_bf16<3>(w1), xv[7], p);
            const float s = (b2 ? e4m3_to_f32<1>(sw[u][r]) : e4m3_to_f32<0>(sw[u][r])) * cf[u];
            const float na = __builtin_fmaf(p, s, acc[r]);
            acc[r] = live[u] ? na : acc[r];
          }
        }
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float t = wave_sum(acc[r]);
      if (lane == r && n0 + r < H) y[(int64_t)m * H + n0 + r] = t;
    }
  }
}

// One token (M = 1): the products of k_moe_down<R, U> in the same per-lane
// order (lane l takes pairs l, l + 64, l + 128, ... of the token's routed
// then shared (slot, chunk) pairs), so the same y bit for bit, with the
// memory side rearranged as in k_moe_gate_up_1x:
//  - each lane issues the loads of all KP of its pairs before the first
//    product (one HBM round trip per wavefront instead of one per U pairs);
//  - the h chunks of all pairs (every valid slot's h row, then the shared
//    expert's) are staged once per workgroup in LDS, pair p's 64 bytes
//    where x1x_unit puts chunk p, so that 16 lanes reading 16 consecutive
//    pairs hit distinct banks. Every wavefront used to read all of h
//    through the L1.
// Needs P = (valid slots) I/32 + Is/32 <= 64 KP; the launcher checks the
// bound for topk valid slots.
template <int R, int KP>
__global__ __launch_bounds__(256) void k_moe_down_1x(
    const uint8_t* __restrict__ w2_codes, const uint8_t* __restrict__ w2_scales,
    const float* __restrict__ w2_gscale, const uint16_t* __restrict__ h,
    const float* __restrict__ ga, const int32_t* __restrict__ ids,
    const float* __restrict__ gate_w, int topk, int64_t E, int64_t H, int64_t I,
    float* __restrict__ y, const MoeShared sh) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  u32x4_t* const hl = reinterpret_cast<u32x4_t*>(lds);
  const int lane = threadIdx.x & 63;
  const int64_t n0 =
      ((int64_t)blockIdx.x * kMoeWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6)) * R;
  const int C = (int)(I >> 5);
  const int64_t cb = I >> 1, sb = I >> 4;
  const int64_t ecb = H * cb, esb = H * sb;
  const float invC = 1.0f / (float)C;
  const int Cs = (int)(sh.I >> 5);
  const int64_t cbs = sh.I >> 1, sbs = sh.I >> 4;
  const float gs2 = Cs > 0 ? *sh.g2 : 0.0f;
  const float gah = ga ? *ga : 1.0f;
  int64_t rows[R];
#pragma unroll
  for (int r = 0; r < R; ++r) rows[r] = (n0 + r < H) ? n0 + r : H - 1;
  // the token's valid slots compacted into lanes 0 .. nv-1, in slot order
  // (every wavefront of the workgroup builds the same table)
  const int32_t ev = lane < topk ? ids[lane] : -1;
  const bool valid = lane < topk && ev >= 0 && (int64_t)ev < E;
  const uint64_t vm = __ballot(valid);
  const int nv = __popcll(vm);
  float coef = 0.0f;
  if (valid) coef = ga ? gate_w[lane] * w2_gscale[ev] * gah : gate_w[lane] * w2_gscale[ev];
  const int qv_ = __builtin_amdgcn_mbcnt_hi((uint32_t)(vm >> 32),
                                            __builtin_amdgcn_mbcnt_lo((uint32_t)vm, 0u));
  const int dst = (valid ? qv_ : 63) * 4;   // lane 63 is never read (nv <= 16)
  const int e_c = __builtin_amdgcn_ds_permute(dst, ev);
  const int j_c = __builtin_amdgcn_ds_permute(dst, lane);
  const int f_c = __builtin_amdgcn_ds_permute(dst, __float_as_int(coef));
  const int PR = nv * C;
  const int P = PR + Cs;
  if (P == 0) {   // no valid slot and no shared expert: y = 0 (the whole workgroup)
    if (lane < R && n0 + lane < H) y[n0 + lane] = 0.0f;
    return;
  }
  // the pair of an index: (slot q, chunk c) for routed pairs, chunk c of the
  // shared expert otherwise
  auto pair_of = [&](int pc, bool& shp, int& qi, int& c) {
    shp = pc >= PR;
    const int pr = shp ? 0 : pc;
    qi = (int)(((float)pr + 0.5f) * invC);
    if (qi * C > pr) --qi;
    if ((qi + 1) * C <= pr) ++qi;
    c = shp ? pc - PR : pr - qi * C;
  };
  // h units to stage: KP per thread (P <= 64 KP pairs of 4 units); the
  // surplus threads repeat the last unit
  u32x4_t hs[KP];
#pragma unroll
  for (int k = 0; k < KP; ++k) {
    const int u0 = (int)threadIdx.x + 256 * k;
    const int u = u0 < 4 * P ? u0 : 4 * P - 1;
    bool shp;
    int qi, c;
    pair_of(u >> 2, shp, qi, c);
    const int jj = __shfl(j_c, qi, 64);
    const uint16_t* src = shp ? sh.h + (int64_t)c * 32 : h + (int64_t)jj * I + c * 32;
    hs[k] = reinterpret_cast<const u32x4_t*>(src)[u & 3];
  }
  // every pair's weights
  u32x4_t qw[KP][R];
  uint32_t sw[KP][R];
  float cf[KP];
  bool live[KP];
  int pcs[KP];
#pragma unroll
  for (int k = 0; k < KP; ++k) {
    const int p = lane + 64 * k;
    live[k] = p < P;
    const int pc = live[k] ? p : P - 1;
    pcs[k] = pc;
    bool shp;
    int qi, c;
    pair_of(pc, shp, qi, c);
    const int ee = __shfl(e_c, qi, 64);
    const float fr = __int_as_float(__shfl(f_c, qi, 64));
    cf[k] = shp ? gs2 : fr;
    const uint8_t* cbase = shp ? sh.c2 + (int64_t)c * 16
                               : w2_codes + (int64_t)ee * ecb + (int64_t)c * 16;
    const uint8_t* sbase = shp ? sh.s2 + (int64_t)c * 2
                               : w2_scales + (int64_t)ee * esb + (int64_t)c * 2;
    const int64_t rcb = shp ? cbs : cb, rsb = shp ? sbs : sb;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      qw[k][r] = load_stream(cbase + rows[r] * rcb);
      sw[k][r] = *reinterpret_cast<const uint16_t*>(sbase + rows[r] * rsb);
    }
  }
#pragma unroll
  for (int k = 0; k < KP; ++k) {
    const int u0 = (int)threadIdx.x + 256 * k;
    const int u = u0 < 4 * P ? u0 : 4 * P - 1;
    hl[x1x_unit(u)] = hs[k];
  }
  __syncthreads();
  if (n0 >= H) return;
  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.0f;
#pragma unroll
  for (int k = 0; k < KP; ++k) {
    const int pc = pcs[k];
#pragma unroll
    for (int b2 = 0; b2 < 2; ++b2) {
      const u32x4_t xa = hl[x1x_unit(4 * pc + 2 * b2)];
      const u32x4_t xb = hl[x1x_unit(4 * pc + 2 * b2 + 1)];
      const bf16x2_t xv[8] = {as_bf16x2(xa.x), as_bf16x2(xa.y), as_bf16x2(xa.z),
                              as_bf16x2(xa.w), as_bf16x2(xb.x), as_bf16x2(xb.y),
                              as_bf16x2(xb.z), as_bf16x2(xb.w)};
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const uint32_t w0 = b2 ? qw[k][r].z : qw[k][r].x;
        const uint32_t w1 = b2 ? qw[k][r].w : qw[k][r].y;
        float p = 0.0f;
        p = dot2(e2m1x2_to_bf16<0>(w0), xv[0], p);
        p = dot2(e2m1x2_to_bf16<1>(w0), xv[1], p);
        p = dot2(e2m1x2_to_bf16<2>(w0), xv[2], p);
        p = dot2(e2m1x2_to_bf16<3>(w0), xv[3], p);
        p = dot2(e2m1x2_to_bf16<0>(w1), xv[4], p);
        p = dot2(e2m1x2_to_bf16<1>(w1), xv[5], p);
        p = dot2(e2m1x2_to_bf16<2>(w1), xv[6], p);
        p = dot2(e2m1x2_to_bf16<3>(w1), xv[7], p);
        const float s = (b2 ? e4m3_to_f32<1>(sw[k][r]) : e4m3_to_f32<0>(sw[k][r])) * cf[k];
        const float na = __builtin_fmaf(p, s, acc[r]);
        acc[r] = live[k] ? na : acc[r];
      }
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float t = wave_sum(acc[r]);
    if (lane == r && n0 + r < H) y[n0 + r] = t;
  }
}

constexpr int kMaxTok = NVFP4_MOE_MAX_M_INTERNAL;  // tokens per call
constexpr int kMaxSl = NVFP4_MAX_TOPK_INTERNAL;    // slots per token
constexpr int kSplitRows = 8;                      // k_moe_down_split: rows per workgroup,
constexpr int kSplitUnroll = 2;                    //   (slot, chunk) pairs in flight per lane
constexpr int kSplitWaves = 8;                     //   and wavefronts per workgroup

// The down pass and combine for M >= 2, split over wavefronts. The same
// dot products as k_moe_down, dealt out differently: a workgroup of NW
// wavefronts owns R output rows, and the units of work of all its tokens
// (token m, a block of 64U consecutive (slot, chunk) pairs of that token's
// valid slots and shared-expert chunks) go to its wavefronts round robin.
// Units are numbered token by token, so a wavefront finishes its units of
// one token before it starts the next: each lane keeps one partial per row
// of the current token only (R registers, not R per token), and the
// wavefront sums them into LDS when it moves on. The wavefronts' sums meet
// in LDS and are added in wavefront order (deterministic). Compared with one
// wavefront walking every token's pairs for its rows, this keeps several
// times more wavefronts, and so more loads, in flight for the same work per
// weight byte; the slot compaction of every token is built once per
// workgroup in LDS.
template <int R, int U, int NW>
__global__ __launch_bounds__(64 * NW) void k_moe_down_split(
    const uint8_t* __restrict__ w2_codes, const uint8_t* __restrict__ w2_scales,
    const float* __restrict__ w2_gscale, const uint16_t* __restrict__ h,
    const float* __restrict__ ga, const int32_t* __restrict__ ids,
    const float* __restrict__ gate_w, int M, int topk, int64_t E, int64_t H, int64_t I,
    float* __restrict__ y, const MoeShared sh) {
  __shared__ int s_e[kMaxTok][kMaxSl];
  __shared__ int s_j[kMaxTok][kMaxSl];
  __shared__ float s_f[kMaxTok][kMaxSl];
  __shared__ int s_nv[kMaxTok];
  __shared__ float s_part[NW][R][kMaxTok];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t n0 = (int64_t)blockIdx.x * R;
  const int C = (int)(I >> 5);
  const int64_t cb = I >> 1, sb = I >> 4;
  const int64_t ecb = H * cb, esb = H * sb;
  const float invC = 1.0f / (float)C;
  const int Cs = (int)(sh.I >> 5);
  const int64_t cbs = sh.I >> 1, sbs = sh.I >> 4;
  const float gs2 = Cs > 0 ? *sh.g2 : 0.0f;
  const float gah = ga ? *ga : 1.0f;
  for (int m = w; m < M; m += NW) {
    const int jl = m * topk + lane;
    const int32_t ev = lane < topk ? ids[jl] : -1;
    const bool valid = lane < topk && ev >= 0 && (int64_t)ev < E;
    const uint64_t vm = __ballot(valid);
    const int q = __builtin_amdgcn_mbcnt_hi((uint32_t)(vm >> 32),
                                            __builtin_amdgcn_mbcnt_lo((uint32_t)vm, 0u));
    if (valid) {
      s_e[m][q] = ev;
      s_j[m][q] = jl;
      s_f[m][q] = ga ? gate_w[jl] * w2_gscale[ev] * gah : gate_w[jl] * w2_gscale[ev];
    }
    if (lane == 0) s_nv[m] = __popcll(vm);
  }
  __syncthreads();
  int64_t rows[R];
#pragma unroll
  for (int r = 0; r < R; ++r) rows[r] = (n0 + r < H) ? n0 + r : H - 1;
  int unit = 0;
  for (int m = 0; m < M; ++m) {
    // the lane's partials of token m: only the current token's are live
    float tok[R];
#pragma unroll
    for (int r = 0; r < R; ++r) tok[r] = 0.0f;
    bool any = false;
    const int nv = __builtin_amdgcn_readfirstlane(s_nv[m]);
    const int PR = nv * C;
    const int P = PR + Cs;
    const int nb = (P + 64 * U - 1) / (64 * U);
    for (int b = 0; b < nb; ++b, ++unit) {
      if (unit % NW != w) continue;
      any = true;
      u32x4_t qv[U][R];
      uint32_t sw[U][R];
      u32x4_t hv[U][4];
      float cf[U];
      bool live[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int p = b * 64 * U + lane + 64 * u;
        live[u] = p < P;
        const int pc = live[u] ? p : P - 1;
        const bool shp = pc >= PR;
        const int pr = shp ? 0 : pc;
        int qi = (int)(((float)pr + 0.5f) * invC);
        if (qi * C > pr) --qi;
        if ((qi + 1) * C <= pr) ++qi;
        const int c = shp ? pc - PR : pr - qi * C;
        const int ee = s_e[m][qi];
        const int jj = s_j[m][qi];
        const float fr = s_f[m][qi];
        cf[u] = shp ? gs2 : fr;
        const uint8_t* cbase = shp ? sh.c2 + (int64_t)c * 16
                                   : w2_codes + (int64_t)ee * ecb + (int64_t)c * 16;
        const uint8_t* sbase = shp ? sh.s2 + (int64_t)c * 2
                                   : w2_scales + (int64_t)ee * esb + (int64_t)c * 2;
        const int64_t rcb = shp ? cbs : cb, rsb = shp ? sbs : sb;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          qv[u][r] = load_stream(cbase + rows[r] * rcb);
          sw[u][r] = *reinterpret_cast<const uint16_t*>(sbase + rows[r] * rsb);
        }
        const uint16_t* hrow = shp ? sh.h + (int64_t)m * sh.I : h + (int64_t)jj * I;
        const u32x4_t* hp = reinterpret_cast<const u32x4_t*>(hrow + c * 32);
#pragma unroll
        for (int t = 0; t < 4; ++t) hv[u][t] = hp[t];
      }
      float acc[R];
#pragma unroll
      for (int r = 0; r < R; ++r) acc[r] = 0.0f;
#pragma unroll
      for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int b2 = 0; b2 < 2; ++b2) {
          const u32x4_t xa = hv[u][2 * b2], xb = hv[u][2 * b2 + 1];
          const bf16x2_t xv[8] = {as_bf16x2(xa.x), as_bf16x2(xa.y), as_bf16x2(xa.z),
                                  as_bf16x2(xa.w), as_bf16x2(xb.x), as_bf16x2(xb.y),
                                  as_bf16x2(xb.z), as_bf16x2(xb.w)};
#pragma unroll
          for (int r = 0; r < R; ++r) {
            const uint32_t w0 = b2 ? qv[u][r].z : qv[u][r].x;
            const uint32_t w1 = b2 ? qv[u][r].w : qv[u][r].y;
            float p = 0.0f;
            p = dot2(e2m1x2_to_bf16<0>(w0), xv[0], p);
            p = dot2(e2m1x2_to_bf16<1>(w0), xv[1], p);
            p = dot2(e2m1x2_to_bf16<2>(w0), xv[2], p);
            p = dot2(e2m1x2_to_bf16<3>(w0), xv[3], p);
            p = dot2(e2m1x2_to_bf16<0>(w1), xv[4], p);
            p = dot2(e2m1x2_to_bf16<1>(w1), xv[5], p);
            p = dot2(e2m1x2_to_bf16<2>(w1), xv[6], p);
            p = dot2(e2m1x2_to_bf16<3>(w1), xv[7], p);
            const float s = (b2 ? e4m3_to_f32<1>(sw[u][r]) : e4m3_to_f32<0>(sw[u][r])) * cf[u];
            const float na = __builtin_fmaf(p, s, acc[r]);
            acc[r] = live[u] ? na : acc[r];
          }
        }
      }
#pragma unroll
      for (int r = 0; r < R; ++r) tok[r] += acc[r];
    }
    // the wave's sums of token m (zero when it took none of its units)
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float t = any ? wave_sum(tok[r]) : 0.0f;
      if (lane == 0) s_part[w][r][m] = t;
    }
  }
  __syncthreads();
  const int t = threadIdx.x;
  if (t < R * M) {
    const int r = t / M, m = t % M;
    float sum = 0.0f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) sum += s_part[ww][r][m];
    if (n0 + r < H) y[(int64_t)m * H + n0 + r] = sum;
  }
}

hipError_t launch_moe(const uint8_t* w13_codes, const uint8_t* w13_scales,
                      const float* w13_gscale, const uint8_t* w2_codes,
                      const uint8_t* w2_scales, const float* w2_gscale, const uint16_t* x,
                      const int32_t* ids, const float* gate_w, int M, int64_t E, int64_t H,
                      int64_t I, int topk, const MoeShared* shared, const MoeW4a4* w4a4,
                      float* y, void* workspace, hipStream_t stream) {
  MoeShared sh = {};
  if (shared) sh = *shared;
  const MoeLayout L = moe_layout(M, H, I, topk, sh.I, w4a4 != nullptr);
  char* ws = static_cast<char*>(workspace);
  uint16_t* h = reinterpret_cast<uint16_t*>(ws + L.h_off);
  sh.h = reinterpret_cast<uint16_t*>(ws + L.hs_off);
  const int S = M * topk;
  const uint16_t* xr = x;        // routed gate|up input
  const uint16_t* hr = h;        // routed down input
  const float* ga13 = nullptr;
  const float* ga2 = nullptr;
  if (w4a4 && M == 1) {
    // x onto the grid of its static scale, then gate|up, which also puts h
    // on the grid of its own: three launches
    uint16_t* hq = reinterpret_cast<uint16_t*>(ws + L.hq_off);
    uint16_t* xq = reinterpret_cast<uint16_t*>(ws + L.xq_off);
    hipError_t e = launch_quantize_decode(x, M, H, w4a4->ga13, nullptr, 0, xq, stream);
    if (e != hipSuccess) return e;
    const int64_t rows = sh.I > I ? sh.I : I;
    const int64_t gx = (rows + 2 * kW4Waves - 1) / (2 * kW4Waves);
    const dim3 grid((unsigned)gx, S + (sh.I > 0 ? 1 : 0));
    if ((int64_t)grid.x * grid.y * kW4Waves > kOneRoundWaves6)
      hipLaunchKernelGGL(k_moe_gate_up_w4a4_1<true>, grid, dim3(64 * kW4Waves), 0, stream,
                         w13_codes, w13_scales, w13_gscale, x, xq, w4a4->ga13, w4a4->ga2, ids,
                         topk, E, H, I, h, hq, sh);
    else
      hipLaunchKernelGGL(k_moe_gate_up_w4a4_1<false>, grid, dim3(64 * kW4Waves), 0, stream,
                         w13_codes, w13_scales, w13_gscale, x, xq, w4a4->ga13, w4a4->ga2, ids,
                         topk, E, H, I, h, hq, sh);
    xr = nullptr;   // gate|up is done
    hr = hq;
    ga2 = w4a4->ga2;
  } else if (w4a4) {
    // the token's activations onto the NVFP4 grid of their static scale
    uint16_t* xq = reinterpret_cast<uint16_t*>(ws + L.xq_off);
    hipError_t e = launch_quantize_decode(x, M, H, w4a4->ga13, nullptr, 0, xq, stream);
    if (e != hipSuccess) return e;
    xr = xq;
    hr = reinterpret_cast<const uint16_t*>(ws + L.hq_off);
    ga13 = w4a4->ga13;
    ga2 = w4a4->ga2;
  }
  if (xr) {
    const int64_t pairs = ((sh.I > I ? sh.I : I) + 1) / 2;
    const int64_t yb = (pairs + kMoeWaves - 1) / kMoeWaves;
    const dim3 grid((unsigned)yb, S + (sh.I > 0 ? 1 : 0));
    const bool w7 = (int64_t)grid.x * grid.y * kMoeWaves > kOneRoundWaves6;
    if (M == 1 && H == 4096) {
      const size_t lds = (size_t)H * sizeof(uint16_t);
      if (w7)
        hipLaunchKernelGGL((k_moe_gate_up_1x<2, true>), grid, dim3(256), lds, stream, w13_codes,
                           w13_scales, w13_gscale, x, xr, ga13, ids, E, H, I, h, sh);
      else
        hipLaunchKernelGGL((k_moe_gate_up_1x<2, false>), grid, dim3(256), lds, stream, w13_codes,
                           w13_scales, w13_gscale, x, xr, ga13, ids, E, H, I, h, sh);
    } else if (M == 1 && w7)
      hipLaunchKernelGGL((k_moe_gate_up<1, true>), grid, dim3(256), 0, stream, w13_codes,
                         w13_scales, w13_gscale, x, xr, ga13, ids, S, topk, E, H, I, h, sh, M);
    else if (M == 1)
      hipLaunchKernelGGL((k_moe_gate_up<1, false>), grid, dim3(256), 0, stream, w13_codes,
                         w13_scales, w13_gscale, x, xr, ga13, ids, S, topk, E, H, I, h, sh, M);
    else if (H == 4096)
      hipLaunchKernelGGL((k_moe_gate_up_mx<2>), grid, dim3(256), (size_t)4 * H, stream,
                         w13_codes, w13_scales, w13_gscale, x, xr, ga13, ids, S, topk, E, H, I,
                         h, sh, M);
    else
      hipLaunchKernelGGL((k_moe_gate_up<kGateUpSlots, false>), grid, dim3(256), 0, stream,
                         w13_codes, w13_scales, w13_gscale, x, xr, ga13, ids, S, topk, E, H, I,
                         h, sh, M);
  }
  if (w4a4 && xr) {
    // h of every valid slot onto the NVFP4 grid of its static scale
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_quantize_decode(h, S, I, ga2, ids, E, const_cast<uint16_t*>(hr), stream);
    if (e != hipSuccess) return e;
  }
  const int64_t pmax = (int64_t)topk * (I >> 5) + (sh.I >> 5);   // pairs with every slot valid
  if (M == 1 && pmax >= 1 && pmax <= 64 * 8) {
    const int64_t wgs = (H + kDownRows * kMoeWaves - 1) / (kDownRows * kMoeWaves);
    const int kp = (int)((pmax + 63) / 64);
    const size_t lds = (size_t)pmax * 64;
#define NVFP4_DOWN1X(KK)                                                                  \
  hipLaunchKernelGGL((k_moe_down_1x<kDownRows, KK>), dim3((unsigned)wgs), dim3(256), lds, \
                     stream, w2_codes, w2_scales, w2_gscale, hr, ga2, ids, gate_w, topk, E, H, \
                     I, y, sh)
    if (kp <= 2) NVFP4_DOWN1X(2);
    else if (kp <= 4) NVFP4_DOWN1X(4);
    else if (kp <= 6) NVFP4_DOWN1X(6);
    else if (kp <= 7) NVFP4_DOWN1X(7);
    else NVFP4_DOWN1X(8);
#undef NVFP4_DOWN1X
  } else if (M == 1) {
    const int64_t wgs = (H + kDownRows * kMoeWaves - 1) / (kDownRows * kMoeWaves);
    hipLaunchKernelGGL((k_moe_down<kDownRows, kDownUnroll>), dim3((unsigned)wgs), dim3(256), 0,
                       stream, w2_codes, w2_scales, w2_gscale, hr, ga2, ids, gate_w, M, topk, E,
                       H, I, y, sh);
  } else {
    const int64_t wgs = (H + kSplitRows - 1) / kSplitRows;
    hipLaunchKernelGGL((k_moe_down_split<kSplitRows, kSplitUnroll, kSplitWaves>), dim3((unsigned)wgs),
                       dim3(64 * kSplitWaves), 0, stream, w2_codes, w2_scales, w2_gscale, hr, ga2,
                       ids, gate_w, M, topk, E, H, I, y, sh);
  }
  return hipGetLastError();
}

}  // namespace nvfp4
