// gemv_mt.hip -- NVFP4 g16 W4A16 GEMV on the CDNA4 matrix cores for
// 9 <= M <= 128 activation rows (many tokens: the blueprint's "multi_seq"
// plan arm takes 2 to 128 rows, and its planner settings enable the tensor
// cores for W4A16, "w4a16_tc=on").
//
//   y[m, n] = g * sum_k e2m1(c[n,k]) * e4m3(s[n, k/16]) * x[m, k]
//
// Why a kernel of its own. The M <= 8 kernels put two 16-element blocks
// side by side in one v_mfma_f32_16x16x32_bf16 (eight tokens per block half)
// and scale the output by the block scale; that spends the instruction's
// sixteen A rows on two blocks. With more tokens every A row is a token: the
// E4M3 block scale is folded into the weights instead (e2m1 * s has at most
// 6 significant bits in [2^-10, 2688], so it is exact in bf16), the decode of
// a weight fragment costs about 2 instructions per weight once, and every
// group of 16 tokens adds one MFMA per fragment with no per-block work.
//
// Work split. A workgroup is 4 wavefronts and owns T tiles of 16 weight rows
// (of one segment) and GW groups of 16 tokens; its wavefronts split K into
// four contiguous ranges of 128-k steps and meet once, at the end, in LDS
// (their partial tiles summed in wavefront order: deterministic). The
// token groups of a row block are separate workgroups on the grid's second
// dimension, mapped so that all of them go to the same XCD (workgroups are
// dealt to the 8 XCDs round robin in linear order): the weights they share
// are read from HBM once and served to the others by that XCD's L2.
//
// Operand mapping of v_mfma_f32_16x16x32_bf16 (lane l, i = l % 16,
// g = l / 16): A (16 x 32) lane holds A[i][8g .. 8g+7], B (32 x 16) lane
// holds B[8g .. 8g+7][i], D (16 x 16) lane holds D[4g + r][i], r < 4. Step s
// covers k in [128 s, 128 s + 128): lane (i, g) loads the 16 code bytes of
// weight row i at k = 128 s + 32 g (two blocks) and MFMA d (d < 4) takes its
// dword d, k = 128 s + 32 g + 8 d .. +8, as B; A row t of that MFMA is token
// t's x at the same k. Lanes whose 32 k lie past K (K % 128 != 0) feed zeros
// on both sides.
#include "device.h"
#include "internal.h"

namespace nvfp4 {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kMtWaves = 4;

// bf16x8 of the 8 E2M1 codes of `word` times the block scale s: exact (the
// products have at most 6 significant bits and lie in bf16's range).
__device__ __forceinline__ bf16x8_t mt_decode8(uint32_t word, float s) {
  const float2_t p0 = e2m1x2_to_f32<0>(word);
  const float2_t p1 = e2m1x2_to_f32<1>(word);
  const float2_t p2 = e2m1x2_to_f32<2>(word);
  const float2_t p3 = e2m1x2_to_f32<3>(word);
  const bf16x2_t b0 = __builtin_convertvector(p0 * s, bf16x2_t);
  const bf16x2_t b1 = __builtin_convertvector(p1 * s, bf16x2_t);
  const bf16x2_t b2 = __builtin_convertvector(p2 * s, bf16x2_t);
  const bf16x2_t b3 = __builtin_convertvector(p3 * s, bf16x2_t);
  bf16x8_t r;
  r[0] = b0[0]; r[1] = b0[1]; r[2] = b1[0]; r[3] = b1[1];
  r[4] = b2[0]; r[5] = b2[1]; r[6] = b3[0]; r[7] = b3[1];
  return r;
}

__device__ __forceinline__ bf16x8_t mt_bf16x8(u32x4_t v) {
  bf16x8_t r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

// The weights of one step for T tiles: lane (i, g)'s 16 code bytes and its
// two scale bytes (first block in bits 7..0) per tile.
template <int T>
struct MtWeights {
  u32x4_t q[T];
  uint32_t s[T];
};

}  // namespace

template <int T, int GW>
__global__ __launch_bounds__(64 * kMtWaves) void k_gemv_mt(const SegTable tab,
                                                           const uint16_t* __restrict__ x,
                                                           int M, int64_t K, int64_t units,
                                                           int groups) {
  // blockIdx.x -> (row block, token group): the groups of a row block share
  // the XCD that blockIdx.x % 8 selects
  const int64_t b = blockIdx.x;
  const int64_t per = 8 * (int64_t)groups;
  const int64_t unit = (b / per) * 8 + (b % 8);
  const int grp = (int)((b % per) / 8);
  if (unit >= units) return;   // the same for the whole workgroup
  const Seg sg = find_seg(tab, unit);
  const uint8_t* __restrict__ codes = sg.codes;
  const uint8_t* __restrict__ scales = sg.scales;
  const int64_t N = sg.N;

  extern __shared__ __attribute__((aligned(16))) f32x4_t red[];   // [W][T][GW][64]
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i = lane & 15, g = lane >> 4;
  const int64_t n0 = sg.unit * (16 * T);
  const int64_t cb = K >> 1, sbytes = K >> 4;
  const int64_t S = (K + 127) >> 7;                 // 128-k steps
  const int64_t s0 = S * w / kMtWaves, s1 = S * (w + 1) / kMtWaves;
  const int tok0 = grp * 16 * GW;

  // this lane's weight rows (a ragged last tile re-reads row N - 1; its
  // outputs are not stored) and token rows (tokens >= M feed zeros)
  const uint8_t* cp[T];
  const uint8_t* sp[T];
#pragma unroll
  for (int u = 0; u < T; ++u) {
    const int64_t n = n0 + 16 * u + i;
    const int64_t row = n < N ? n : N - 1;
    cp[u] = codes + row * cb + 16 * g;
    sp[u] = scales + row * sbytes + 2 * g;
  }
  const uint16_t* xp[GW];
  bool xok[GW];
#pragma unroll
  for (int q = 0; q < GW; ++q) {
    const int t = tok0 + 16 * q + i;
    xok[q] = t < M;
    xp[q] = x + (int64_t)(xok[q] ? t : 0) * K + 32 * g;
  }

  f32x4_t acc[T][GW];
#pragma unroll
  for (int u = 0; u < T; ++u)
#pragma unroll
    for (int q = 0; q < GW; ++q) acc[u][q] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // the weights of step s (zeros for a lane whose 32 k lie past K)
  auto load_w = [&](int64_t s, MtWeights<T>& wt) {
    const bool ok = 128 * s + 32 * g < K;
#pragma unroll
    for (int u = 0; u < T; ++u) {
      if (ok) {
        wt.q[u] = load_stream(cp[u] + 64 * s);
        wt.s[u] = *reinterpret_cast<const uint16_t*>(sp[u] + 8 * s);
      } else {
        wt.q[u] = u32x4_t{0u, 0u, 0u, 0u};
        wt.s[u] = 0u;
      }
    }
  };

  if (s0 < s1) {
    MtWeights<T> cur, nxt;
    load_w(s0, cur);
    for (int64_t s = s0; s < s1; ++s) {
      if (s + 1 < s1) load_w(s + 1, nxt);
      const bool ok = 128 * s + 32 * g < K;
      // A operands: 64 bytes of each token row at k = 128 s + 32 g
      u32x4_t xa[GW][4];
#pragma unroll
      for (int q = 0; q < GW; ++q) {
        const u32x4_t* p = reinterpret_cast<const u32x4_t*>(xp[q] + 128 * s);
#pragma unroll
        for (int d = 0; d < 4; ++d)
          xa[q][d] = (ok && xok[q]) ? p[d] : u32x4_t{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        bf16x8_t bw[T];
#pragma unroll
        for (int u = 0; u < T; ++u) {
          const float sc = d < 2 ? e4m3_to_f32<0>(cur.s[u]) : e4m3_to_f32<1>(cur.s[u]);
          const uint32_t word = d == 0 ? cur.q[u].x : d == 1 ? cur.q[u].y
                              : d == 2 ? cur.q[u].z : cur.q[u].w;
          bw[u] = mt_decode8(word, sc);
        }
#pragma unroll
        for (int q = 0; q < GW; ++q)
#pragma unroll
          for (int u = 0; u < T; ++u)
            acc[u][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(mt_bf16x8(xa[q][d]), bw[u],
                                                                acc[u][q], 0, 0, 0);
      }
      if (s + 1 < s1) cur = nxt;
    }
  }

  // the four wavefronts' partial tiles, summed in wavefront order
#pragma unroll
  for (int u = 0; u < T; ++u)
#pragma unroll
    for (int q = 0; q < GW; ++q) red[((w * T + u) * GW + q) * 64 + lane] = acc[u][q];
  __syncthreads();
  const float gs = *sg.gscale;
  // pair p = (u, q) is summed and stored by wavefront p % 4
#pragma unroll
  for (int p = 0; p < T * GW; ++p) {
    if (p % kMtWaves != w) continue;
    const int u = p / GW, q = p % GW;
    f32x4_t sum = red[((0 * T + u) * GW + q) * 64 + lane];
#pragma unroll
    for (int v = 1; v < kMtWaves; ++v) sum += red[((v * T + u) * GW + q) * 64 + lane];
    const int64_t n = n0 + 16 * u + i;
    if (n < N) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = tok0 + 16 * q + 4 * g + r;   // lane (i, g) holds D[4g + r][i]
        if (m < M) sg.y[(int64_t)m * N + n] = sum[r] * gs;
      }
    }
  }
}

bool mt_applicable(int M) { return M > NVFP4_MAX_M_SMALL && M <= NVFP4_MAX_M_INTERNAL; }

// Launch shape: token groups of 16 per workgroup GW (1 up to 32 tokens,
// 2 above) and tiles per workgroup T (2 when the matrices give at least 8
// workgroups per CU that way, else 1).
hipError_t launch_gemv_mt(const SegDesc* d, int n, const uint16_t* x, int M, int64_t K,
                          hipStream_t stream) {
  if (!mt_applicable(M) || n < 1 || n > kMaxSegments) return hipErrorInvalidValue;
  const int GW = M <= 32 ? 1 : 2;
  const int groups = (M + 16 * GW - 1) / (16 * GW);
  int64_t rows = 0;
  for (int s = 0; s < n; ++s) rows += d[s].N;
  const int T = (rows / 32) * groups >= 8 * 256 ? 2 : 1;
  const SegTable tab = make_seg_table(d, n, 16 * T);
  const int64_t units = tab.start[kMaxSegments];
  // whole multiples of 8 units so that the XCD mapping stays a bijection
  const int64_t grid = ((units + 7) / 8) * 8 * groups;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  const size_t lds = (size_t)kMtWaves * T * GW * 64 * sizeof(f32x4_t);
#define NVFP4_MT(TT, GG)                                                                    \
  hipLaunchKernelGGL((k_gemv_mt<TT, GG>), dim3((unsigned)grid), dim3(64 * kMtWaves), lds, \
                     stream, tab, x, M, K, units, groups)
  if (T == 2) {
    if (GW == 1) NVFP4_MT(2, 1); else NVFP4_MT(2, 2);
  } else {
    if (GW == 1) NVFP4_MT(1, 1); else NVFP4_MT(1, 2);
  }
#undef NVFP4_MT
  return hipGetLastError();
}

}  // namespace nvfp4
