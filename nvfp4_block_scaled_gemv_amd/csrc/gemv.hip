// gemv.hip -- dense NVFP4 g16 W4A16 GEMV on gfx950, vector-ALU path for
// M = 1, for M = 2 on small matrices or K that the matrix-core kernels do
// not split, and for 3 <= M <= 5 on matrices of at most 1024 rows at K =
// 4096 (M = 2 from 4096 rows with K % 256 == 0, and 3 <= M <= 8 otherwise,
// go to the matrix-core kernels of gemv_g8.hip, gemv_g8r.hip,
// gemv_splitk.hip and gemv_mfma.hip; 9 <= M <= 128 to gemv_mt.hip):
//   y[m, n] = g * sum_k e2m1(c[n,k]) * s[n, k/16] * x[m, k]
// (graph.json node "l0.kda.q": act bf16, weight nvfp4/g16 -> bf16,
// accumulate f32, scale f32). Bandwidth-bound: every weight byte is read
// from HBM exactly once; x (at most 8 x K bf16) stays in the caches.
#include "gemv_core.h"
#include "internal.h"

namespace nvfp4 {

constexpr int kWavesPerBlock = 4;
constexpr int64_t kM2MatrixCoreRows = 4096;   // M = 2 takes the matrix cores from here
constexpr int64_t kStagedManyRows = 1024;     // 3 <= M <= 5 on the vector ALUs up to here

// Each wavefront takes groups of R consecutive rows of one segment, striding
// over the groups of all segments. The nblk workgroups are numbered so that
// each XCD streams a contiguous eighth of the rows: workgroups are dealt to
// the 8 XCDs round robin in launch order, so launch index b runs workgroup
// (b % 8) * ceil(nblk / 8) + b / 8 (the grid is rounded up to a multiple of
// 8; the extra workgroups exit). Against the plain order, same-process A/B:
// LM head 50.7 -> 50.4 us, 4096 x 4096 4.74 -> 4.67 us, 12288 x 4096 at M =
// 2 10.08 -> 9.97 us (a pure read stream: 6.95 -> 7.05 TB/s).
template <int M, int R, bool SEG>
__global__ __launch_bounds__(256) void k_gemv(const SegTable tab, const uint16_t* __restrict__ x,
                                              int64_t K, unsigned nblk) {
  const int lane = threadIdx.x & 63;
  const unsigned per = (nblk + 7) / 8;
  const unsigned blk = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (blk >= nblk) return;
  // wavefront index, made provably uniform so loop control stays scalar
  const int64_t wave =
      (int64_t)blk * kWavesPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)nblk * kWavesPerBlock;
  const int64_t units = tab.start[kMaxSegments];
  const uint16_t* xs[M];
#pragma unroll
  for (int m = 0; m < M; ++m) xs[m] = x + (int64_t)m * K;

  // A single matrix reads its tensor scale once, before the loop (a load
  // after the dot products would add its latency to every wavefront's tail),
  // and skips the segment lookup (it costs registers in this loop).
  const float g0 = SEG ? 0.0f : *tab.gscale[0];
  for (int64_t u = wave; u < units; u += nwaves) {
    const Seg sg = SEG ? find_seg(tab, u)
                       : Seg{tab.codes[0], tab.scales[0], tab.gscale[0], tab.y[0], tab.N[0], u, 0};
    const float g = SEG ? *sg.gscale : g0;
    const int64_t N = sg.N;
    const int64_t n0 = sg.unit * R;
    int64_t rows[R];
#pragma unroll
    for (int r = 0; r < R; ++r) rows[r] = (n0 + r < N) ? (n0 + r) : (N - 1);
    float acc[R][M];
    wave_row_dots<M, R>(sg.codes, sg.scales, K, rows, xs, M, acc);
    // lane (r * M + m) stores one result
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int m = 0; m < M; ++m)
        if (lane == r * M + m && n0 + r < N) sg.y[(int64_t)m * N + n0 + r] = acc[r][m] * g;
  }
}

// Below 32768 rows with K = 2048 CL (launched for K = 4096, CL = 2): each wavefront has
// exactly one group of R rows (the grid covers every group), so its loads
// can all be issued at once. The workgroup stages x (M rows, x1x_unit
// layout) in LDS while the weights are in flight; every lane then issues
// the codes and scales of all CL of its chunks before the first product,
// and reads x from LDS. The products and their order per lane are those of
// wave_row_dots<M, R>, so y is the same bit for bit; the memory side waits
// for one HBM round trip per wavefront instead of CL, and x crosses the L1
// once per workgroup instead of once per wavefront. Same-process A/B at M = 1
// (calls queued back to back): 1024 x 4096 3.47 -> 3.22 us, 4096 x 4096
// 4.70 -> 4.45, 16384 x 4096 9.24 -> 8.63, 24576 x 4096 12.3 -> 11.0; at
// M = 2, 1024 x 4096 3.95 -> 3.57 and 2048 x 4096 5.02 -> 4.02. At K = 2048
// (one chunk per lane) it was slower (2048 x 2048 2.96 -> 3.08 us), so that
// K keeps k_gemv.
template <int M, int R, int CL, bool SEG>
__global__ __launch_bounds__(256) void k_gemv_1x(const SegTable tab, const uint16_t* __restrict__ x,
                                                 int64_t K, unsigned nblk) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  u32x4_t* const xl = reinterpret_cast<u32x4_t*>(lds);
  const int lane = threadIdx.x & 63;
  const unsigned per = (nblk + 7) / 8;
  const unsigned blk = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (blk >= nblk) return;   // the whole workgroup
  const int64_t u =
      (int64_t)blk * kWavesPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t units = tab.start[kMaxSegments];
  const bool act = u < units;   // the whole wavefront
  const int nu = (int)(M * (K >> 3));
  u32x4_t xv[M * CL];
  x1x_load<256, M * CL>(x, nu, xv);
  const Seg sg = SEG ? find_seg(tab, act ? u : 0)
                     : Seg{tab.codes[0], tab.scales[0], tab.gscale[0], tab.y[0], tab.N[0], u, 0};
  const int64_t N = sg.N;
  const int64_t n0 = sg.unit * R;
  const int64_t cb = K >> 1, sbytes = K >> 4;
  u32x4_t q[CL][R];
  uint32_t sw[CL][R];
  if (act) {
#pragma unroll
    for (int cl = 0; cl < CL; ++cl)
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int64_t row = (n0 + r < N) ? (n0 + r) : (N - 1);
        const int64_t c = lane + 64 * cl;
        q[cl][r] = load_stream(sg.codes + row * cb + c * 16);
        sw[cl][r] = *reinterpret_cast<const uint16_t*>(sg.scales + row * sbytes + c * 2);
      }
  }
  x1x_store<256, M * CL>(xl, nu, xv);
  __syncthreads();
  if (!act) return;
  const float g = *sg.gscale;
  float acc[R][M];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;
  const int ku = (int)(K >> 3);   // units per row of x
#pragma unroll
  for (int cl = 0; cl < CL; ++cl) {
    const int c = lane + 64 * cl;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      bf16x2_t wd[R][8];
      float s[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const uint32_t w0 = b ? q[cl][r].z : q[cl][r].x;
        const uint32_t w1 = b ? q[cl][r].w : q[cl][r].y;
        wd[r][0] = e2m1x2_to_bf16<0>(w0);
        wd[r][1] = e2m1x2_to_bf16<1>(w0);
        wd[r][2] = e2m1x2_to_bf16<2>(w0);
        wd[r][3] = e2m1x2_to_bf16<3>(w0);
        wd[r][4] = e2m1x2_to_bf16<0>(w1);
        wd[r][5] = e2m1x2_to_bf16<1>(w1);
        wd[r][6] = e2m1x2_to_bf16<2>(w1);
        wd[r][7] = e2m1x2_to_bf16<3>(w1);
        s[r] = b ? e4m3_to_f32<1>(sw[cl][r]) : e4m3_to_f32<0>(sw[cl][r]);
      }
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const u32x4_t xa = xl[x1x_unit(m * ku + 4 * c + 2 * b)];
        const u32x4_t xb = xl[x1x_unit(m * ku + 4 * c + 2 * b + 1)];
        const bf16x2_t xq[8] = {as_bf16x2(xa.x), as_bf16x2(xa.y), as_bf16x2(xa.z),
                                as_bf16x2(xa.w), as_bf16x2(xb.x), as_bf16x2(xb.y),
                                as_bf16x2(xb.z), as_bf16x2(xb.w)};
#pragma unroll
        for (int r = 0; r < R; ++r) {
          float p = 0.0f;
#pragma unroll
          for (int j = 0; j < 8; ++j) p = dot2(wd[r][j], xq[j], p);
          acc[r][m] = __builtin_fmaf(p, s[r], acc[r][m]);
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const float t = wave_sum(acc[r][m]);
      if (lane == r * M + m && n0 + r < N) sg.y[(int64_t)m * N + n0 + r] = t * g;
    }
}

// W4A4 at M <= 2: k_gemv's loop with NVFP4 activations read and decoded in
// place (wave_row_dots_q), and the tensor scale g_w * g_x (one fp32
// rounding), over one matrix or the segment table of several.
template <int M, int R, bool SEG>
__global__ __launch_bounds__(256) void k_gemv_w4a4(const SegTable tab,
                                                   const uint8_t* __restrict__ codes_x,
                                                   const uint8_t* __restrict__ scales_x,
                                                   const float* __restrict__ gscale_x,
                                                   int64_t K) {
  const int lane = threadIdx.x & 63;
  const int64_t wave =
      (int64_t)blockIdx.x * kWavesPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * kWavesPerBlock;
  const int64_t units = tab.start[kMaxSegments];
  const uint8_t* xc[M];
  const uint8_t* xs[M];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    xc[m] = codes_x + (int64_t)m * (K / 2);
    xs[m] = scales_x + (int64_t)m * (K / 16);
  }
  const float gx = *gscale_x;
  const float g0 = SEG ? 0.0f : *tab.gscale[0] * gx;
  for (int64_t u = wave; u < units; u += nwaves) {
    const Seg sg = SEG ? find_seg(tab, u)
                       : Seg{tab.codes[0], tab.scales[0], tab.gscale[0], tab.y[0], tab.N[0], u, 0};
    const float g = SEG ? *sg.gscale * gx : g0;
    const int64_t N = sg.N;
    const int64_t n0 = sg.unit * R;
    int64_t rows[R];
#pragma unroll
    for (int r = 0; r < R; ++r) rows[r] = (n0 + r < N) ? (n0 + r) : (N - 1);
    float acc[R][M];
    wave_row_dots_q<M, R>(sg.codes, sg.scales, K, rows, xc, xs, acc);
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int m = 0; m < M; ++m)
        if (lane == r * M + m && n0 + r < N) sg.y[(int64_t)m * N + n0 + r] = acc[r][m] * g;
  }
}

__global__ void k_fill_zero(float* y, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    y[i] = 0.0f;
}

hipError_t launch_fill_zero(float* y, size_t n, hipStream_t stream) {
  if (n) {
    const size_t want = (n + 255) / 256;
    hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)(want < 1024 ? want : 1024)), dim3(256),
                       0, stream, y, n);
  }
  return hipGetLastError();
}

// One wavefront per row group, no grid-stride reuse unless the matrix is huge:
// a launch-shape sweep on the 151936 x 4096 LM head measured 53.1 us with
// one group per wavefront against 56.1 us with the grid capped at 8
// workgroups per CU. Rows per wavefront grow with the row count so that small
// matrices still spread over every CU (1024 rows: R = 1 -> 3.5 us, R = 4 ->
// 4.6 us).
template <int M, int R>
static void launch_m(const SegDesc* d, int n, const uint16_t* x, int64_t K,
                     hipStream_t stream) {
  const SegTable tab = make_seg_table(d, n, R);
  const int64_t units = tab.start[kMaxSegments];
  const int64_t want = (units + kWavesPerBlock - 1) / kWavesPerBlock;
  const int64_t cap = (int64_t)1 << 20;
  const unsigned nblk = (unsigned)(want < cap ? want : cap);
  const unsigned grid = (nblk + 7) / 8 * 8;
  if constexpr (R <= 2) {
    if (K == 4096 && want <= cap) {
      // one row group per wavefront: the staged kernel, two chunks per lane
      const size_t lds = (size_t)M * K * sizeof(uint16_t);
      if (n == 1)
        hipLaunchKernelGGL((k_gemv_1x<M, R, 2, false>), dim3(grid), dim3(256), lds, stream, tab,
                           x, K, nblk);
      else
        hipLaunchKernelGGL((k_gemv_1x<M, R, 2, true>), dim3(grid), dim3(256), lds, stream, tab,
                           x, K, nblk);
      return;
    }
  }
  if (n == 1)
    hipLaunchKernelGGL((k_gemv<M, R, false>), dim3(grid), dim3(256), 0, stream, tab, x, K, nblk);
  else
    hipLaunchKernelGGL((k_gemv<M, R, true>), dim3(grid), dim3(256), 0, stream, tab, x, K, nblk);
}

// 3 <= M <= 5 on matrices of at most 1024 rows at K = 4096: the staged
// kernel, one row per wavefront. There the matrix-core kernel has only 64
// workgroups of 16 tiles; same-process A/B (calls queued back to back), 1024
// x 4096: M = 3 4.92 -> 3.86 us, M = 5 5.09 -> 4.51 us. At M = 8 (5.34
// against 5.52 us) and from 2048 rows (M = 5: 5.17 against 5.57 us) the
// matrix cores stay ahead.
template <int M, int R>
static void launch_staged(const SegDesc* d, int n, const uint16_t* x, int64_t K,
                          hipStream_t stream) {
  const SegTable tab = make_seg_table(d, n, R);
  const int64_t units = tab.start[kMaxSegments];
  const unsigned nblk = (unsigned)((units + kWavesPerBlock - 1) / kWavesPerBlock);
  const unsigned grid = (nblk + 7) / 8 * 8;
  const size_t lds = (size_t)M * K * sizeof(uint16_t);
  if (n == 1)
    hipLaunchKernelGGL((k_gemv_1x<M, R, 2, false>), dim3(grid), dim3(256), lds, stream, tab, x,
                       K, nblk);
  else
    hipLaunchKernelGGL((k_gemv_1x<M, R, 2, true>), dim3(grid), dim3(256), lds, stream, tab, x,
                       K, nblk);
}

template <int M>
static void launch_valu(const SegDesc* d, int n, int64_t rows, const uint16_t* x, int64_t K,
                        hipStream_t stream) {
  if (rows >= 32768)
    launch_m<M, 4>(d, n, x, K, stream);
  else if (rows >= 4096)
    launch_m<M, 2>(d, n, x, K, stream);
  else
    launch_m<M, 1>(d, n, x, K, stream);
}

hipError_t launch_gemv_segments(const SegDesc* d, int n, const uint16_t* x, int M, int64_t K,
                                hipStream_t stream) {
  if (n < 1 || n > kMaxSegments || M < 1 || M > NVFP4_MAX_M_INTERNAL) return hipErrorInvalidValue;
  int64_t rows = 0;
  for (int s = 0; s < n; ++s) rows += d[s].N;
  switch (M) {
    case 1: launch_valu<1>(d, n, rows, x, K, stream); break;
    case 2:
      // Two tokens on the matrix cores from 4096 rows (same-process A/B at
      // K = 4096 and 12288: 4096 x 4096 5.60 -> 5.09 us, 12288 x 4096
      // 10.06 -> 8.31, 4096 x 12288 12.15 -> 9.28, the 151936-row LM head
      // 78.7 -> 57.1); at 1024 rows the vector ALUs stay faster (3.95
      // against 4.63 us).
      if (rows >= kM2MatrixCoreRows &&
          (g8r_applicable(M, n, n == 1 ? d[0].N : 0, K) || g8_applicable(M, K)))
        return launch_gemv_mfma(d, n, x, M, K, stream);
      launch_valu<2>(d, n, rows, x, K, stream);
      break;
    default:
      if (M <= 5 && K == 4096 && rows <= kStagedManyRows) {
        if (M == 3) launch_staged<3, 1>(d, n, x, K, stream);
        else if (M == 4) launch_staged<4, 1>(d, n, x, K, stream);
        else launch_staged<5, 1>(d, n, x, K, stream);
        break;
      }
      if (M > NVFP4_MAX_M_SMALL && !g8_groups_applicable(d, n, M, K))
        return launch_gemv_mt(d, n, x, M, K, stream);
      return launch_gemv_mfma(d, n, x, M, K, stream);
  }
  return hipGetLastError();
}

template <int M, int R>
static void launch_w4a4_m(const SegDesc* d, int n, const uint8_t* codes_x,
                          const uint8_t* scales_x, const float* gscale_x, int64_t K,
                          hipStream_t stream) {
  const SegTable tab = make_seg_table(d, n, R);
  const int64_t units = tab.start[kMaxSegments];
  const int64_t want = (units + kWavesPerBlock - 1) / kWavesPerBlock;
  const int64_t cap = (int64_t)1 << 20;
  const unsigned grid = (unsigned)(want < cap ? want : cap);
  if (n == 1)
    hipLaunchKernelGGL((k_gemv_w4a4<M, R, false>), dim3(grid), dim3(256), 0, stream, tab,
                       codes_x, scales_x, gscale_x, K);
  else
    hipLaunchKernelGGL((k_gemv_w4a4<M, R, true>), dim3(grid), dim3(256), 0, stream, tab,
                       codes_x, scales_x, gscale_x, K);
}

template <int M>
static void launch_w4a4_valu(const SegDesc* d, int n, const uint8_t* codes_x,
                             const uint8_t* scales_x, const float* gscale_x, int64_t K,
                             hipStream_t stream) {
  int64_t rows = 0;
  for (int s = 0; s < n; ++s) rows += d[s].N;
  if (rows >= 32768)
    launch_w4a4_m<M, 4>(d, n, codes_x, scales_x, gscale_x, K, stream);
  else if (rows >= 4096)
    launch_w4a4_m<M, 2>(d, n, codes_x, scales_x, gscale_x, K, stream);
  else
    launch_w4a4_m<M, 1>(d, n, codes_x, scales_x, gscale_x, K, stream);
}

hipError_t launch_gemv_w4a4_valu(const SegDesc* d, int n, const uint8_t* codes_x,
                                 const uint8_t* scales_x, const float* gscale_x, int M,
                                 int64_t K, hipStream_t stream) {
  if (n < 1 || n > kMaxSegments) return hipErrorInvalidValue;
  switch (M) {
    case 1: launch_w4a4_valu<1>(d, n, codes_x, scales_x, gscale_x, K, stream); break;
    case 2: launch_w4a4_valu<2>(d, n, codes_x, scales_x, gscale_x, K, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gemv(const uint8_t* codes, const uint8_t* scales, const float* gscale,
                       const uint16_t* x, int M, int64_t N, int64_t K, float* y,
                       hipStream_t stream) {
  const SegDesc d = {codes, scales, gscale, y, N};
  return launch_gemv_segments(&d, 1, x, M, K, stream);
}

}  // namespace nvfp4
