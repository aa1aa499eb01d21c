// gemv_g8r.hip -- NVFP4 g16 W4A16 GEMV on the CDNA4 matrix cores for
// 2 <= M <= 8 activation rows and very tall matrices (an LM head: 2^17 rows
// and more, K a multiple of 256 up to 4096, one matrix per call):
//
//   y[m, n] = g * sum_k e2m1(c[n,k]) * e4m3(s[n, k/16]) * x[m, k]
//
// Why a second eight-token kernel. In gemv_g8.hip a workgroup covers all of
// K for one to three 16-row tiles, so each workgroup reads all of x (8
// tokens x K bf16: 64 KB at K = 4096) for 32 or 48 rows of weights (72 or
// 108 KB). Its L1 then sees about as many x requests (L2 hits) as weight
// requests, and on the 151936 x 4096 LM head the address unit waits on the
// cache for about 40 % of the kernel; the time grows with the token count
// (M = 3, 5, 8: 64, 67, 73 us), as the x lanes of tokens past M load
// nothing.
//
// Here the wavefronts split the rows instead. A workgroup of 16 wavefronts
// fills LDS once with x, already in the per-lane arrangement of the A
// operands of gemv_g8.hip (window w, lane l: token (l % 16) % 8's 16-byte
// piece g or 4 + g of the window, g = l / 16), and every wavefront streams
// its own rows over all of K: two or three whole 16-row tiles (the T tiles
// of the matrix dealt out evenly, wavefront v taking tiles [v T / W,
// (v + 1) T / W) of W), the weights of the next two slices in flight. The
// grid is 256 workgroups (one per CU: x takes 64 KB of LDS) as long as three
// tiles per wavefront cover N. Whole tiles matter: with rows dealt out
// evenly instead (37 or 38 per wavefront on the LM head) every wavefront ran
// three tiles' matrix-core and decode work for 2.3 tiles of rows (63.2 ->
// 59.9 us at M = 8). A wavefront owns its rows' sums over all of K: no
// cross-wavefront reduction, and the summation order (window by window, then
// the two blocks' halves) does not depend on the grid.
//
// Per slice and tile the work is that of gemv_g8.hip: the codes are loaded
// row-major (eight 128-byte rows per load) and transposed through a small
// per-wavefront LDS stage with the scales; two MFMAs per 64-k window pair
// blocks (0, 1) and (2, 3), whose D halves are scaled by the lanes' own block
// scales. The A operands of a slice are read from the x image once and
// serve every tile of the wavefront: a live lane (one whose token piece
// belongs to its half of the MFMA, see gemv_g8.hip) reads its own entry and
// its row partner's (lane ^ 8) under the live mask, and the other lanes keep
// zeros, which replaces the AND and DPP rotation of gemv_g8.hip (32 vector
// instructions per slice).
#include "g8_ops.h"
#include "internal.h"

namespace nvfp4 {

namespace {

constexpr int kRWaves = 16;      // wavefronts per workgroup
constexpr int kRTiles = 3;       // 16-row tiles per wavefront at most
constexpr int kRMaxK = 4096;     // the x image of 8 tokens fills 64 KB of LDS
constexpr int kRGrid = 256;      // one workgroup per CU
constexpr int64_t kRMinRows = 131072;   // from here every wavefront has 2 or 3 tiles
// per wavefront: the code stage (16 rows, 144-byte pitch), then the scale
// area of its tiles (16 rows x 16 bytes each)
constexpr int kRStage = 16 * kG8Pitch + kRTiles * 256;

}  // namespace

// The weights of NT tiles of 16 rows, rows [R0, R1), streamed by one
// wavefront, two slices in flight (a ring of two register sets). Stores the x
// image that xf holds and meets the workgroup once.
template <int M, int NT>
__device__ __forceinline__ void g8r_stream(const uint8_t* __restrict__ codes,
                                           const uint8_t* __restrict__ scales,
                                           const float* __restrict__ gscale,
                                           float* __restrict__ y, int64_t N, int64_t K,
                                           int64_t R0, int64_t R1, unsigned char* lds,
                                           const u32x4_t (&xf)[kRMaxK / 1024]) {
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i = lane & 15, g = lane >> 4;
  const int S = (int)(K / kG8Slice);
  const int nwin = (int)(K / 64);
  const uint32_t cbu = (uint32_t)(K >> 1), sbu = (uint32_t)(K >> 4);
  unsigned char* const ximg = lds;                                   // [nwin][64][16 B]
  unsigned char* const stage = lds + (size_t)nwin * 1024 + w * kRStage;

  // per tile: bounded resources from the tile's first row (rows past R1 read
  // as zeros), row-major code offsets and the lane's scale offset
  __amdgpu_buffer_rsrc_t rc[NT], rs[NT];
#pragma unroll
  for (int u = 0; u < NT; ++u) {
    const int64_t b = R0 + 16 * u;
    const int64_t nr = R1 - b > 0 ? R1 - b : 0;
    rc[u] = buf_rsrc(codes + b * (int64_t)cbu, nr * (int64_t)cbu);
    rs[u] = buf_rsrc(scales + b * (int64_t)sbu, nr * (int64_t)sbu);
  }
  const int rr = lane >> 3;
  const uint32_t coff = rr * cbu + 16u * (lane & 7);
  // The scales come two slices at a time: one 8-byte load per lane and
  // tile (row l / 4, bytes 8 (l % 4) of the row's 32 for slices 2q, 2q + 1),
  // 16 lines for 512 bytes, where a 4-byte load per slice touched 16 lines
  // for 256. At the start of each slice the lanes holding that slice write
  // its 16 bytes per row for all tiles into the wavefront's scale area, which
  // frees the group's registers for the next group one slice ahead. The
  // area holds a row's even blocks in its first 8 bytes and the odd blocks in
  // the next 8, so that a lane reads exactly the scales of its half of each
  // MFMA (blocks 4j, 4j + 2 or 4j + 1, 4j + 3 of window j) at fixed bytes.
  const uint32_t soff = (lane >> 2) * sbu + 8u * (lane & 3);
  u32x4_t rq[2][NT][2];
  uint2 grp[NT];
  // codes of slice s into ring slot p; past the last slice every lane reads zeros
  auto issue_codes = [&](int s, int p) {
    const bool ok = s < S;
#pragma unroll
    for (int u = 0; u < NT; ++u) {
      const uint32_t c0 = ok ? coff + 128u * (uint32_t)s : (uint32_t)kBufOob;
      const uint32_t c1 = ok ? coff + 8u * cbu + 128u * (uint32_t)s : (uint32_t)kBufOob;
      rq[p][u][0] = buf_load16<kBufNt>(rc[u], (int)c0);
      rq[p][u][1] = buf_load16<kBufNt>(rc[u], (int)c1);
    }
  };
  // the scales of slices s, s + 1 (s even)
  auto issue_scales = [&](int s) {
    const bool ok = s < S;
#pragma unroll
    for (int u = 0; u < NT; ++u)
      grp[u] = __builtin_bit_cast(
          uint2, __builtin_amdgcn_raw_buffer_load_b64(
                     rs[u], ok ? (int)(soff + 16u * (uint32_t)s) : kBufOob, 0, 0));
  };
  // in a fixed order (the waits in the loop count loads in issue order, and
  // the first pass must match the later ones)
  issue_scales(0);
  __builtin_amdgcn_sched_barrier(0);
  issue_codes(0, 0);
  __builtin_amdgcn_sched_barrier(0);
  issue_codes(1, 1);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int k = 0; k < kRMaxK / 1024; ++k) {
    const int e = (int)threadIdx.x + 1024 * k;
    if (e < nwin * 64) *reinterpret_cast<u32x4_t*>(ximg + (size_t)e * 16) = xf[k];
  }
  __syncthreads();
  if (R0 >= R1) return;   // no rows (past the end of the matrix)

  // ---- stream the slices
  const bool live = (i < 8) == (g < 2);
  // A operands: live lanes read their own entry of a window and their row
  // partner's (lane ^ 8); dead lanes keep the zeros set here
  u32x4_t a[4][2];
#pragma unroll
  for (int j = 0; j < 4; ++j) a[j][0] = a[j][1] = u32x4_t{0u, 0u, 0u, 0u};
  const unsigned char* const xa1 = ximg + lane * 16;
  const unsigned char* const xa2 = ximg + (lane ^ 8) * 16;
  const int sh = g < 2 ? 0 : 8;    // the lane's blocks: even (byte offset 0) or odd (8)
  const uint32_t* const st_rd = reinterpret_cast<const uint32_t*>(stage + kG8Pitch * i + 4 * g);
  // the wavefront's scale area: [tile][16 rows][16 bytes] of the current slice
  unsigned char* const sca = stage + 16 * kG8Pitch;
  f32x4_t acc[NT];
#pragma unroll
  for (int u = 0; u < NT; ++u) acc[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int s0 = 0; s0 < S; s0 += 2) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int s = s0 + p;
      if (s < S) {
        // this slice's scales of every tile into the scale area (the lanes
        // holding it: bytes 8 (l % 2) of row l / 4's 16); after the second
        // slice of a group, the next group's loads
        if (p == 0) {
          // even blocks to the low word, odd blocks to the high word
#pragma unroll
          for (int u = 0; u < NT; ++u)
            grp[u] = uint2{__builtin_amdgcn_perm(grp[u].y, grp[u].x, 0x06040200u),
                           __builtin_amdgcn_perm(grp[u].y, grp[u].x, 0x07050301u)};
        }
        if (((lane >> 1) & 1) == p) {
#pragma unroll
          for (int u = 0; u < NT; ++u) {
            unsigned char* const r = sca + 256 * u + 16 * (lane >> 2) + 4 * (lane & 1);
            *reinterpret_cast<uint32_t*>(r) = grp[u].x;
            *reinterpret_cast<uint32_t*>(r + 8) = grp[u].y;
          }
        }
        if (p == 1) {
          __builtin_amdgcn_sched_barrier(0);
          issue_scales(s + 1);
          __builtin_amdgcn_sched_barrier(0);
        }
        // the A operands of the slice's 8 MFMAs, from the x image
        if (live) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            a[j][0] = *reinterpret_cast<const u32x4_t*>(xa1 + (size_t)(4 * s + j) * 1024);
            a[j][1] = *reinterpret_cast<const u32x4_t*>(xa2 + (size_t)(4 * s + j) * 1024);
          }
        }
#pragma unroll
        for (int u = 0; u < NT; ++u) {
          *reinterpret_cast<u32x4_t*>(stage + kG8Pitch * rr + 16 * (lane & 7)) = rq[p][u][0];
          *reinterpret_cast<u32x4_t*>(stage + kG8Pitch * (rr + 8) + 16 * (lane & 7)) =
              rq[p][u][1];
          uint32_t b[4][2];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            b[j][0] = st_rd[8 * j];
            b[j][1] = st_rd[8 * j + 4];
          }
          const uint2 sv = *reinterpret_cast<const uint2*>(sca + 256 * u + 16 * i + sh);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t sw = j < 2 ? sv.x : sv.y;
            const float s01 = (j & 1) ? e4m3_to_f32<2>(sw) : e4m3_to_f32<0>(sw);
            const float s23 = (j & 1) ? e4m3_to_f32<3>(sw) : e4m3_to_f32<1>(sw);
            const f32x4_t d0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                g8_bf16x8(a[j][0]), g8_e2m1x8(b[j][0]), f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
            const f32x4_t d1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                g8_bf16x8(a[j][1]), g8_e2m1x8(b[j][1]), f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              acc[u][r] = __builtin_fmaf(d0[r], s01, acc[u][r]);
              acc[u][r] = __builtin_fmaf(d1[r], s23, acc[u][r]);
            }
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      issue_codes(s + 2, p);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---- the two blocks' halves merged, scaled by g, stored
  const float gs = *gscale;
  const int m0 = 4 * ((lane >> 4) & 1) + (lane >> 5);   // tokens m0 and m0 + 2
#pragma unroll
  for (int u = 0; u < NT; ++u) {
    const f32x2_t v = g8_merge_halves(acc[u]);
    const int64_t n = R0 + 16 * u + (lane & 15);
    if (n < R1) {
      if (m0 < M) y[(int64_t)m0 * N + n] = v[0] * gs;
      if (m0 + 2 < M) y[(int64_t)(m0 + 2) * N + n] = v[1] * gs;
    }
  }
}

template <int M>
__global__ __launch_bounds__(64 * kRWaves) void k_gemv_g8r(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    const float* __restrict__ gscale, const uint16_t* __restrict__ x, float* __restrict__ y,
    int64_t N, int64_t K, int64_t T) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nwin = (int)(K / 64);
  const uint32_t Ku = (uint32_t)K;

  // ---- this wavefront's tiles [T0, T1) of the T in the matrix (two or
  // three: whole tiles, dealt out evenly), rows [R0, R1)
  const int64_t W = (int64_t)gridDim.x * kRWaves;
  const int64_t gw = (int64_t)blockIdx.x * kRWaves + w;
  const int64_t T0 = gw * T / W, T1 = (gw + 1) * T / W;
  const int64_t R0 = 16 * T0 < N ? 16 * T0 : N;
  const int64_t R1 = 16 * T1 < N ? 16 * T1 : N;

  // ---- issue the x image loads (an L2 round trip, needed first); the
  // stream issues the weights of the first two slices, then stores the image
  // and meets the workgroup once.
  const __amdgpu_buffer_rsrc_t rx = buf_rsrc(x, (int64_t)M * K * 2);
  u32x4_t xf[kRMaxK / 1024];
#pragma unroll
  for (int k = 0; k < kRMaxK / 1024; ++k) {
    const int e = (int)threadIdx.x + 1024 * k;   // (window, lane) entry
    const int l = e & 63, li = l & 15, lg = l >> 4, t = li & 7;
    const bool lv = (li < 8) == (lg < 2);
    const uint32_t off = (e < nwin * 64 && t < M)
                             ? (t * Ku + 64u * (uint32_t)(e >> 6) + 8u * (lv ? lg : 4 + lg)) * 2u
                             : (uint32_t)kBufOob;
    xf[k] = buf_load16<0>(rx, (int)off);
  }
  __builtin_amdgcn_sched_barrier(0);
  if (T1 - T0 >= 3)
    g8r_stream<M, 3>(codes, scales, gscale, y, N, K, R0, R1, lds, xf);
  else
    g8r_stream<M, 2>(codes, scales, gscale, y, N, K, R0, R1, lds, xf);
}

bool g8r_applicable(int M, int n, int64_t N, int64_t K) {
  return M >= 2 && M <= NVFP4_MAX_M_SMALL && n == 1 && N >= kRMinRows && K > 0 &&
         K % kG8Slice == 0 && K <= kRMaxK;
}

hipError_t launch_gemv_g8r(const SegDesc& d, const uint16_t* x, int M, int64_t K,
                           hipStream_t stream) {
  if (!g8r_applicable(M, 1, d.N, K)) return hipErrorInvalidValue;
  // 256 workgroups while three tiles per wavefront cover N, more beyond
  const int64_t T = (d.N + 15) / 16;
  int64_t grid = (T + (int64_t)kRWaves * kRTiles - 1) / ((int64_t)kRWaves * kRTiles);
  if (grid < kRGrid) grid = kRGrid;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  const size_t lds = (size_t)(K / 64) * 1024 + (size_t)kRWaves * kRStage;
#define NVFP4_G8R(MM)                                                                          \
  hipLaunchKernelGGL((k_gemv_g8r<MM>), dim3((unsigned)grid), dim3(64 * kRWaves), lds, stream, \
                     d.codes, d.scales, d.gscale, x, d.y, d.N, K, T)
  switch (M) {
    case 2: NVFP4_G8R(2); break;
    case 3: NVFP4_G8R(3); break;
    case 4: NVFP4_G8R(4); break;
    case 5: NVFP4_G8R(5); break;
    case 6: NVFP4_G8R(6); break;
    case 7: NVFP4_G8R(7); break;
    default: NVFP4_G8R(8); break;
  }
#undef NVFP4_G8R
  return hipGetLastError();
}

}  // namespace nvfp4
