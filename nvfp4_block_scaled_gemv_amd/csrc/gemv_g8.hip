// gemv_g8.hip -- NVFP4 g16 W4A16 GEMV on the CDNA4 matrix cores for
// 2 <= M <= 8 activation rows (9 to 16 as two groups of 8) and K a multiple
// of 256:
//
//   y[m, n] = g * sum_k e2m1(c[n,k]) * e4m3(s[n, k/16]) * x[m, k]
//
// Work split. A workgroup owns TW tiles of 16 weight rows (of one segment)
// and all of K; its W wavefronts split K into ranges of S slices of 256 k.
// Every wavefront issues all of its loads at once (its part of x, then the
// weights), computes, and the W partial tiles meet once in LDS, summed
// in wavefront order (deterministic). There is no loop over tiles: workgroups
// are small and many, and the hardware dispatcher hands them to CUs as CUs
// free up, which keeps the HBM stream at the rate of a plain read.
//
// MFMA layout (v_mfma_f32_16x16x32_bf16; lane l, i = l % 16, g = l / 16: A
// lane holds A[i][8g .. 8g+7], B lane holds B[8g .. 8g+7][i], D lane holds
// D[4g + r][i]). Each MFMA multiplies two 16-element blocks of 16 weight
// rows: A rows 0..7 are the tokens with x at the first block's k (lane
// groups 0, 1) and zeros elsewhere, A rows 8..15 the tokens with x at the
// second block's k (lane groups 2, 3). So D rows 0..7 are single-block
// partials of one block and rows 8..15 of the other, and each lane scales
// its four D values by the E4M3 scale of its own block before accumulating
// in fp32; the weights enter as plain E2M1 values (exact in bf16).
//
// x in whole cache lines. A window is 64 k (4 blocks, 128 bytes of x per
// token, pieces 2b and 2b+1 of 16 bytes being block b). One 16-byte load per
// lane covers a window for all 8 tokens with every line fully used. The
// lanes that carry x in an A operand ("live": rows i < 8 in lane groups 0
// and 1, rows i >= 8 in groups 2 and 3) load token i % 8's piece g, which is
// exactly the A operand of the MFMA pairing blocks 0 and 1 once the other
// lanes are zeroed. The other lanes load piece 4 + g of the same token: that
// is what the live lane i ^ 8 of the same 16-lane row needs for the MFMA
// pairing blocks 2 and 3, so a DPP row rotation by 8 folded into the
// zeroing select builds that operand. Tokens past M lie past the bound of
// x's buffer resource and load as zeros. The weights follow the same k
// order: for the first MFMA of a window lane (n, g) feeds dword g of row
// n's 32 code bytes of the window, for the second dword 4 + g.
//
// Weights in whole cache lines. A slice of a tile is 16 rows x 128 code
// bytes; it is loaded row-major (eight rows of 128 bytes per load) and
// transposed through a small per-wavefront LDS buffer, together with its 16
// rows x 16 scale bytes. All loads are bounded buffer loads from resources
// based at the workgroup's first row: rows past N read as zeros, so no
// address is clamped.
#include "g8_ops.h"
#include "internal.h"

namespace nvfp4 {

constexpr int kG8MaxWaves = 16;
// tokens per call: groups of 8 (9..16 tokens run as two groups; past that the
// many-token kernel of gemv_mt.hip decodes each weight once for 32 tokens)
constexpr int kG8MaxTokens = 16;

// TW tiles of 16 rows per workgroup, S slices per wavefront, up to 16
// wavefronts (128 registers per lane). codes, scales and x are plain loads:
// the code is straight-line, so the compiler's waits count exactly.
// Tokens come in groups of at most 8 (M is the group size; Mt tokens in
// all, ng = ceil(Mt / 8) groups): the ng workgroups of a unit read the same
// weights for different tokens. Their workgroup indices differ by multiples
// of 8, so they are dealt to the same XCD (workgroups go to the 8 XCDs
// round robin in linear order) close together in time, and the later ones
// find the weights in that XCD's L2.
template <int M, int TW, int S>
__global__ __launch_bounds__(64 * kG8MaxWaves) __attribute__((amdgpu_waves_per_eu(S == 1 && TW <= 2 ? 8 : 1))) void k_gemv_g8(const SegTable tab,
                                                              const uint16_t* __restrict__ x,
                                                              int64_t K, int Mt, int ng,
                                                              int units) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int W = blockDim.x >> 6;
  const int i = lane & 15, g = lane >> 4;
  const int b = (int)blockIdx.x;
  const int grp = (b >> 3) % ng;                      // token group
  const int unit = (b >> 3) / ng * 8 + (b & 7);
  if (unit >= units) return;                          // the whole workgroup
  const int Mq = Mt - 8 * grp < M ? Mt - 8 * grp : M; // tokens of this group
  const Seg sg = find_seg32(tab, unit);
  const int64_t N = sg.N;
  const int64_t n0 = sg.unit * (16 * TW);
  const int64_t kw = (int64_t)w * S * kG8Slice;     // this wavefront's first k
  const int64_t cb = K >> 1, sbytes = K >> 4;
  unsigned char* const stage = lds + w * kG8StageBytes;
  f32x2_t* const red = reinterpret_cast<f32x2_t*>(lds + W * kG8StageBytes);   // [slices][TW][64]

  // ---- issue every load: x first (an L2 round trip, needed by the first
  // MFMA), then the weights slice by slice, so that the waits before slice s
  // leave the later slices in flight. Every wavefront has exactly S slices
  // (W S 256 = K) and every lane loads: the code has no branches, and the
  // scheduling barriers keep the issue order, so the compiler's wait before
  // each slice counts only the loads issued before it.
  u32x4_t q[S][TW][2];
  uint32_t sc[S][TW];
  u32x4_t xv[S][4];
  const bool live = (i < 8) == (g < 2);    // lanes of the A operands that carry x
  const int t = i & 7;
  // tokens of the group past Mq lie past the bound and read as zeros
  const __amdgpu_buffer_rsrc_t rx = buf_rsrc(x + (int64_t)8 * grp * K, (int64_t)Mq * K * 2);
  const __amdgpu_buffer_rsrc_t rc = buf_rsrc(sg.codes + n0 * cb, (N - n0) * cb);
  const __amdgpu_buffer_rsrc_t rs = buf_rsrc(sg.scales + n0 * sbytes, (N - n0) * sbytes);
  // byte offsets, 32-bit (K <= 16384 keeps every offset below 2^20), and
  // unsigned: an out-of-bound base plus a window offset stays past the bound
  // and below 2^32
  const uint32_t Ku = (uint32_t)K, cbu = (uint32_t)cb, sbu = (uint32_t)sbytes, kwu = (uint32_t)kw;
  const uint32_t xoff =
      t < M ? (t * Ku + kwu + 8u * (live ? g : 4 + g)) * 2u : (uint32_t)kBufOob;
  const int rr = lane >> 3;                          // row-major load: row rr, 16 B at 16 (l % 8)
  const uint32_t coff = rr * cbu + (kwu >> 1) + 16u * (lane & 7);
  const uint32_t soff = (lane >> 2) * sbu + (kwu >> 4) + 4u * (lane & 3);
#pragma unroll
  for (int s = 0; s < S; ++s)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      xv[s][j] = buf_load16<0>(rx, (int)(xoff + 2u * (s * kG8Slice + 64 * j)));
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int s = 0; s < S; ++s) {
#pragma unroll
    for (int u = 0; u < TW; ++u) {
      const uint32_t cu = coff + 16u * u * cbu + 128u * s;
      q[s][u][0] = buf_load16<kBufNt>(rc, (int)cu);
      q[s][u][1] = buf_load16<kBufNt>(rc, (int)(cu + 8u * cbu));
      sc[s][u] = buf_load4<0>(rs, (int)(soff + 16u * u * sbu + 16u * s));
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---- compute
  const int sh = g < 2 ? 0 : 8;
  // all ones in the live lanes, zero elsewhere: an AND, not a select, so
  // that the row rotation is never moved under a lane mask (a DPP read from
  // a lane outside the mask would not see its value) and folds into it
  // (v_and_b32 with a DPP source). The empty asm hides the value, which
  // would otherwise turn the AND back into a select.
  uint32_t keep = live ? 0xFFFFFFFFu : 0u;
  asm volatile("" : "+v"(keep));           // the lane's block: first (0) or second (8) byte
  // one partial per slice and tile: the workgroup sums the slices in slice
  // order, so the result does not depend on how K is split over wavefronts
  f32x4_t acc[S][TW];
#pragma unroll
  for (int s = 0; s < S; ++s)
#pragma unroll
    for (int u = 0; u < TW; ++u) acc[s][u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // the staged codes of row i: dwords g, g + 4, g + 8, ... of the slice row
  const uint32_t* const st_rd = reinterpret_cast<const uint32_t*>(stage + kG8Pitch * i + 4 * g);
  const u32x4_t* const st_sc = reinterpret_cast<const u32x4_t*>(stage + 16 * kG8Pitch + 16 * i);
#pragma unroll
  for (int s = 0; s < S; ++s) {
    // the A operands of the slice's 8 MFMAs (two per window): prepared once
    // per slice when several tiles share them, else window by window
    u32x4_t a[TW > 1 ? 4 : 1][2];
    auto prep = [&](int j, u32x4_t (&aj)[2]) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t v = xv[s][j][c];
        aj[0][c] = v & keep;
        aj[1][c] = g8_row_ror8(v) & keep;
      }
    };
    if constexpr (TW > 1) {
#pragma unroll
      for (int j = 0; j < 4; ++j) prep(j, a[j]);
    }
#pragma unroll
    for (int u = 0; u < TW; ++u) {
      // transpose through the stage: rows rr and rr + 8, then the scales
      *reinterpret_cast<u32x4_t*>(stage + kG8Pitch * rr + 16 * (lane & 7)) = q[s][u][0];
      *reinterpret_cast<u32x4_t*>(stage + kG8Pitch * (rr + 8) + 16 * (lane & 7)) = q[s][u][1];
      *reinterpret_cast<uint32_t*>(stage + 16 * kG8Pitch + 16 * (lane >> 2) + 4 * (lane & 3)) =
          sc[s][u];
      uint32_t b[4][2];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        b[j][0] = st_rd[8 * j];
        b[j][1] = st_rd[8 * j + 4];
      }
      const u32x4_t sv = *st_sc;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x4_t aj[2];
        if constexpr (TW > 1) {
          aj[0] = a[j][0];
          aj[1] = a[j][1];
        } else {
          prep(j, aj);
        }
        // window j's block scales: bytes 4j .. 4j + 3; the lane's first or
        // second block of each pair
        const uint32_t sw = sv[j] >> sh;
        const float s01 = e4m3_to_f32<0>(sw), s23 = e4m3_to_f32<2>(sw);
        const f32x4_t d0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            g8_bf16x8(aj[0]), g8_e2m1x8(b[j][0]), f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        const f32x4_t d1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            g8_bf16x8(aj[1]), g8_e2m1x8(b[j][1]), f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          acc[s][u][r] = __builtin_fmaf(d0[r], s01, acc[s][u][r]);
          acc[s][u][r] = __builtin_fmaf(d1[r], s23, acc[s][u][r]);
        }
      }
    }
  }

  // ---- the slice partials of every tile, summed in slice order
#pragma unroll
  for (int s = 0; s < S; ++s)
#pragma unroll
    for (int u = 0; u < TW; ++u) red[((w * S + s) * TW + u) * 64 + lane] = g8_merge_halves(acc[s][u]);
  __syncthreads();
  const float gs = *sg.gscale;
  const int slices = W * S;
  // (tile u, lane) entries dealt to the wavefronts: 64 per wavefront
  for (int e = w * 64 + lane; e < TW * 64; e += W * 64) {
    const int u = e >> 6, l = e & 63;
    f32x2_t sum = red[u * 64 + l];
    for (int v = 1; v < slices; ++v) sum += red[(v * TW + u) * 64 + l];
    const int64_t n = n0 + 16 * u + (l & 15);
    const int m0 = 4 * ((l >> 4) & 1) + (l >> 5);   // tokens m0 and m0 + 2
    if (n < N) {
      float* const yq = sg.y + (int64_t)8 * grp * N;
      if (m0 < Mq) yq[(int64_t)m0 * N + n] = sum[0] * gs;
      if (m0 + 2 < Mq) yq[(int64_t)(m0 + 2) * N + n] = sum[1] * gs;
    }
  }
}

// Whether S slices per wavefront split K evenly over at most 16 wavefronts.
static bool g8_split_ok(int64_t K, int S) {
  if (K <= 0 || (K % kG8Slice) != 0 || S < 1 || S > 4) return false;
  const int64_t slices = K / kG8Slice;
  return slices % S == 0 && slices / S <= kG8MaxWaves;
}

bool g8_applicable(int M, int64_t K) {
  if (M < 2 || M > kG8MaxTokens) return false;
  for (int s = 1; s <= 4; ++s)
    if (g8_split_ok(K, s)) return true;
  return false;
}

// 9 <= M <= 16 as two token groups, where that beats the many-token kernel
// (one decode per weight for 32 tokens): on 12288 x 4096, 4096 x 12288 and
// 4096 x 4096 (13.3 / 19.7 / 7.4 us against 15.0 / 28.8 / 13.3 at M = 9 to
// 16) but not on the 151936-row LM head (128 against 82 us), where the
// second group's reads of the weights miss the L2.
bool g8_groups_applicable(const SegDesc* d, int n, int M, int64_t K) {
  if (M <= NVFP4_MAX_M_SMALL || M > kG8MaxTokens || !g8_applicable(M, K)) return false;
  int64_t rows = 0;
  for (int k = 0; k < n; ++k) rows += d[k].N;
  return rows < 131072;
}

// Launch shape, from A/B sweeps (1024 .. 151936 rows at K = 4096 and 12288,
// M = 2, 5 and 8). S, the slices per wavefront, as small as 16 wavefronts
// allow: one slice per wavefront at K = 4096 keeps the registers at about
// 64, so each CU holds 32 wavefronts (two workgroups) where two slices per
// wavefront held 16 (LM head at M = 8: 74.7 against 85.9 us; 4096 and 1024
// rows: 5.3 against 5.8 us and 5.1 against 5.5 us). TW, the tiles per
// workgroup, with one slice per wavefront (the registers of more slices and
// tiles would not fit; one tile otherwise):
//   - 3 where the three-tile grid is one round of one workgroup per CU
//     (248 .. 256 workgroups; the three-tile kernel runs one workgroup per
//     CU): 12288 rows at M = 8, 8.8 us against 10.3 with TW = 2; 6144 rows
//     at M = 12 and 16 (two token groups), 7.6 / 7.8 us against 9.4 / 9.5;
//   - 2 from 384 tiles otherwise: a three-tile grid past one round leaves
//     most CUs idle in its last round (16384 rows at M = 8: 14.5 us with
//     TW = 3, 10.6 with TW = 2; 30000 rows 21.0 against 17.9; 24576 rows at
//     M = 5 14.7 against 13.8);
//   - 1 below 384 tiles;
//   - at M = 2 from 1280 tiles (20480 rows), one tile with two slices per
//     wavefront (8 wavefronts): 20480, 24576, 30000 and 49152 rows 11.3,
//     12.7, 14.8 and 21.7 us against 12.5, 13.3, 15.6 and 22.7 with TW = 2.
// With two token groups two tiles also won from 8192 rows up (M = 16:
// 16384 / 20480 / 24576 rows 16.8 / 20.5 / 23.8 us against 18.9 / 24.2 /
// 24.9 with TW = 3; 12288 rows 13.4 against 13.5). The summation order does
// not depend on the shape.
void g8_shape(int64_t rows, int64_t K, int M, int* TW, int* S, int* W) {
  const int64_t tiles = (rows + 15) / 16;
  int s = 0;
  for (int c = 1; c <= 4 && !s; ++c)
    if (g8_split_ok(K, c)) s = c;
  int tw;
  if (s != 1) {
    tw = 1;
  } else if (M == 2 && tiles >= 1280 && g8_split_ok(K, 2)) {
    tw = 1;
    s = 2;
  } else {
    // workgroups of the three-tile grid: one per (unit, token group)
    const int64_t g3 = (tiles + 2) / 3 * (M > 8 ? 2 : 1);
    tw = (g3 >= 248 && g3 <= 256) ? 3 : (tiles >= 384 ? 2 : 1);
  }
  *TW = tw;
  *S = s;
  *W = s ? (int)(K / kG8Slice / s) : 0;
}

hipError_t launch_gemv_g8_shape(const SegDesc* d, int n, const uint16_t* x, int M, int64_t K,
                                int TW, int S, hipStream_t stream) {
  if (M < 2 || M > kG8MaxTokens || !g8_split_ok(K, S) || n < 1 || n > kMaxSegments)
    return hipErrorInvalidValue;
  const int64_t slices = K / kG8Slice;
  const int64_t W = slices / S;
  const SegTable tab = make_seg_table(d, n, 16 * TW);
  const int64_t units = tab.start[kMaxSegments];
  const int ng = (M + 7) / 8;
  const int64_t grid = (units + 7) / 8 * 8 * ng;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  const size_t lds = (size_t)W * kG8StageBytes + (size_t)slices * TW * 64 * sizeof(f32x2_t);
#define NVFP4_G8(MM, TT, SS)                                                                 \
  hipLaunchKernelGGL((k_gemv_g8<MM, TT, SS>), dim3((unsigned)grid), dim3(64 * (unsigned)W),  \
                     lds, stream, tab, x, K, M, ng, (int)units)
#define NVFP4_G8_TS(MM)                                    \
  switch (TW * 10 + S) {                                   \
    case 11: NVFP4_G8(MM, 1, 1); break;                    \
    case 12: NVFP4_G8(MM, 1, 2); break;                    \
    case 13: NVFP4_G8(MM, 1, 3); break;                    \
    case 14: NVFP4_G8(MM, 1, 4); break;                    \
    case 21: NVFP4_G8(MM, 2, 1); break;                    \
    case 31: NVFP4_G8(MM, 3, 1); break;                    \
    default: return hipErrorInvalidValue;                  \
  }
  switch (M) {
    case 2: NVFP4_G8_TS(2); break;
    case 3: NVFP4_G8_TS(3); break;
    case 4: NVFP4_G8_TS(4); break;
    case 5: NVFP4_G8_TS(5); break;
    case 6: NVFP4_G8_TS(6); break;
    case 7: NVFP4_G8_TS(7); break;
    default: NVFP4_G8_TS(8); break;   // 8 tokens, or groups of 8
  }
#undef NVFP4_G8_TS
#undef NVFP4_G8
  return hipGetLastError();
}

hipError_t launch_gemv_g8(const SegDesc* d, int n, const uint16_t* x, int M, int64_t K,
                          hipStream_t stream) {
  int64_t rows = 0;
  for (int k = 0; k < n; ++k) rows += d[k].N;
  int TW, S, W;
  g8_shape(rows, K, M, &TW, &S, &W);
  return launch_gemv_g8_shape(d, n, x, M, K, TW, S, stream);
}

}  // namespace nvfp4
