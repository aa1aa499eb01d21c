// gemv_mfma.hip -- NVFP4 g16 W4A16 GEMV on the CDNA4 matrix cores, for
// 3 <= M <= 8 activation rows (the instruction has room for 16) and K not a
// multiple of 256 (multiples of 256 go to gemv_g8.hip, or to gemv_splitk.hip
// where their slices do not split evenly over 16 wavefronts).
//
// Why MFMA here: at M rows the plain VALU path spends about 0.5 + M/2
// instructions per weight (one bf16 pair dot per two weights per row), which
// at M >= 3 exceeds what the vector ALUs can issue while HBM streams 4.5-bit
// weights at full speed. v_mfma_f32_16x16x32_bf16 does all M rows at once,
// leaving the decode (about 2 instructions per weight) as the ALU cost.
//
// Operand mapping (lane l, i = l % 16, g = l / 16; verified on gfx950):
//   A (16 x 32): lane holds A[i][8g .. 8g+7]   -> x[m = i][k ...]
//   B (32 x 16): lane holds B[8g .. 8g+7][i]   -> w[n0 + i][k ...]
//   D (16 x 16): lane holds D[4g + r][i], r<4  -> y[m = 4g + r][n0 + i]
// One iteration covers 128 k of 16 rows: lane group g loads the 16 code bytes
// at byte 64t + 16g of its row (32 weights, two 16-element blocks) and feeds
// four MFMAs with 8 weights each; the A operand of MFMA q is
// x[m][128t + 32g + 8q .. +8]. The block scale is folded into B: e2m1 * s is
// exact in bf16 (at most 6 significant bits), built in fp32
// (v_cvt_scalef32_pk_f32_fp4 with scale 1.0, times s) and packed with
// v_cvt_pk_bf16_f32 (exact). The tensor scale g is applied at the store.
//
// Memory traffic: per-lane A loads straight from global memory make the L1
// (TCP) the bottleneck (every lane fetches its own 64 bytes of x per
// iteration). Instead each wavefront copies its K-slice of x, M rows by
// 512 k per chunk, into a private LDS double buffer with one contiguous
// 1 KiB global_load_lds_dwordx4 per row, and reads A with ds_read_b128. A
// rows i >= M read row i % M (same LDS address, a broadcast); their D rows
// are never stored. Codes and the chunk's 32 scale bytes per row go to
// registers one chunk ahead.
//
// A workgroup owns 16*T rows and splits the K chunks evenly across its
// wavefronts; partial D tiles are summed through LDS in wavefront order
// (deterministic).
#include "device.h"
#include "internal.h"

namespace nvfp4 {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kMfmaMaxWaves = 8;
constexpr int kChunkIters = 4;                        // 4 x 128 k = 512 k per chunk
constexpr int kXRowBytes = kChunkIters * 128 * 2;     // 1 KiB of bf16 per x row
constexpr int kXRowStride = kXRowBytes + 16;          // pad: rows start 4 banks apart
// s_waitcnt immediate (gfx9 encoding) with expcnt and lgkmcnt at their
// maxima; OR in a vmcnt below 16. Issued as the builtin so that the
// compiler's own wait insertion knows it.
constexpr int kWaitBase = (0x7 << 4) | (0xF << 8);

// bf16x8 of the 8 E2M1 codes of `word` times the scale s (exact).
__device__ __forceinline__ bf16x8_t decode8_scaled(uint32_t word, float s) {
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

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) {
  bf16x8_t r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

// Register stage of one chunk: 4 iterations of code bytes and the 32 scale
// bytes (8 per iteration) of each tile row.
template <int T>
struct Chunk {
  u32x4_t q[T][kChunkIters];
  u32x4_t s[T][2];
};

// cp/sp point at this lane's code bytes of iteration 0 (row, lane-group
// offset) and at its row's scale bytes; t_last is the last iteration whose
// codes this lane may load (its own last in-range iteration), g_sb its scale
// byte offset inside an iteration (2g, or 0 for a lane group wholly past K).
template <int T>
__device__ __forceinline__ void load_chunk_regs(Chunk<T>& ch, const uint8_t* const (&cp)[T],
                                                const uint8_t* const (&sp)[T], int64_t t0,
                                                int64_t t_last, int64_t sb, int g_sb) {
#pragma unroll
  for (int u = 0; u < T; ++u) {
#pragma unroll
    for (int j = 0; j < kChunkIters; ++j) {
      const int64_t t = t0 + j < t_last ? t0 + j : t_last;
      ch.q[u][j] = load_stream(cp[u] + t * 64);
    }
  }
  if (8 * t0 + 32 <= sb) {
    // the chunk's 32 scale bytes of each row lie inside the row
#pragma unroll
    for (int u = 0; u < T; ++u) {
      ch.s[u][0] = load_stream(sp[u] + t0 * 8);
      ch.s[u][1] = load_stream(sp[u] + t0 * 8 + 16);
    }
  } else {
    // last chunk of the row: each lane fetches only its own two bytes per
    // iteration (clamped to its last in-range iteration); s[u][0] then holds
    // those raw 16-bit values, one per iteration (see scale_bits)
#pragma unroll
    for (int u = 0; u < T; ++u) {
#pragma unroll
      for (int j = 0; j < kChunkIters; ++j) {
        const int64_t t = t0 + j < t_last ? t0 + j : t_last;
        ch.s[u][0][j] = *reinterpret_cast<const uint16_t*>(sp[u] + t * 8 + g_sb);
      }
    }
  }
}

// The lane's two scale bytes (first block in bits 7..0) for iteration j of a
// chunk: from the 32-byte image of an interior chunk, or the raw per-iteration
// values of a row's last chunk.
template <int T>
__device__ __forceinline__ uint32_t scale_bits(const Chunk<T>& ch, int u, int j, int g,
                                               bool last_chunk) {
  if (last_chunk) return ch.s[u][0][j];
  const u32x4_t sv = ch.s[u][j >> 1];
  const int sb = 8 * (j & 1) + 2 * g;
  const uint32_t sword = sb < 4 ? sv.x : sb < 8 ? sv.y : sb < 12 ? sv.z : sv.w;
  return (sword >> (8 * (sb & 3))) & 0xFFFFu;
}

// Copy x[m][k0 .. k0+512) for m < M into the LDS chunk buffer `buf` (one
// contiguous 1 KiB wavefront load per row). Lanes past the end of x read a
// clamped in-bounds address; those k are only multiplied by zero weights.
__device__ __forceinline__ void load_chunk_x(unsigned char* buf, const uint16_t* __restrict__ x,
                                             int M, int64_t K, int64_t k0, int lane) {
  int64_t k = k0 + 8 * lane;
  if (k + 8 > K) k = K - 8;
  for (int m = 0; m < M; ++m)
    __builtin_amdgcn_global_load_lds(
        x + (int64_t)m * K + k, (__attribute__((address_space(3))) void*)(buf + m * kXRowStride),
        16, 0, 0);
}

// The four MFMAs of iteration j of a chunk for every tile. `valid` is false
// only for the lane groups of a partial last iteration whose 32 k lie past K:
// they contribute zero weights.
template <int T>
__device__ __forceinline__ void compute_iter(const Chunk<T>& ch, int j, uint32_t xaddr,
                                             int g, bool valid, bool last_chunk,
                                             f32x4_t (&acc)[T]) {
  // A operands: the 64 bytes of this lane's x row at k = 128 j + 32 g of the
  // chunk. The LDS reads are issued as one asm block that waits for its own
  // results; their order after the DMA that filled the buffer comes from the
  // explicit vmcnt wait at the top of the step (the compiler does not track
  // that dependence).
  u32x4_t av[4];
  const uint32_t a = xaddr + j * 256 + 64 * g;
  asm volatile(
      "ds_read_b128 %0, %4\n"
      "ds_read_b128 %1, %4 offset:16\n"
      "ds_read_b128 %2, %4 offset:32\n"
      "ds_read_b128 %3, %4 offset:48\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(av[0]), "=&v"(av[1]), "=&v"(av[2]), "=&v"(av[3])
      : "v"(a));
#pragma unroll
  for (int u = 0; u < T; ++u) {
    const uint32_t sbits = scale_bits<T>(ch, u, j, g, last_chunk);
    const float s0 = e4m3_to_f32<0>(sbits), s1 = e4m3_to_f32<1>(sbits);
    const u32x4_t cw = valid ? ch.q[u][j] : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t word = q == 0 ? cw.x : q == 1 ? cw.y : q == 2 ? cw.z : cw.w;
      const bf16x8_t b = decode8_scaled(word, q < 2 ? s0 : s1);
      acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av[q]), b, acc[u], 0, 0, 0);
    }
  }
}

// One pipeline step: wait for chunk c (registers `cur`, x in the LDS buffer
// at byte address xread), issue x(c+1) into xload and regs(c+2) into `ld`,
// then decode and multiply chunk c.
template <int T>
__device__ __forceinline__ void mfma_step(const Chunk<T>& cur, Chunk<T>& ld, uint32_t xread,
                                          unsigned char* xload, int64_t c, int64_t nch,
                                          int64_t tb, int64_t te, int64_t t_last,
                                          int64_t t_gvalid_end, const uint8_t* const (&cp)[T],
                                          const uint8_t* const (&sp)[T], int64_t sb, int g_sb,
                                          const uint16_t* __restrict__ x, int M, int64_t K,
                                          int lane, int g, f32x4_t (&acc)[T]) {
  __builtin_amdgcn_s_waitcnt(kWaitBase | (6 * T));
  const int64_t t0 = tb + c * kChunkIters;
  if (c + 1 < nch) load_chunk_x(xload, x, M, K, (t0 + kChunkIters) * 128, lane);
  load_chunk_regs<T>(ld, cp, sp, t0 + 2 * kChunkIters, t_last, sb, g_sb);
  __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the math
#pragma unroll
  for (int j = 0; j < kChunkIters; ++j)
    if (t0 + j < te)
      compute_iter<T>(cur, j, xread, g, t0 + j < t_gvalid_end, 8 * t0 + 32 > sb, acc);
}

template <int T>
__global__ __launch_bounds__(64 * kMfmaMaxWaves) void k_gemv_mfma(
    const SegTable tab, const uint16_t* __restrict__ x, int M, int64_t K) {
  // workgroup = one unit of 16T rows of one segment
  const Seg sg = find_seg(tab, blockIdx.x);
  const uint8_t* __restrict__ codes = sg.codes;
  const uint8_t* __restrict__ scales = sg.scales;
  const float* __restrict__ gscale = sg.gscale;
  float* __restrict__ y = sg.y;
  const int64_t N = sg.N;
  // dynamic LDS: per wavefront two x chunk buffers of M rows, then the
  // cross-wavefront reduction area (W * T * 32 lanes * 4 floats)
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int lane = threadIdx.x & 63;
  // wavefront index, made provably uniform so loop control stays scalar
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int W = blockDim.x >> 6;
  const int i = lane & 15, g = lane >> 4;
  const int64_t n0 = sg.unit * (16 * T);
  const int64_t cb = K >> 1, sb = K >> 4;
  const int64_t IT = (K + 127) >> 7;
  // this wavefront's chunks of kChunkIters iterations (the last may be short)
  const int64_t nch_all = (IT + kChunkIters - 1) / kChunkIters;
  const int64_t cbeg = nch_all * w / W, cend = nch_all * (w + 1) / W;
  const int64_t tb = cbeg * kChunkIters;
  const int64_t te = cend * kChunkIters < IT ? cend * kChunkIters : IT;

  const int xbuf = M * kXRowStride;       // bytes of one chunk buffer
  unsigned char* xl0 = smem + (2 * w) * xbuf;
  unsigned char* xl1 = xl0 + xbuf;
  float* red = reinterpret_cast<float*>(smem + 2 * W * xbuf);

  // lane group g covers k >= K only in a partial last iteration (K % 128 != 0);
  // its loads are clamped to its last in-range iteration, and a group with no
  // k < K at all (K < 32 g + 32) reads the row start instead
  const int64_t t_gvalid_end = (K - 32 * g + 127) >> 7;
  const bool g_ok = 32 * g < K;
  const int64_t t_last = g_ok ? t_gvalid_end - 1 : 0;
  const int g_sb = g_ok ? 2 * g : 0;
  const uint8_t* cp[T];
  const uint8_t* sp[T];
#pragma unroll
  for (int u = 0; u < T; ++u) {
    const int64_t n = n0 + 16 * u + i;
    const int64_t row = n < N ? n : N - 1;
    cp[u] = codes + row * cb + (g_ok ? 16 * g : 0);
    sp[u] = scales + row * sb;
  }
  // LDS byte addresses of this lane's A row in the two chunk buffers
  const uint32_t xa0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)(
                           xl0 + (i % M) * kXRowStride);
  const uint32_t xa1 = xa0 + (uint32_t)xbuf;

  f32x4_t acc[T];
#pragma unroll
  for (int u = 0; u < T; ++u) acc[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int64_t nch = cend - cbeg;
  if (nch > 0) {
    // Software pipeline. Per chunk c the loads are: x(c) into an LDS buffer
    // by DMA (M loads), then the code and scale registers (6T loads, 8T for
    // a row's last chunk). The registers form a ring of three stages and are
    // fetched two chunks ahead; x uses two LDS buffers, one chunk ahead.
    // Issue order is regs(0), x(0), regs(1), then per step c:
    // x(c+1), regs(c+2). At the top of step c only regs(c+1) -- issued after
    // x(c) -- may still be outstanding, so waiting for vmcnt <= 6T completes
    // regs(c) and x(c) (memory operations retire in issue order). The LDS
    // reads are ordered after that wait explicitly: the compiler does not
    // track the DMA's writes. regs(c+2) past this wavefront's range repeat
    // clamped in-range addresses (cache hits), so the count never changes.
    Chunk<T> S0, S1, S2;
    load_chunk_regs<T>(S0, cp, sp, tb, t_last, sb, g_sb);
    load_chunk_x(xl0, x, M, K, tb * 128, lane);
    load_chunk_regs<T>(S1, cp, sp, tb + kChunkIters, t_last, sb, g_sb);
    for (int64_t c = 0;;) {
      mfma_step<T>(S0, S2, xa0, xl1, c, nch, tb, te, t_last, t_gvalid_end, cp, sp, sb, g_sb, x, M, K, lane, g, acc);
      if (++c >= nch) break;
      mfma_step<T>(S1, S0, xa1, xl0, c, nch, tb, te, t_last, t_gvalid_end, cp, sp, sb, g_sb, x, M, K, lane, g, acc);
      if (++c >= nch) break;
      mfma_step<T>(S2, S1, xa0, xl1, c, nch, tb, te, t_last, t_gvalid_end, cp, sp, sb, g_sb, x, M, K, lane, g, acc);
      if (++c >= nch) break;
      mfma_step<T>(S0, S2, xa1, xl0, c, nch, tb, te, t_last, t_gvalid_end, cp, sp, sb, g_sb, x, M, K, lane, g, acc);
      if (++c >= nch) break;
      mfma_step<T>(S1, S0, xa0, xl1, c, nch, tb, te, t_last, t_gvalid_end, cp, sp, sb, g_sb, x, M, K, lane, g, acc);
      if (++c >= nch) break;
      mfma_step<T>(S2, S1, xa1, xl0, c, nch, tb, te, t_last, t_gvalid_end, cp, sp, sb, g_sb, x, M, K, lane, g, acc);
      if (++c >= nch) break;
    }
  }

  const float gs = *gscale;
  if (W > 1) {
    if (lane < 32) {
#pragma unroll
      for (int u = 0; u < T; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[((w * T + u) * 32 + lane) * 4 + r] = acc[u][r];
    }
    __syncthreads();
    if (w != 0) return;
    if (lane < 32) {
#pragma unroll
      for (int u = 0; u < T; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float s = 0.0f;
          for (int v = 0; v < W; ++v) s += red[((v * T + u) * 32 + lane) * 4 + r];
          acc[u][r] = s;
        }
    }
  }
  // lane (i, g) holds y[4g + r][n0 + 16u + i]
#pragma unroll
  for (int u = 0; u < T; ++u) {
    const int64_t n = n0 + 16 * u + i;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = 4 * g + r;
      if (m < M && n < N) y[(int64_t)m * N + n] = acc[u][r] * gs;
    }
  }
}

// Launch shape: T row tiles per workgroup and W wavefronts splitting K.
void mfma_shape(int64_t tiles, int64_t K, int* T_out, int* W_out) {
  const int64_t chunks = ((K + 127) / 128 + kChunkIters - 1) / kChunkIters;
  const int T = 1;  // two tiles per workgroup spill registers with the 3-stage ring
  const int64_t wgs = (tiles + T - 1) / T;
  // enough wavefronts to cover the chip (about 8 per CU), at least 2 chunks
  // per wavefront
  int W = 1;
  while (W < kMfmaMaxWaves && wgs * W < 1024 && chunks / (2 * W) >= 1) W *= 2;
  *T_out = T;
  *W_out = W;
}

hipError_t launch_gemv_mfma_shape(const SegDesc* d, int n, const uint16_t* x, int M,
                                  int64_t K, int T, int W, hipStream_t stream) {
  (void)T;   // one tile per workgroup
  const SegTable tab = make_seg_table(d, n, 16);
  const int64_t wgs = tab.start[kMaxSegments];
  const size_t lds = (size_t)2 * W * M * kXRowStride + (size_t)W * 32 * 4 * sizeof(float);
  hipLaunchKernelGGL((k_gemv_mfma<1>), dim3((unsigned)wgs), dim3(64 * W), lds, stream, tab, x, M,
                     K);
  return hipGetLastError();
}

hipError_t launch_gemv_mfma(const SegDesc* d, int n, const uint16_t* x, int M, int64_t K,
                            hipStream_t stream) {
  if (g8r_applicable(M, n, n == 1 ? d[0].N : 0, K)) return launch_gemv_g8r(d[0], x, M, K, stream);
  if (g8_applicable(M, K)) return launch_gemv_g8(d, n, x, M, K, stream);
  if (splitk_applicable(M, K)) return launch_gemv_splitk(d, n, x, M, K, stream);
  int64_t tiles = 0;
  for (int s = 0; s < n; ++s) tiles += (d[s].N + 15) / 16;
  int T, W;
  mfma_shape(tiles, K, &T, &W);
  return launch_gemv_mfma_shape(d, n, x, M, K, T, W, stream);
}

}  // namespace nvfp4
