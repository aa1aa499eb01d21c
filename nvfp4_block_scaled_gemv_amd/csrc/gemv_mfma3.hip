// gemv_mfma3.hip -- NVFP4 g16 W4A16 GEMV on the CDNA4 matrix cores for
// 3 <= M <= 8 activation rows and K a multiple of 512 (every real projection
// shape; other K use gemv_mfma.hip).
//
// Block scale on the output. In v_mfma_f32_16x16x32_bf16 lane l (i = l % 16,
// g = l / 16, the 16-lane row g) supplies B[8g .. 8g+7][i] and A[i][8g .. 8g+7]
// and receives D[4g + r][i], r < 4. Lane (i, g) loads the 16 code bytes at
// 64t + 16g of weight row n0 + i for each 128-k step t: dwords d0..d3, where
// d0, d1 are the two halves of block 2g and d2, d3 those of block 2g + 1. Two
// v_permlane16_swap per step (on d0/d1 and on d2/d3) exchange dwords between
// rows 0 and 1 and between rows 2 and 3, after which for MFMA m (taking
// dword m of every lane) rows 0 and 1 hold the two halves of block b_m and
// rows 2 and 3 those of block b_m + 4, b_m = 0, 2, 1, 3. The A operand's rows
// 0..7 are the tokens with x only in the k positions of lane rows 0 and 1
// (zero elsewhere) and rows 8..15 the tokens with x only in those of lane rows
// 2 and 3, so D rows 0..7 are the tokens' dot products over block b_m alone
// and rows 8..15 over block b_m + 4 alone: every lane multiplies its four D
// values by the E4M3 scale of its own block and accumulates in fp32. The
// weights enter the MFMA as plain E2M1 values (v_cvt_scalef32_pk_bf16_fp4 with
// scale 1, exact): one instruction per two weights and no multiply. Lanes l
// and l + 32 (the two block halves of the same outputs) are added at the end.
//
// Data movement per chunk of J steps of 128 k (the launcher uses J = 2; the
// template also builds J = 4) of a 16-row tile: codes (J x 16 bytes per lane) and the
// row's 8J scale bytes go to registers, x (M rows x 256J bytes) goes to LDS by
// global_load_lds. Both use a ring of S stages, S - 1 chunks ahead;
// x and codes of a chunk are issued together, so the in-order vmcnt wait for
// one chunk never waits for a later one. Lanes whose A is zero read a shared
// zero region.
//
// A wavefront owns T tiles of 16 rows (T = 1, 2); with T = 2 each A operand
// and x stage serve both tiles, which halves the x traffic and LDS per weight
// byte and doubles the weight streams in flight per wavefront. A workgroup
// owns those 16T rows and splits the chunks over W wavefronts; partial tiles
// are summed through LDS in wavefront order (deterministic).
#include "device.h"
#include "internal.h"

namespace nvfp4 {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

// A chunk is CK = 128 J k (J steps of 128 k, J = 2 or 4): per tile row 64J
// code bytes and 8J scale bytes; x rows of 2 CK bytes + 16 pad in LDS.
template <int J> struct Chunk {
  static constexpr int kK = 128 * J;
  static constexpr int kXRow = 2 * kK + 16;   // 16-byte pad: 4-bank shift per row
};
constexpr int kChunkAlign = 512;           // K granularity this path accepts
constexpr int kZero = 1024;                // shared zero region
constexpr int kRed = 32 * 4 * 4;           // per-wavefront, per-tile reduction slot
constexpr int kMaxWaves3 = 8;
constexpr int kLdsMax = 160 * 1024;

// s_waitcnt immediate (gfx9 encoding: vmcnt bits 3..0 and 15..14, expcnt
// 6..4, lgkmcnt 11..8) that waits for vmcnt <= n only.
constexpr int vmcnt_imm(int n) {
  return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8);
}

__device__ __forceinline__ bf16x8_t e2m1x8(uint32_t w) {
  const bf16x2_t b0 = e2m1x2_to_bf16<0>(w);
  const bf16x2_t b1 = e2m1x2_to_bf16<1>(w);
  const bf16x2_t b2 = e2m1x2_to_bf16<2>(w);
  const bf16x2_t b3 = e2m1x2_to_bf16<3>(w);
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

template <int T, int J>
struct Regs {
  u32x4_t q[T][J];       // code bytes of the J steps of 128 k, per tile
  u32x4_t s[T][J / 2];   // the row's 8J scale bytes of the chunk, per tile
};

}  // namespace

template <int M, int S, int T, int J>
struct Mfma3 {
  static constexpr int kXStage = M * Chunk<J>::kXRow;
  static constexpr int kIssue = (J + J / 2) * T + M;    // VMEM instructions per chunk
  static_assert((S - 2) * kIssue <= 63, "vmcnt is a 6-bit counter");

  const uint8_t* cp[T];   // this lane's code bytes of chunk 0, per tile
  const uint8_t* sp[T];   // this lane's row scales of chunk 0, per tile
  const uint16_t* xs;     // this lane's x slot of chunk 0, token 0
  int64_t K;
  unsigned char* xring;   // this wavefront's S x stages

  // The register loads are asm so that the compiler's wait insertion does not
  // track them: across the ring's loop back-edge it loses their position and
  // would wait for every outstanding load. Their results are used only after
  // the explicit vmcnt wait of the step that consumes them, and every issued
  // load is consumed (none is left in flight for the compiler to reuse its
  // registers).
  __device__ __forceinline__ void issue(int64_t c, int st, Regs<T, J>& R) const {
#pragma unroll
    for (int u = 0; u < T; ++u) {
      const uint8_t* a = cp[u] + c * (64 * J);
      const uint8_t* b = sp[u] + c * (8 * J);
      if constexpr (J == 4) {
        asm volatile(
            "global_load_dwordx4 %0, %6, off nt\n"
            "global_load_dwordx4 %1, %6, off offset:64 nt\n"
            "global_load_dwordx4 %2, %6, off offset:128 nt\n"
            "global_load_dwordx4 %3, %6, off offset:192 nt\n"
            "global_load_dwordx4 %4, %7, off nt\n"
            "global_load_dwordx4 %5, %7, off offset:16 nt"
            : "=&v"(R.q[u][0]), "=&v"(R.q[u][J > 1 ? 1 : 0]), "=&v"(R.q[u][J > 2 ? 2 : 0]),
              "=&v"(R.q[u][J > 3 ? 3 : 0]), "=&v"(R.s[u][0]), "=&v"(R.s[u][J > 2 ? 1 : 0])
            : "v"(a), "v"(b)
            : "memory");
      } else {
        asm volatile(
            "global_load_dwordx4 %0, %3, off nt\n"
            "global_load_dwordx4 %1, %3, off offset:64 nt\n"
            "global_load_dwordx4 %2, %4, off nt"
            : "=&v"(R.q[u][0]), "=&v"(R.q[u][J > 1 ? 1 : 0]), "=&v"(R.s[u][0])
            : "v"(a), "v"(b)
            : "memory");
      }
    }
    // one 16-byte copy per lane and token row; a 256-k chunk row (512
    // bytes) needs lanes 0..31 only
    unsigned char* xb = xring + st * kXStage;
#pragma unroll
    for (int m = 0; m < M; ++m)
      if (J == 4 || (threadIdx.x & 63) < 32)
        __builtin_amdgcn_global_load_lds(xs + (int64_t)m * K + c * Chunk<J>::kK,
                                         LDS_PTR(xb + m * Chunk<J>::kXRow), 16, 0, 0);
  }
};

// The A operands of one 128-k step: for MFMA m the 16 bytes at LDS byte
// address a + 32 b_m (b_m = 0, 2, 1, 3). Issued as one asm block that waits
// for its own results: the compiler neither sees these reads (it would
// otherwise wait for every outstanding global_load_lds first) nor can move
// them above the ring's explicit wait.
__device__ __forceinline__ void lds_read_a(uint32_t a, u32x4_t (&v)[4]) {
  asm volatile(
      "ds_read_b128 %0, %4\n"
      "ds_read_b128 %1, %4 offset:64\n"
      "ds_read_b128 %2, %4 offset:32\n"
      "ds_read_b128 %3, %4 offset:96\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
      : "v"(a));
}

template <int M, int S, int T, int J>
__device__ __forceinline__ void mfma3_compute(const Regs<T, J>& R, uint32_t xa, int g,
                                              f32x4_t (&acc)[T]) {
  // a bitwise select: a plain ?: on two array elements becomes a dynamically
  // indexed (scratch) load
  const uint32_t hmask = g >= 2 ? 0xFFFFFFFFu : 0u;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    u32x4_t av[4];
    lds_read_a(xa + 256 * j, av);
#pragma unroll
    for (int u = 0; u < T; ++u) {
      // scale of block b_m (+ 4 in lane rows 2, 3) of step j: byte b_m of
      // dword 2j + g / 2 of the row's 32 chunk scale bytes
      const u32x4_t sv = R.s[u][j >> 1];
      const uint32_t lo = (j & 1) ? sv.z : sv.x;
      const uint32_t hi = (j & 1) ? sv.w : sv.y;
      const uint32_t sj = (lo & ~hmask) | (hi & hmask);
      const auto p01 = __builtin_amdgcn_permlane16_swap(R.q[u][j].x, R.q[u][j].y, false, false);
      const auto p23 = __builtin_amdgcn_permlane16_swap(R.q[u][j].z, R.q[u][j].w, false, false);
      const uint32_t word[4] = {p01[0], p01[1], p23[0], p23[1]};
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const f32x4_t d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            as_bf16x8(av[m]), e2m1x8(word[m]), f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        // b_m = 0, 2, 1, 3 for m = 0..3
        const float sc = m == 0 ? e4m3_to_f32<0>(sj) : m == 1 ? e4m3_to_f32<2>(sj)
                       : m == 2 ? e4m3_to_f32<1>(sj) : e4m3_to_f32<3>(sj);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[u][r] = __builtin_fmaf(d[r], sc, acc[u][r]);
      }
    }
  }
}

// One ring step for chunk c held in stage U (registers `cur`, x stage U):
// wait until it has landed, issue chunk c + S - 1 into the stage chunk c - 1
// used (registers `nxt`), then multiply chunk c. The empty asm statements
// with a memory clobber keep the compiler from moving the loads across the
// wait or into the math.
template <int M, int S, int T, int J, int U>
__device__ __forceinline__ void mfma3_step(const Mfma3<M, S, T, J>& eng, const Regs<T, J>& cur,
                                           Regs<T, J>& nxt, int c, int nch, uint32_t xoff,
                                           bool xlive, int g, f32x4_t (&acc)[T]) {
  using G = Mfma3<M, S, T, J>;
  // Chunks c+1 .. min(c+S-2, nch-1) may still be in flight; chunk c has
  // landed once no more than those are outstanding. Only chunks that exist
  // are ever issued: the register loads are invisible to the compiler, so a
  // load whose result nobody consumes could land in a register the compiler
  // has since given to another value.
  if (c + S - 2 < nch)
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((S - 2) * G::kIssue));
  else
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  asm volatile("" ::: "memory");
  constexpr int un = (U + S - 1) % S;
  if (c + S - 1 < nch) eng.issue(c + S - 1, un, nxt);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  mfma3_compute<M, S, T, J>(cur, xoff + (xlive ? U * G::kXStage : 0u), g, acc);
}

// codes, scales and x are deliberately not __restrict__: read-only noalias
// pointers would let the compiler treat their memory as invariant and sink the
// prefetch loads past the ring's ordering points.
template <int M, int S, int T, int J>
__global__ __launch_bounds__(64 * kMaxWaves3) void k_gemv_mfma3(const SegTable tab,
                                                                const uint16_t* x, int64_t K) {
  using G = Mfma3<M, S, T, J>;
  constexpr int CK = Chunk<J>::kK;
  // workgroup = one unit of 16T rows of one segment
  const Seg sg = find_seg(tab, blockIdx.x);
  const uint8_t* codes = sg.codes;
  const uint8_t* scales = sg.scales;
  const float* __restrict__ gscale = sg.gscale;
  float* __restrict__ y = sg.y;
  const int64_t N = sg.N;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int W = blockDim.x >> 6;
  const int i = lane & 15, g = lane >> 4;
  const int64_t n0 = sg.unit * (16 * T);
  const int64_t nch_all = K / CK;
  const int64_t cbeg = nch_all * w / W;
  const int nch = (int)(nch_all * (w + 1) / W - cbeg);

  if (threadIdx.x < kZero / 16)
    *reinterpret_cast<uint4*>(smem + 16 * threadIdx.x) = make_uint4(0u, 0u, 0u, 0u);
  __syncthreads();

  G eng;
#pragma unroll
  for (int u = 0; u < T; ++u) {
    const int64_t n = n0 + 16 * u + i;
    const int64_t row = n < N ? n : N - 1;
    eng.cp[u] = codes + row * (K >> 1) + 16 * g + cbeg * (64 * J);
    eng.sp[u] = scales + row * (K >> 4) + cbeg * (8 * J);
  }
  // x copies: lane L moves the 8 elements at k = 8L of the chunk
  eng.xs = x + 8 * lane + cbeg * CK;
  eng.K = K;
  eng.xring = smem + kZero + (size_t)w * S * G::kXStage;
  float* red = reinterpret_cast<float*>(smem + kZero + (size_t)W * S * G::kXStage);

  // LDS byte address of this lane's A operand: token i % 8 when its half
  // (i < 8) matches the lane row's block half (g < 2), at k offset
  // 64 (g / 2) + 8 (g % 2) of the 128-k step; else the zero region
  const bool xlive = ((i < 8) == (g < 2)) && (i & 7) < M;
  const uint32_t xoff =
      (xlive ? (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)(
                   eng.xring + (i & 7) * Chunk<J>::kXRow)
             : 0u) +
      128 * (g >> 1) + 16 * (g & 1);

  f32x4_t acc[T];
#pragma unroll
  for (int u = 0; u < T; ++u) acc[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  if (nch > 0) {
    Regs<T, J> R0, R1, R2, R3;
    // prologue: chunks 0 .. min(S-1, nch)-1
    eng.issue(0, 0, R0);
    if (1 < nch) eng.issue(1, 1, R1);
    if (S == 4 && 2 < nch) eng.issue(2, 2, R2);
    asm volatile("" ::: "memory");
    if (S == 3) {
      for (int c = 0;;) {
        mfma3_step<M, S, T, J, 0>(eng, R0, R2, c, nch, xoff, xlive, g, acc);
        if (++c >= nch) break;
        mfma3_step<M, S, T, J, 1>(eng, R1, R0, c, nch, xoff, xlive, g, acc);
        if (++c >= nch) break;
        mfma3_step<M, S, T, J, 2>(eng, R2, R1, c, nch, xoff, xlive, g, acc);
        if (++c >= nch) break;
      }
    } else {
      for (int c = 0;;) {
        mfma3_step<M, S, T, J, 0>(eng, R0, R3, c, nch, xoff, xlive, g, acc);
        if (++c >= nch) break;
        mfma3_step<M, S, T, J, 1>(eng, R1, R0, c, nch, xoff, xlive, g, acc);
        if (++c >= nch) break;
        mfma3_step<M, S, T, J, 2>(eng, R2, R1, c, nch, xoff, xlive, g, acc);
        if (++c >= nch) break;
        mfma3_step<M, S, T, J, 3>(eng, R3, R2, c, nch, xoff, xlive, g, acc);
        if (++c >= nch) break;
      }
    }
  }

  // lanes l and l + 32 hold the two block halves of the same outputs
#pragma unroll
  for (int u = 0; u < T; ++u)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[u][r] += __shfl_xor(acc[u][r], 32, 64);
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
  // lane (i, g < 2) holds y[4g + r][n0 + 16u + i]
  if (lane < 32) {
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
}

// Bytes of dynamic LDS for W wavefronts with S ring stages, T tiles and
// chunks of J steps.
static size_t mfma3_lds(int M, int W, int S, int T, int J) {
  const size_t xrow = (size_t)(256 * J + 16);
  return (size_t)kZero + (size_t)W * ((size_t)S * M * xrow + (size_t)T * kRed);
}

bool mfma3_applicable(int M, int64_t K) {
  return M >= 3 && M <= 8 && K > 0 && (K % kChunkAlign) == 0;
}

// Launch shape (from a sweep of J, T, S and W on the decode-layer and stress
// shapes): 256-k chunks (a smaller x ring in LDS lets more wavefronts in
// flight), one tile per wavefront with a ring of 4 (two tiles with a ring of 3
// once there are at least 1024 tiles of 16 rows), and W wavefronts per unit so
// that about 768 run (three per CU), within the chunk count and the LDS
// budget. `units16` is the number of 16-row tiles over all segments.
void mfma3_shape(int M, int64_t units16, int64_t K, int* W_out, int* S_out, int* T_out,
                 int* J_out) {
  const int J = 2;
  const int64_t chunks = K / (128 * J);
  const int T = units16 >= 1024 ? 2 : 1;
  const int S = T == 2 ? 3 : 4;
  const int64_t units = (units16 + T - 1) / T;
  int64_t want = (768 + units - 1) / units;
  if (want > kMaxWaves3) want = kMaxWaves3;
  if (want > chunks) want = chunks;
  int W = (int)(want < 1 ? 1 : want);
  while (W > 1 && mfma3_lds(M, W, S, T, J) > (size_t)kLdsMax) --W;
  *W_out = W;
  *S_out = S;
  *T_out = T;
  *J_out = J;
}

hipError_t launch_gemv_mfma3_shape(const SegDesc* d, int n, const uint16_t* x, int M,
                                   int64_t K, int W, int S, int T, int J, hipStream_t stream) {
  // (S = 4 with T = 2 would not fit the register file)
  if (!mfma3_applicable(M, K) || n < 1 || n > kMaxSegments || W < 1 || W > kMaxWaves3 ||
      S < 3 || S > 4 || T < 1 || T > 2 || (S == 4 && T == 2) || J != 2 ||
      mfma3_lds(M, W, S, T, J) > (size_t)kLdsMax)
    return hipErrorInvalidValue;
  const size_t lds = mfma3_lds(M, W, S, T, J);
  const SegTable tab = make_seg_table(d, n, 16 * T);
  const unsigned grid = (unsigned)tab.start[kMaxSegments];
#define NVFP4_L3(MM, SS, TT, JJ)                                                             \
  hipLaunchKernelGGL((k_gemv_mfma3<MM, SS, TT, JJ>), dim3(grid), dim3(64 * W), lds, stream, \
                     tab, x, K)
#define NVFP4_L3J(MM, SS, TT) NVFP4_L3(MM, SS, TT, 2)
#define NVFP4_L3M(MM)                              \
  if (S == 4) {                                    \
    NVFP4_L3J(MM, 4, 1);                           \
  } else if (T == 1) {                             \
    NVFP4_L3J(MM, 3, 1);                           \
  } else {                                         \
    NVFP4_L3J(MM, 3, 2);                           \
  }
  switch (M) {
    case 3: NVFP4_L3M(3); break;
    case 4: NVFP4_L3M(4); break;
    case 5: NVFP4_L3M(5); break;
    case 6: NVFP4_L3M(6); break;
    case 7: NVFP4_L3M(7); break;
    default: NVFP4_L3M(8); break;
  }
#undef NVFP4_L3M
#undef NVFP4_L3J
#undef NVFP4_L3
  return hipGetLastError();
}

hipError_t launch_gemv_mfma3(const SegDesc* d, int n, const uint16_t* x, int M, int64_t K,
                             hipStream_t stream) {
  int64_t units16 = 0;
  for (int s = 0; s < n; ++s) units16 += (d[s].N + 15) / 16;
  int W, S, T, J;
  mfma3_shape(M, units16, K, &W, &S, &T, &J);
  return launch_gemv_mfma3_shape(d, n, x, M, K, W, S, T, J, stream);
}

}  // namespace nvfp4
