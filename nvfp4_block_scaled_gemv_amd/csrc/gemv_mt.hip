// gemv_mt.hip -- NVFP4 g16 W4A16 GEMV on the CDNA4 matrix cores for
// 9 <= M <= 128 activation rows (many tokens: the blueprint's "multi_seq"
// plan arm takes 2 to 128 rows, and its planner settings enable the tensor
// cores for W4A16, "w4a16_tc=on").
//
//   y[m, n] = g * sum_k e2m1(c[n,k]) * e4m3(s[n, k/16]) * x[m, k]
//
// Why a kernel of its own. The M <= 8 kernels put two 16-element blocks
// side by side in one MFMA (eight tokens per block half) and scale the
// output by the block scale. With more tokens every A row is a token: the
// E4M3 block scale is folded into the weights instead (e2m1 * s has at most
// 6 significant bits in [2^-10, 2688], so it is exact in bf16) and every
// group of 32 tokens adds one v_mfma_f32_32x32x16_bf16 per decoded weight
// fragment with no per-block work. The decode (about two instructions per
// weight) is the vector-ALU cost; a wavefront decodes its weights once for
// all the token groups it holds.
//
// Work split. A workgroup owns R row tiles of 32 rows (one per "row
// wavefront") of one segment and G <= 2 groups of 32 tokens; its W k-groups
// of R wavefronts split K into slices of 256 k, slice W r + j going to
// k-group j in round r. More tokens than G * 32 take several token blocks
// (separate workgroups); the token blocks of a row block are mapped to the
// same XCD (workgroups are dealt to the 8 XCDs round robin in linear order),
// whose L2 then serves the weights they share. The partial tiles of the W
// k-groups meet in LDS at the end and are summed in k-group order: the
// result is bit-reproducible for a given launch shape.
//
// Memory access. Every load covers whole 128-byte lines where the data
// allows: the L1 looks up about one line per clock, so a load whose 64
// lanes touch 32 lines costs four times one that touches 8. Codes are
// loaded row-major (eight rows of 128 bytes per load) and transposed
// through a per-wavefront LDS stage; x is loaded by the k-group's threads in
// whole lines (16 threads per token) into a shared, swizzled LDS buffer that
// the R row wavefronts read as MFMA A fragments. All loads are bounded
// buffer loads: rows past N and tokens past M lie past their buffer's bound
// and read as zeros without touching memory, and pieces past K are sent
// past it, so nothing is clamped or masked afterwards. x is loaded two
// halves of a slice ahead (two register sets, two LDS buffers, one barrier
// per half), the weights one slice ahead, in the order x, weights, x: each
// wait for x then leaves the newer weight loads in flight. Nothing loaded
// is used (not even by a select) before it is needed, which would make the
// wave wait early.
//
// Operand mapping (v_mfma_f32_32x32x16_bf16, lane l, n = l % 32,
// h = l / 32: A lane holds A[n][8h .. 8h+7], B lane holds B[8h .. 8h+7][n],
// D lane holds D[8(r/4) + 4h + r%4][n] in register r). Within a slice, half
// h of the MFMA k covers k = 128 h .. 128 h + 127: step s of quarter c reads
// k = 128 h + 32 c + 8 s .. + 7. So a lane's B words for quarter c are 16
// staged code bytes of its row (64 h + 16 c), and its scale bytes for the
// slice are the 8 blocks 8 h .. 8 h + 7 of its row; token t's x for the
// same step sits at the same k.
#include "device.h"
#include "internal.h"

namespace nvfp4 {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kMtSlice = 256;          // k per slice
constexpr int kMtTokBytes = 256;       // staged x of one token for half a slice (128 k)
constexpr int kMtWPitch = 144;         // staged code row: 128 + 16 bytes
constexpr int kMtWStage = 32 * kMtWPitch;
constexpr int kMtMaxWaves = 8;         // two per SIMD, 256 registers each
constexpr int64_t kMtLdsMax = 80 * 1024;   // two workgroups per CU
constexpr int64_t kMtLdsOne = 160 * 1024;  // one workgroup per CU (all of its LDS)
constexpr int64_t kMtOneRound = 256;       // workgroups that one per CU runs in one round

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

// A wavefront's weights for one slice as loaded: 32 rows x 128 code bytes
// row-major (q[i]: row 8 i + l / 8, bytes 16 (l % 8) .. + 15) and the lane's
// 8 scale bytes (row l % 32, blocks 8 h .. 8 h + 7 of the slice: one 8-byte
// load, or four 2-byte loads).
struct MtW {
  u32x4_t q[4];
  uint32_t s[4];
};

}  // namespace

// KA: K % 128 == 0, so a lane's 8 scale bytes of a slice are one aligned
// 8-byte load that lies wholly inside or wholly outside K; else four 2-byte
// loads (rows start 2-byte aligned).
template <int G, int R, bool KA>
__global__ __launch_bounds__(64 * kMtMaxWaves) void k_gemv_mt(const SegTable tab,
                                                              const uint16_t* __restrict__ x,
                                                              int M, int64_t K, int64_t units,
                                                              int tblocks, int W) {
  static_assert((8 * G) % R == 0, "x staging: whole 16-byte pieces per thread");
  constexpr int P = 8 * G / R;                   // staged pieces per thread per half slice
  constexpr int kBuf = G * 32 * kMtTokBytes;     // half a slice of x for G * 32 tokens

  // blockIdx.x -> (row block, token block): the token blocks of a row block
  // share the XCD that blockIdx.x % 8 selects
  const int64_t b = blockIdx.x;
  const int64_t per = 8 * (int64_t)tblocks;
  const int64_t unit = (b / per) * 8 + (b % 8);
  const int tb = (int)((b % per) / 8);
  if (unit >= units) return;   // the same for the whole workgroup
  const Seg sg = find_seg(tab, unit);
  const int64_t N = sg.N;

  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rw = w % R, kg = w / R;
  const int n = lane & 31, h = lane >> 5;
  const int64_t n0 = sg.unit * (32 * R) + 32 * rw;
  const int tok0 = tb * G * 32;
  const int64_t cb = K >> 1, sbytes = K >> 4;
  const int64_t slices = (K + kMtSlice - 1) / kMtSlice;
  const int64_t rounds = (slices + W - 1) / W;
  unsigned char* const xbuf = lds + kg * 2 * kBuf;
  unsigned char* const stage = lds + (int64_t)W * 2 * kBuf + w * kMtWStage;

  // Every load is a bounded buffer load, issued unconditionally: rows past N
  // and tokens past M lie past the bound of their buffer and read as zeros,
  // and pieces past K are sent past it. Codes go row-major (eight whole
  // 128-byte lines per load) through the wavefront's LDS stage; each lane
  // loads its own scale bytes.
  const __amdgpu_buffer_rsrc_t rc = buf_rsrc(sg.codes + n0 * cb, (N - n0) * cb);
  const __amdgpu_buffer_rsrc_t rs = buf_rsrc(sg.scales + n0 * sbytes, (N - n0) * sbytes);
  const __amdgpu_buffer_rsrc_t rx = buf_rsrc(x, (int64_t)M * K * 2);
  int coff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) coff[i] = (int)((8 * i + (lane >> 3)) * cb) + 16 * (lane & 7);
  const int soff = (int)(n * sbytes) + 8 * h;
  auto load_w = [&](int64_t sl, MtW& wt) {
    const int64_t k0 = sl * kMtSlice;
    const bool cok = sl < slices && k0 + 32 * (lane & 7) < K;
#pragma unroll
    for (int i = 0; i < 4; ++i) wt.q[i] = buf_load16<kBufNt>(rc, cok ? coff[i] + (int)(k0 >> 1) : kBufOob);
    if (KA) {
      const bool v = sl < slices && k0 + 128 * h < K;
      const uint2 sv = __builtin_bit_cast(
          uint2, __builtin_amdgcn_raw_buffer_load_b64(rs, v ? soff + (int)(k0 >> 4) : kBufOob, 0, 0));
      wt.s[0] = sv.x;
      wt.s[1] = sv.y;
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const bool v = sl < slices && k0 + 128 * h + 32 * c < K;
        wt.s[c] = __builtin_amdgcn_raw_buffer_load_b16(rs, v ? soff + (int)(k0 >> 4) + 2 * c : kBufOob,
                                                       0, 0);
      }
    }
  };
  // the lane's scale bytes of quarters 2 d and 2 d + 1 (one word)
  auto scale_word = [&](const MtW& wt, int d) -> uint32_t {
    if (KA) return wt.s[d];
    return wt.s[2 * d] | (wt.s[2 * d + 1] << 16);
  };
  auto store_w = [&](const MtW& wt) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<u32x4_t*>(stage + (8 * i + (lane >> 3)) * kMtWPitch + 16 * (lane & 7)) =
          wt.q[i];
  };

  // x staging: piece e = (thread of the k-group) + 64 R p is token e / 16,
  // 16-byte chunk j = e % 16 (quarter j / 8 of the half, MFMA half j / 4 % 2,
  // step j % 4); it goes to LDS byte 256 t + 16 (j ^ (t % 16)). The 16
  // threads of a token read two whole 128-byte lines.
  const int tk = rw * 64 + lane;
  int xsrc[P];
  int xdst[P];
  int xk[P];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int e = tk + 64 * R * p;
    const int tt = e >> 4, j = e & 15;
    xk[p] = 128 * ((j >> 2) & 1) + 32 * (j >> 3);
    xsrc[p] = (int)((tok0 + tt) * K + xk[p] + 8 * (j & 3)) * 2;
    xdst[p] = tt * kMtTokBytes + ((j ^ (tt & 15)) << 4);
  }
  struct XStage {
    u32x4_t v[P];
  };
  // half e of slice sl: quarters 2 e and 2 e + 1
  auto stage_load = [&](int64_t sl, int e, XStage& xs) {
    const int64_t k0 = sl * kMtSlice + 64 * e;
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const bool v = sl < slices && k0 + xk[p] < K;
      xs.v[p] = buf_load16<0>(rx, v ? xsrc[p] + (int)(k0 * 2) : kBufOob);
    }
  };
  auto stage_store = [&](const XStage& xs, unsigned char* buf) {
#pragma unroll
    for (int p = 0; p < P; ++p) *reinterpret_cast<u32x4_t*>(buf + xdst[p]) = xs.v[p];
  };

  // the A fragment of group q, quarter c of a half, step s: token 32 q + n,
  // chunk 8 c + 4 h + s
  int xrd[2][4];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int s = 0; s < 4; ++s)
      xrd[c][s] = n * kMtTokBytes + (((8 * c + 4 * h + s) ^ (n & 15)) << 4);
  // the B words of quarter c: row n, code bytes 64 h + 16 c .. + 15
  const unsigned char* const wrd = stage + n * kMtWPitch + 64 * h;

  f32x16_t acc[G];
#pragma unroll
  for (int q = 0; q < G; ++q)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[q][i] = 0.f;

  // half e of the slice from x buffer buf and the staged codes
  auto compute = [&](const MtW& wt, const unsigned char* buf, int e) {
    const uint32_t sw = scale_word(wt, e);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int cq = 2 * e + c;
      // the quarter's operands first, so that the LDS reads overlap
      const u32x4_t bq = *reinterpret_cast<const u32x4_t*>(wrd + 16 * cq);
      u32x4_t a[4][G];
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int q = 0; q < G; ++q)
          a[s][q] = *reinterpret_cast<const u32x4_t*>(buf + q * 32 * kMtTokBytes + xrd[c][s]);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        // block 8 h + 2 cq + s / 2 of the slice: byte (2 cq + s / 2) % 4 of sw
        const float sc = ((2 * cq + (s >> 1)) & 3) == 0   ? e4m3_to_f32<0>(sw)
                         : ((2 * cq + (s >> 1)) & 3) == 1 ? e4m3_to_f32<1>(sw)
                         : ((2 * cq + (s >> 1)) & 3) == 2 ? e4m3_to_f32<2>(sw)
                                                           : e4m3_to_f32<3>(sw);
        const bf16x8_t bw = mt_decode8(bq[s], sc);
#pragma unroll
        for (int q = 0; q < G; ++q)
          acc[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(mt_bf16x8(a[s][q]), bw, acc[q], 0, 0, 0);
      }
    }
  };

  // x is loaded two halves ahead of its use (two sets of registers, two LDS
  // buffers), the weights one slice ahead. Per round the loads go out in the
  // order x, weights, x, so that each wait for x leaves the newer loads in
  // flight.
  unsigned char* const buf0 = xbuf;
  unsigned char* const buf1 = xbuf + kBuf;
  MtW wc, wn;
  XStage xa, xb;
  load_w(kg, wc);
  stage_load(kg, 0, xb);
  stage_load(kg, 1, xa);
  stage_store(xb, buf0);
  __syncthreads();
  for (int64_t r = 0; r < rounds; ++r) {
    const int64_t sl = r * W + kg;
    store_w(wc);
    // first half (x in buf0, the second half's x in xa)
    stage_load(sl + W, 0, xb);
    load_w(sl + W, wn);
    __builtin_amdgcn_sched_barrier(0);
    compute(wc, buf0, 0);
    __builtin_amdgcn_sched_barrier(0);
    stage_store(xa, buf1);
    __syncthreads();
    // second half (x in buf1, the next slice's first half in xb)
    stage_load(sl + W, 1, xa);
    __builtin_amdgcn_sched_barrier(0);
    compute(wc, buf1, 1);
    __builtin_amdgcn_sched_barrier(0);
    stage_store(xb, buf0);
    __syncthreads();
    wc = wn;
  }

  // the k-groups' partial tiles, summed in k-group order by k-group 0 (the
  // loop's last barrier has freed the x buffers and stages)
  if (W > 1) {
    float* const red = reinterpret_cast<float*>(lds);   // [W - 1][R][G][16][64]
    if (kg > 0) {
#pragma unroll
      for (int q = 0; q < G; ++q)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          red[((((kg - 1) * R + rw) * G + q) * 16 + i) * 64 + lane] = acc[q][i];
    }
    __syncthreads();
    if (kg == 0) {
      for (int v = 1; v < W; ++v)
#pragma unroll
        for (int q = 0; q < G; ++q)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            acc[q][i] += red[((((v - 1) * R + rw) * G + q) * 16 + i) * 64 + lane];
    }
  }
  if (kg == 0 && n0 + n < N) {
    const float gs = *sg.gscale;
#pragma unroll
    for (int q = 0; q < G; ++q)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int m = tok0 + 32 * q + 8 * (i >> 2) + 4 * h + (i & 3);
        if (m < M) sg.y[(int64_t)m * N + n0 + n] = acc[q][i] * gs;
      }
  }
}

bool mt_applicable(int M) { return M > NVFP4_MAX_M_SMALL && M <= NVFP4_MAX_M_INTERNAL; }

int64_t mt_lds_bytes(const MtShape& sh) {
  const int64_t xb = (int64_t)2 * sh.W * sh.G * 32 * kMtTokBytes + (int64_t)sh.R * sh.W * kMtWStage;
  const int64_t rb = (int64_t)(sh.W - 1) * sh.R * sh.G * 16 * 64 * 4;
  return xb > rb ? xb : rb;
}

MtShape mt_shape(const SegDesc* d, int n, int M, int64_t K) {
  auto units = [&](int rows) {
    int64_t u = 0;
    for (int s = 0; s < n; ++s) u += (d[s].N + rows - 1) / rows;
    return u;
  };
  // Chosen from measured launch-shape sweeps on the stress (12288 x 4096,
  // 4096 x 12288) and LM-head (151936 x 4096) matrices at 16 and 128 tokens.
  MtShape sh;
  const int mg = (M + 31) / 32;
  // two token groups per workgroup (one decode for both) when the row
  // blocks of 128 rows still number 192 or more in all, else one
  sh.G = mg >= 2 && units(128) * ((mg + 1) / 2) >= 192 ? 2 : 1;
  sh.tblocks = (mg + sh.G - 1) / sh.G;
  // row wavefronts sharing each staged piece of x: as many as leave 192
  // workgroups
  sh.R = units(128) * sh.tblocks >= 192 ? 4 : (units(64) * sh.tblocks >= 192 ? 2 : 1);
  // k-groups. Where the grid fits on the CUs one workgroup each, LDS for a
  // second workgroup per CU buys nothing: up to 4 k-groups (8 wavefronts)
  // within all of the CU's LDS, since with one or two wavefronts per SIMD
  // the weight stream waits on load latency and more k-groups keep more
  // slices in flight (warm same-process A/B: 4096 x 12288 at 128 tokens
  // 36.0 -> 33.0 us; 12288 x 4096 at 128 tokens 28.6 -> 28.3 us, and at 32
  // tokens 15.6 -> 15.4 and 29.1 -> 28.8 us). Otherwise one with two token
  // groups, else two (three with one row wavefront), within half of it.
  // Never more than there are slices.
  const int64_t slices = (K + kMtSlice - 1) / kMtSlice;
  const bool one_round = units(32 * sh.R) * sh.tblocks <= kMtOneRound;
  const int64_t budget = one_round ? kMtLdsOne : kMtLdsMax;
  int64_t W;
  if (one_round)
    W = kMtMaxWaves / sh.R < 4 ? kMtMaxWaves / sh.R : 4;
  else
    W = sh.G == 2 ? 1 : (sh.R == 1 ? 3 : 2);
  sh.W = (int)(W > slices ? slices : W);
  while (sh.W > 1 && mt_lds_bytes(sh) > budget) --sh.W;
  return sh;
}

hipError_t launch_gemv_mt_shape(const SegDesc* d, int n, const uint16_t* x, int M, int64_t K,
                                const MtShape& sh, hipStream_t stream) {
  if (!mt_applicable(M) || n < 1 || n > kMaxSegments || K <= 0) return hipErrorInvalidValue;
  // buffer offsets are 32-bit: the x of a token block and 32 rows of codes
  // stay far below the bound
  if (K > (1 << 20)) return hipErrorInvalidValue;
  if (sh.G < 1 || sh.G > 2 || (sh.R != 1 && sh.R != 2 && sh.R != 4) || (sh.G == 2 && sh.R == 1) ||
      sh.W < 1 || sh.R * sh.W > kMtMaxWaves || sh.tblocks < 1 ||
      (int64_t)sh.tblocks * sh.G * 32 < M || mt_lds_bytes(sh) > kMtLdsOne)
    return hipErrorInvalidValue;
  const SegTable tab = make_seg_table(d, n, 32 * sh.R);
  const int64_t units = tab.start[kMaxSegments];
  if (units == 0) return hipSuccess;
  // whole multiples of 8 units so that the XCD mapping stays a bijection
  const int64_t grid = ((units + 7) / 8) * 8 * sh.tblocks;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  const size_t lds = (size_t)mt_lds_bytes(sh);
  const bool ka = K % 128 == 0;
#define NVFP4_MT(GG, RR)                                                                      \
  do {                                                                                        \
    if (ka)                                                                                   \
      hipLaunchKernelGGL((k_gemv_mt<GG, RR, true>), dim3((unsigned)grid),                     \
                         dim3(64 * sh.R * sh.W), lds, stream, tab, x, M, K, units, sh.tblocks, \
                         sh.W);                                                               \
    else                                                                                      \
      hipLaunchKernelGGL((k_gemv_mt<GG, RR, false>), dim3((unsigned)grid),                    \
                         dim3(64 * sh.R * sh.W), lds, stream, tab, x, M, K, units, sh.tblocks, \
                         sh.W);                                                               \
  } while (0)
  switch (sh.G * 10 + sh.R) {
    case 11: NVFP4_MT(1, 1); break;
    case 12: NVFP4_MT(1, 2); break;
    case 14: NVFP4_MT(1, 4); break;
    case 22: NVFP4_MT(2, 2); break;
    case 24: NVFP4_MT(2, 4); break;
    default: return hipErrorInvalidValue;
  }
#undef NVFP4_MT
  return hipGetLastError();
}

hipError_t launch_gemv_mt(const SegDesc* d, int n, const uint16_t* x, int M, int64_t K,
                          hipStream_t stream) {
  if (!mt_applicable(M) || n < 1 || n > kMaxSegments || K <= 0) return hipErrorInvalidValue;
  return launch_gemv_mt_shape(d, n, x, M, K, mt_shape(d, n, M, K), stream);
}

}  // namespace nvfp4
