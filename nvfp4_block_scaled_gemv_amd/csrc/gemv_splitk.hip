// gemv_splitk.hip -- NVFP4 g16 W4A16 GEMV on the CDNA4 matrix cores for
// 3 <= M <= 8 activation rows and K a multiple of 256, with K split over the
// wavefronts of a workgroup.
//
// Work split. A workgroup of W wavefronts owns a contiguous range of 16-row
// tiles. K is cut into slices of 256 and wavefront w owns the KS consecutive
// slices starting at k = 256 KS w (K = 256 KS W). For every tile each
// wavefront multiplies its part of the 16 weight rows by its part of x. With
// KS = 1 (K <= 4096) a wavefront's x operands are the same for every tile:
// they are loaded into registers once, and the loop streams nothing but codes
// and scales. With KS > 1 the x operands of a slice are loaded together with
// its weights (they come from L2: every workgroup reads the same x).
//
// Weight stream. A slice of a tile is 16 rows x 128 code bytes, one cache line
// per row. The matrix-core layout gives each lane 16 bytes of one row, so a
// load in that layout would touch 16 lines for 64 bytes each and the L1 would
// forward every half line to L2 on its own (measured: 47 bytes per L1-to-L2
// request instead of 121, and the texture addresser stalled on the cache).
// The codes are therefore loaded row-major, eight whole lines per load, and
// transposed through a small per-wavefront LDS buffer. The row's 16 scale
// bytes of the slice are loaded with caching: the same line serves the eight
// wavefronts whose slices it covers. Loads go through a ring of D register
// stages, D - 1 items ahead of the math. They are inline asm so that the
// compiler's wait insertion does not track them (across the loop back-edge it
// would wait for all of them); every step waits explicitly for its own item,
// and every issued load is consumed.
//
// Reduction. A wavefront that has finished a tile writes its partial tile
// into one of kSlots LDS slots and counts itself in with an LDS atomic; the
// last of the W to arrive sums the partials in wavefront order (so the result
// does not depend on timing), stores the tile and frees the slot. Wavefronts
// never wait for each other except when one is kSlots tiles ahead of the
// slowest (a workgroup barrier per tile cost a quarter of the time).
//
// Block scale on the output. In v_mfma_f32_16x16x32_bf16 lane l (i = l % 16,
// g = l / 16, the 16-lane row g) supplies B[8g .. 8g+7][i] and A[i][8g .. 8g+7]
// and receives D[4g + r][i], r < 4. Step j (j = 0, 1) of a slice multiplies
// eight of its sixteen blocks: blocks 4j .. 4j+3 in lane rows 0 and 1 and
// blocks 8 + 4j .. 8 + 4j + 3 in lane rows 2 and 3 (relative blocks 0..3 and
// 4..7 of the step). Lane (i, g) holds the 16 code bytes of relative blocks 2g
// and 2g + 1 of row i: dwords d0, d1 are the two halves of the first, d2, d3
// those of the second. Two v_permlane16_swap (on d0/d1 and on d2/d3) exchange
// dwords between lane rows 0 and 1 and between rows 2 and 3; afterwards MFMA
// m (taking dword m of every lane) sees the two halves of relative block b_m
// in rows 0 and 1 and those of relative block b_m + 4 in rows 2 and 3,
// b_m = 0, 2, 1, 3. The A operand's rows 0..7 hold the tokens with x only at
// the k positions of lane rows 0 and 1 (zero elsewhere) and rows 8..15 the
// tokens with x only at those of lane rows 2 and 3. So D rows 0..7 are dot
// products over one block alone and rows 8..15 over another, and every lane
// scales its four D values by the E4M3 scale of its own block before
// accumulating in fp32: byte b_m of scale dword j (rows 0, 1) or 2 + j (rows
// 2, 3) of the slice, which makes a lane's two scale dwords adjacent. The
// weights enter the MFMA as plain E2M1 values (v_cvt_scalef32_pk_bf16_fp4 with
// scale 1, exact). Lanes l and l + 32 (the two block halves of the same
// outputs) are added at the end of a tile; the tensor scale multiplies the
// final sum.
#include "device.h"
#include "internal.h"
#include "splitk_slots.h"

namespace nvfp4 {

// 512 zero bytes: the A-operand source of lanes whose operand is all zero
// (tokens >= M, or the other half of the block pair). Never written.
__device__ __attribute__((aligned(64))) uint32_t g_splitk_zero[128];

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kSliceK = 256;
// wavefronts per workgroup at most: x held in registers for one slice (128
// registers per lane), for two slices, or streamed with every slice
constexpr int sk_max_waves(int XS) { return XS == 1 ? 16 : 8; }
constexpr int kSkCUs = 256;

// s_waitcnt immediate (gfx9 encoding: vmcnt bits 3..0 and 15..14, expcnt
// 6..4, lgkmcnt 11..8) that waits for vmcnt <= n only.
constexpr int sk_vmcnt(int n) {
  return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8);
}

__device__ __forceinline__ bf16x8_t sk_e2m1x8(uint32_t w) {
  const bf16x2_t b0 = e2m1x2_to_bf16<0>(w);
  const bf16x2_t b1 = e2m1x2_to_bf16<1>(w);
  const bf16x2_t b2 = e2m1x2_to_bf16<2>(w);
  const bf16x2_t b3 = e2m1x2_to_bf16<3>(w);
  bf16x8_t r;
  r[0] = b0[0]; r[1] = b0[1]; r[2] = b1[0]; r[3] = b1[1];
  r[4] = b2[0]; r[5] = b2[1]; r[6] = b3[0]; r[7] = b3[1];
  return r;
}

__device__ __forceinline__ bf16x8_t sk_bf16x8(u32x4_t v) {
  bf16x8_t r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

// v + (v of lane l + 32) in lanes l < 32, by v_permlane32_swap (a vector-ALU
// exchange of the wavefront's two halves; a shuffle would go through LDS).
__device__ __forceinline__ f32x4_t sk_add_upper_half(f32x4_t v) {
  f32x4_t r;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t u = __float_as_uint(v[k]);
    const auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    r[k] = v[k] + __uint_as_float(p[1]);
  }
  return r;
}

// One ring stage (an item): per slice the codes of the two row-major loads
// and the lane's two scale dwords; when x is streamed (XS = 0, one slice per
// item), also the slice's A operands.
template <int XS>
struct SkStage {
  static constexpr int kSl = XS == 0 ? 1 : XS;   // slices per item
  u32x4_t q[kSl][2];
  u32x2_t s[kSl];
  u32x4_t a[XS == 0 ? 8 : 1];
};

// Codes of one slice (two loads, rows 8t + l / 8 at byte 16 (l % 8) of the
// slice, lane l) and the lane's scale dwords 2 (g / 2) and 2 (g / 2) + 1 of
// the slice. The scales are loaded without the non-temporal hint: other
// wavefronts read the same line.
__device__ __forceinline__ void sk_load_weights(const uint8_t* c0, const uint8_t* c1,
                                                const uint8_t* sp, u32x4_t (&q)[2], u32x2_t& s) {
  asm volatile(
      "global_load_dwordx4 %0, %3, off nt\n"
      "global_load_dwordx4 %1, %4, off nt\n"
      "global_load_dwordx2 %2, %5, off"
      : "=&v"(q[0]), "=&v"(q[1]), "=&v"(s)
      : "v"(c0), "v"(c1), "v"(sp)
      : "memory");
}

// The eight A operands of a slice: a[4j + m] (step j, MFMA m) is the 16 bytes
// at byte offset 128 j + 32 b_m of the lane's x pointer (b_m = 0, 2, 1, 3).
__device__ __forceinline__ void sk_load_x(const unsigned char* p, u32x4_t* a) {
  asm volatile(
      "global_load_dwordx4 %0, %8, off\n"
      "global_load_dwordx4 %1, %8, off offset:64\n"
      "global_load_dwordx4 %2, %8, off offset:32\n"
      "global_load_dwordx4 %3, %8, off offset:96\n"
      "global_load_dwordx4 %4, %8, off offset:128\n"
      "global_load_dwordx4 %5, %8, off offset:192\n"
      "global_load_dwordx4 %6, %8, off offset:160\n"
      "global_load_dwordx4 %7, %8, off offset:224"
      : "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3]), "=&v"(a[4]), "=&v"(a[5]),
        "=&v"(a[6]), "=&v"(a[7])
      : "v"(p)
      : "memory");
}

// acc += this lane's share of one slice (two 128-k steps).
__device__ __forceinline__ void sk_compute(const u32x4_t (&q)[2], u32x2_t sv, const u32x4_t* a,
                                           f32x4_t& acc) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    // the scales of the lane's blocks in step j: bytes b_m of its dword j
    const uint32_t sj = j ? sv.y : sv.x;
    const auto p01 = __builtin_amdgcn_permlane16_swap(q[j].x, q[j].y, false, false);
    const auto p23 = __builtin_amdgcn_permlane16_swap(q[j].z, q[j].w, false, false);
    const uint32_t word[4] = {p01[0], p01[1], p23[0], p23[1]};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const f32x4_t d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          sk_bf16x8(a[4 * j + m]), sk_e2m1x8(word[m]), f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
      const float sc = m == 0 ? e4m3_to_f32<0>(sj) : m == 1 ? e4m3_to_f32<2>(sj)
                     : m == 2 ? e4m3_to_f32<1>(sj) : e4m3_to_f32<3>(sj);
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] = __builtin_fmaf(d[r], sc, acc[r]);
    }
  }
}

}  // namespace

// A segment cursor with the segment's pointers (read from kernel-argument
// memory with a wavefront-uniform index whenever the cursor moves).
struct SkCursor {
  SegCursor c;
  const uint8_t* codes;
  const uint8_t* scales;
  const float* gscale;
  float* y;
  int64_t N;
  float gs;             // *gscale (read by the cursor that finishes tiles)

  __device__ __forceinline__ int64_t first() const { return c.first; }
  __device__ __forceinline__ void load(const SegTable& t) {
    codes = t.codes[c.k];
    scales = t.scales[c.k];
    gscale = t.gscale[c.k];
    y = t.y[c.k];
    N = t.N[c.k];
  }
  // the tensor scale through a scalar load: it is counted apart from the
  // vector loads of the ring, so waiting for it does not wait for them
  __device__ __forceinline__ void load_gs() {
    gs = *(const __attribute__((address_space(4))) float*)(gscale);
  }
  __device__ __forceinline__ void begin(const SegTable& t, int64_t u) {
    c.begin(t, u);
    load(t);
  }
  // true when the segment changed (u is a tile of this workgroup)
  __device__ __forceinline__ bool seek(const SegTable& t, int64_t u) {
    if (!c.seek(t, u)) return false;
    load(t);
    return true;
  }
};

// Per-wavefront state of the weight stream.
template <int XS>
struct SkEngine {
  int64_t K;
  int64_t kw;                 // wavefront's first k
  const unsigned char* xl;    // lane's x operand pointer of slice 0
  int64_t xstride;            // bytes per slice (0 for all-zero lanes)
  int i, g, lane;

  // item (tile, slice sl) when x is streamed; (tile, all XS slices) else
  __device__ __forceinline__ void issue(const SkCursor& cs, int64_t tile, int sl,
                                        SkStage<XS>& st) const {
    const int64_t r0 = (tile - cs.first()) * 16;
    const int64_t n = r0 + i;              // scale row of lane (i, g)
    const int64_t a = r0 + (lane >> 3);    // code rows of the two loads
    const int64_t row = n < cs.N ? n : cs.N - 1;
    const int64_t row0 = a < cs.N ? a : cs.N - 1;
    const int64_t row1 = a + 8 < cs.N ? a + 8 : cs.N - 1;
#pragma unroll
    for (int u = 0; u < SkStage<XS>::kSl; ++u) {
      const int64_t k0 = kw + (int64_t)(sl + u) * kSliceK;
      const uint8_t* cb = cs.codes + (k0 >> 1) + 16 * (lane & 7);
      sk_load_weights(cb + row0 * (K >> 1), cb + row1 * (K >> 1),
                      cs.scales + row * (K >> 4) + (k0 >> 4) + 8 * (g >> 1), st.q[u], st.s[u]);
    }
    if constexpr (XS == 0) sk_load_x(xl + sl * xstride, st.a);
  }
};

// LDS of a workgroup: partial-tile slots, per-wavefront transpose buffers and
// the slots' arrival and release counters.
constexpr int kSlots = kSkSlots;
constexpr int kStagePitch = 144;            // bytes per staged row (128 + 16: bank skew)
constexpr int kStageBytes = 16 * kStagePitch;
constexpr int kSpinLimit = 1 << 22;         // bound of a slot wait (never reached)

// Set (bit 0) by a wavefront that gave up a slot wait; read and cleared by
// splitk_take_fault. One word per device (this file's code object).
__device__ uint32_t g_splitk_fault = 0u;
constexpr int kRedBatch = 4;                // partial loads in flight in the sum

struct SkShared {
  f32x4_t* part;       // [kSlots][W][32]
  unsigned char* stage;  // [W][kStageBytes]
  uint32_t* cnt;       // [kSlots] arrivals, all rounds
  uint32_t* done;      // [kSlots] rounds summed
};

static size_t splitk_lds(int W) {
  return (size_t)kSlots * W * 32 * 16 + (size_t)W * kStageBytes + 2 * kSlots * sizeof(uint32_t);
}

// Count this wavefront's partial of local tile tl (global tile `tile`) into
// its slot; the last arrival sums the W partials in wavefront order and
// stores the tile.
template <int M, int WMAX>
__device__ __forceinline__ void sk_finish(const SkCursor& cs, int64_t tile, int tl, f32x4_t& acc,
                                          uint32_t done_seen, const SkShared& sh, int w, int W,
                                          int lane, int spin_limit) {
  // lanes l and l + 32 hold the two block halves of the same outputs
  acc = sk_add_upper_half(acc);
  const int s = sk_slot(tl);
  const uint32_t round = sk_round(tl);
  // the slot's previous round must have been summed (it normally has been
  // long ago; the wait only holds a wavefront kSlots tiles ahead). done_seen
  // is the slot's release count read before this tile's math. A negative
  // limit (a test of the fault path) gives up at once.
  bool free = spin_limit >= 0 && sk_slot_free(done_seen, round);
  for (int spin = 0; !free && spin < spin_limit; ++spin) {
    __builtin_amdgcn_s_sleep(1);
    free = sk_slot_free(
        __hip_atomic_load(&sh.done[s], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP), round);
  }
  if (!free) {
    // give up: record the fault and arrive with a NaN partial
    if (lane == 0) atomicOr(&g_splitk_fault, 1u);
    acc = f32x4_t{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
  }
  f32x4_t* slot = sh.part + s * (W * 32);
  if (lane < 32) slot[w * 32 + lane] = acc;
  // the partial is written before the arrival is counted: LDS executes one
  // wavefront's operations in issue order, so only the compiler is held back
  asm volatile("" ::: "memory");
  uint32_t old = 0;
  if (lane == 0) old = atomicAdd(&sh.cnt[s], 1u);
  old = __builtin_amdgcn_readfirstlane(old);
  asm volatile("" ::: "memory");
  if (sk_last_arrival(old, round, W)) {
    // lane l < 32 sums partials 0 .. h-1 of entry l, lane l + 32 partials
    // h .. W-1 (h = ceil(W / 2)); the loads are unconditional (clamped to a
    // valid partial) so that they are all in flight before the first add
    const int h = (W + 1) >> 1;
    const int vb = lane < 32 ? 0 : h;
    const int ve = lane < 32 ? h : W;
    const f32x4_t* src = slot + (lane & 31);
    f32x4_t sum = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int v0 = 0; v0 < WMAX / 2; v0 += kRedBatch) {   // kRedBatch loads in flight
      f32x4_t p[kRedBatch];
#pragma unroll
      for (int v = 0; v < kRedBatch; ++v) {
        const int vv = vb + v0 + v < ve ? vb + v0 + v : ve - 1;
        p[v] = src[(vv < 0 ? 0 : vv) * 32];
      }
#pragma unroll
      for (int v = 0; v < kRedBatch; ++v)
        if (vb + v0 + v < ve) sum += p[v];
    }
    sum = sk_add_upper_half(sum);
    // the slot is released after the partials have been read (in LDS order)
    asm volatile("" ::: "memory");
    if (lane == 0)
      __hip_atomic_store(&sh.done[s], round + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (lane < 32) {
      const float gs = cs.gs;
      const int64_t n = (tile - cs.first()) * 16 + (lane & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 4 * (lane >> 4) + r;   // lane (i, g < 2) holds D[4g + r][i]
        if (m < M && n < cs.N) cs.y[(int64_t)m * cs.N + n] = sum[r] * gs;
      }
    }
  }
  acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
}

// codes, scales and x are deliberately not __restrict__: read-only noalias
// pointers would let the compiler treat their memory as invariant and move
// the ring's loads across its ordering points.
template <int M, int XS, int D>
__global__ __launch_bounds__(64 * sk_max_waves(XS)) void
k_gemv_splitk(const SegTable tab, const uint16_t* x, int64_t K, int KS, int spin_limit) {
  constexpr bool WX = XS == 0;
  constexpr int kSl = SkStage<XS>::kSl;
  constexpr int kIssue = 3 * kSl + (WX ? 8 : 0);   // vector-memory instructions per item
  static_assert(D >= 3 && D <= 5 && (D - 2) * kIssue <= 63, "vmcnt is a 6-bit counter");
  extern __shared__ __attribute__((aligned(16))) f32x4_t lds[];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int W = blockDim.x >> 6;
  const int i = lane & 15, g = lane >> 4;
  const int64_t tiles = tab.start[kMaxSegments];
  const int64_t t0 = tiles * blockIdx.x / gridDim.x;
  const int nt = (int)(tiles * (blockIdx.x + 1) / gridDim.x - t0);
  if (nt <= 0) return;   // the same for the whole workgroup
  const int ks = WX ? KS : XS;   // slices per wavefront
  const int ipt = WX ? KS : 1;   // items per tile
  const int n = nt * ipt;        // items of every wavefront

  SkShared sh;
  sh.part = lds;
  sh.stage = reinterpret_cast<unsigned char*>(lds + kSlots * W * 32);
  sh.cnt = reinterpret_cast<uint32_t*>(sh.stage + W * kStageBytes);
  sh.done = sh.cnt + kSlots;
  if (threadIdx.x < 2 * kSlots) sh.cnt[threadIdx.x] = 0u;
  __syncthreads();   // before any load of the ring is in flight

  SkEngine<XS> eng;
  eng.K = K;
  eng.kw = (int64_t)w * ks * kSliceK;
  eng.i = i;
  eng.g = g;
  eng.lane = lane;
  // This lane's A operand: token i % 8 when its half (i < 8) matches the lane
  // row's block half (g < 2), at k offset 128 (g / 2) + 8 (g % 2) of the
  // slice (+ 64 j + 16 b_m); else zeros.
  const bool xlive = ((i < 8) == (g < 2)) && (i & 7) < M;
  eng.xl = xlive ? reinterpret_cast<const unsigned char*>(x + (int64_t)(i & 7) * K + eng.kw +
                                                          128 * (g >> 1) + 8 * (g & 1))
                 : reinterpret_cast<const unsigned char*>(g_splitk_zero);
  eng.xstride = xlive ? 2 * kSliceK : 0;
  // this wavefront's transpose buffer: the two row-major loads are written as
  // rows l / 8 and 8 + l / 8, and for step j lane (i, g) reads the 16 bytes of
  // relative blocks 2g, 2g + 1 of row i, at 32 j + 16 (g % 2) + 64 (g / 2)
  unsigned char* const stage = sh.stage + w * kStageBytes;
  u32x4_t* const st_w0 = reinterpret_cast<u32x4_t*>(stage + kStagePitch * (lane >> 3) + 16 * (lane & 7));
  u32x4_t* const st_w1 = st_w0 + 8 * kStagePitch / 16;
  const u32x4_t* const st_r =
      reinterpret_cast<const u32x4_t*>(stage + kStagePitch * i + 16 * (g & 1) + 64 * (g >> 1));

  // stationary x operands (issued first: the first step's wait covers them)
  u32x4_t xa[WX ? 1 : XS][8];
  if constexpr (!WX) {
#pragma unroll
    for (int u = 0; u < XS; ++u) sk_load_x(eng.xl + u * eng.xstride, xa[u]);
  }

  SkStage<XS> R0, R1, R2, R3, R4;
  SkCursor ci, cf;   // segments of the next tile to issue and to finish
  ci.begin(tab, t0);
  cf = ci;
  cf.load_gs();
  int64_t itile = t0;   // next item to issue: (itile, isl)
  int isl = 0;
  auto issue_next = [&](SkStage<XS>& st) {
    eng.issue(ci, itile, isl, st);
    if (++isl == ipt) {
      isl = 0;
      if (++itile < t0 + nt) ci.seek(tab, itile);
    }
  };
  // prologue: items 0 .. min(D - 1, n) - 1
  issue_next(R0);
  if (1 < n) issue_next(R1);
  if (D >= 4 && 2 < n) issue_next(R2);
  if (D >= 5 && 3 < n) issue_next(R3);
  asm volatile("" ::: "memory");

  f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
  int64_t ctile = t0;   // item being multiplied: (ctile, csl)
  int csl = 0;
  // One ring step for item c held in `cur`: wait until it has landed (items
  // c + 1 .. c + D - 2 may stay in flight), issue item c + D - 1 into `nxt`
  // (the stage item c - 1 used), multiply item c, and finish the tile after
  // its last item.
  auto step = [&](const SkStage<XS>& cur, SkStage<XS>& nxt, int c) {
    if (c + D - 2 < n)
      __builtin_amdgcn_s_waitcnt(sk_vmcnt((D - 2) * kIssue));
    else
      __builtin_amdgcn_s_waitcnt(sk_vmcnt(0));
    asm volatile("" ::: "memory");
    if (c + D - 1 < n) issue_next(nxt);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    // a tile's last item: read its slot's release count now, so that the
    // check after the math finds it in a register
    const bool last = csl + 1 == ipt;
    uint32_t done_seen = 0xFFFFFFFFu;
    if (last)
      done_seen = __hip_atomic_load(&sh.done[(int)(ctile - t0) % kSlots], __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_WORKGROUP);
#pragma unroll
    for (int u = 0; u < kSl; ++u) {
      // the transpose: the buffer's previous reads were waited for by the
      // compiler before their results were used, and LDS keeps one
      // wavefront's accesses in order
      *st_w0 = cur.q[u][0];
      *st_w1 = cur.q[u][1];
      const u32x4_t qt[2] = {st_r[0], st_r[2]};
      if constexpr (WX)
        sk_compute(qt, cur.s[u], cur.a, acc);
      else
        sk_compute(qt, cur.s[u], xa[u], acc);
    }
    if (++csl == ipt) {
      sk_finish<M, sk_max_waves(XS)>(cf, ctile, (int)(ctile - t0), acc, done_seen, sh, w, W,
                                     lane, spin_limit);
      csl = 0;
      if (++ctile < t0 + nt && cf.seek(tab, ctile)) cf.load_gs();
    }
  };
  if constexpr (D == 3) {
    for (int c = 0;;) {
      step(R0, R2, c);
      if (++c >= n) break;
      step(R1, R0, c);
      if (++c >= n) break;
      step(R2, R1, c);
      if (++c >= n) break;
    }
  } else if constexpr (D == 4) {
    for (int c = 0;;) {
      step(R0, R3, c);
      if (++c >= n) break;
      step(R1, R0, c);
      if (++c >= n) break;
      step(R2, R1, c);
      if (++c >= n) break;
      step(R3, R2, c);
      if (++c >= n) break;
    }
  } else {
    for (int c = 0;;) {
      step(R0, R4, c);
      if (++c >= n) break;
      step(R1, R0, c);
      if (++c >= n) break;
      step(R2, R1, c);
      if (++c >= n) break;
      step(R3, R2, c);
      if (++c >= n) break;
      step(R4, R3, c);
      if (++c >= n) break;
    }
  }
}

// The slot-wait bound the launches pass (a test may lower it, or make it
// negative to force the fault path).
static int g_splitk_spin_limit = kSpinLimit;

void splitk_set_spin_limit(int limit) { g_splitk_spin_limit = limit == 0 ? kSpinLimit : limit; }

hipError_t splitk_take_fault(hipStream_t stream, uint32_t* fault) {
  hipError_t e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return e;
  e = hipMemcpyFromSymbol(fault, HIP_SYMBOL(g_splitk_fault), sizeof(uint32_t), 0,
                          hipMemcpyDeviceToHost);
  if (e != hipSuccess || *fault == 0u) return e;
  const uint32_t zero = 0u;
  return hipMemcpyToSymbol(HIP_SYMBOL(g_splitk_fault), &zero, sizeof(uint32_t), 0,
                           hipMemcpyHostToDevice);
}

bool splitk_applicable(int M, int64_t K) {
  return M >= 3 && M <= 8 && K > 0 && (K % kSliceK) == 0;
}

// Default launch shape (from sweeps of the decode-layer, stress and LM-head
// shapes): two x slices held per wavefront with a ring of 4 while the slice
// count is even and fits 8 wavefronts (K = 512 .. 4096), one held slice with a
// ring of 3 while it fits 16, else x streamed with KS slices per wavefront, KS
// the smallest divisor of the slice count that fits 8 wavefronts.
void splitk_default_shape(int64_t K, int* KS, int* XS, int* D) {
  const int64_t S = K / kSliceK;
  if (S % 2 == 0 && S / 2 <= sk_max_waves(2)) {
    *KS = 2, *XS = 2, *D = 4;
  } else if (S <= sk_max_waves(1)) {
    *KS = 1, *XS = 1, *D = 3;
  } else {
    int64_t ks = (S + sk_max_waves(0) - 1) / sk_max_waves(0);
    while (S % ks) ++ks;
    *KS = (int)ks, *XS = 0, *D = 3;
  }
}

// Launch with KS slices per wavefront (x held in registers for XS = KS = 1
// or 2 slices; XS = 0 streams x), D ring stages and `grid` workgroups (0: as
// many as fill the chip once).
hipError_t launch_gemv_splitk_shape(const SegDesc* d, int n, const uint16_t* x, int M,
                                    int64_t K, int KS, int XS, int D, int64_t grid,
                                    hipStream_t stream) {
  // shapes that are built: one held slice with a ring of 3 (a ring of 4 does
  // not fit the 128 registers of a 16-wavefront workgroup), two held slices
  // with a ring of 4 (5 spills), streamed x with rings of 3 and 4
  const bool built = (XS == 1 && D == 3) || (XS == 2 && D == 4) ||
                     (XS == 0 && (D == 3 || D == 4));
  if (!splitk_applicable(M, K) || n < 1 || n > kMaxSegments || KS < 1 || !built ||
      (XS != 0 && KS != XS))
    return hipErrorInvalidValue;
  const int64_t S = K / kSliceK;
  if (S % KS) return hipErrorInvalidValue;
  const int W = (int)(S / KS);
  if (W > sk_max_waves(XS)) return hipErrorInvalidValue;
  const SegTable tab = make_seg_table(d, n, 16);
  const int64_t tiles = tab.start[kMaxSegments];
  if (grid <= 0) grid = (int64_t)kSkCUs * (sk_max_waves(XS) == 16 ? 16 / W : 8 / W);
  if (grid > tiles) grid = tiles;
  if (grid > (1 << 20)) return hipErrorInvalidValue;
  const size_t lds = splitk_lds(W);
#define NVFP4_SK(MM, XX, DD)                                                              \
  hipLaunchKernelGGL((k_gemv_splitk<MM, XX, DD>), dim3((unsigned)grid), dim3(64 * W), lds, \
                     stream, tab, x, K, KS, g_splitk_spin_limit)
#define NVFP4_SKM(MM)                    \
  if (XS == 1) {                         \
    NVFP4_SK(MM, 1, 3);                  \
  } else if (XS == 2) {                  \
    NVFP4_SK(MM, 2, 4);                  \
  } else {                               \
    if (D == 3) NVFP4_SK(MM, 0, 3);      \
    else NVFP4_SK(MM, 0, 4);             \
  }
  switch (M) {
    case 3: NVFP4_SKM(3); break;
    case 4: NVFP4_SKM(4); break;
    case 5: NVFP4_SKM(5); break;
    case 6: NVFP4_SKM(6); break;
    case 7: NVFP4_SKM(7); break;
    default: NVFP4_SKM(8); break;
  }
#undef NVFP4_SKM
#undef NVFP4_SK
  return hipGetLastError();
}

hipError_t launch_gemv_splitk(const SegDesc* d, int n, const uint16_t* x, int M, int64_t K,
                              hipStream_t stream) {
  int KS, XS, D;
  splitk_default_shape(K, &KS, &XS, &D);
  return launch_gemv_splitk_shape(d, n, x, M, K, KS, XS, D, 0, stream);
}

}  // namespace nvfp4
