// segments.h -- the segment table of a multi-matrix GEMV launch.
//
// One launch can cover up to kMaxSegments weight matrices that share the same
// activations x[M, K] (q|k|v, gate|up): each segment has its own codes,
// scales, tensor scale, row count and output. The kernels number their work
// units (a group of rows: R rows of the vector-ALU kernel, a 16-row tile of
// the matrix-core kernels) across the segments in order; start[s] is the
// first unit of segment s. The table is passed by value as a kernel argument.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__) || defined(__HIP__)
#define NVFP4_HD __host__ __device__
#else
#define NVFP4_HD
#endif

namespace nvfp4 {

constexpr int kMaxSegments = 8;

struct SegTable {
  const uint8_t* codes[kMaxSegments];
  const uint8_t* scales[kMaxSegments];
  const float* gscale[kMaxSegments];
  float* y[kMaxSegments];
  int64_t N[kMaxSegments];
  int64_t start[kMaxSegments + 1];   // start[n] = total units
  int n;
};

// Host-side description of one segment.
struct SegDesc {
  const uint8_t* codes;
  const uint8_t* scales;
  const float* gscale;
  float* y;
  int64_t N;
};

// The table for n segments with `rows` rows per work unit.
inline SegTable make_seg_table(const SegDesc* d, int n, int64_t rows) {
  SegTable t = {};
  t.n = n;
  int64_t u = 0;
  for (int s = 0; s < n; ++s) {
    t.codes[s] = d[s].codes;
    t.scales[s] = d[s].scales;
    t.gscale[s] = d[s].gscale;
    t.y[s] = d[s].y;
    t.N[s] = d[s].N;
    t.start[s] = u;
    u += (d[s].N + rows - 1) / rows;
  }
  for (int s = n; s <= kMaxSegments; ++s) t.start[s] = u;
  return t;
}

// The segment of a unit index that only moves forward (a kernel's running
// tile): k is the segment and [first, end) its units. The cursor never moves
// past the last segment, so a unit at or past the total (one past a
// workgroup's last tile) leaves it on the last segment instead of reading
// beyond the table. Empty segments are stepped over. Host and device code.
struct SegCursor {
  int k;
  int64_t first, end;

  NVFP4_HD void begin(const SegTable& t, int64_t u) {
    k = 0;
    first = 0;
    end = t.start[1];
    advance(t, u);
  }
  // true when the segment changed
  NVFP4_HD bool seek(const SegTable& t, int64_t u) {
    return u < end ? false : advance(t, u);
  }
  NVFP4_HD bool advance(const SegTable& t, int64_t u) {
    bool moved = false;
    while (u >= end && k + 1 < t.n) {
      ++k;
      first = end;
      end = t.start[k + 1];
      moved = true;
    }
    return moved;
  }
};

#if defined(__HIPCC__) || defined(__HIP__)
// The segment of work unit u (wavefront-uniform) with its pointers. The scan
// reads only start[] (start is non-decreasing, so the segment is the number
// of later starts at or below u, empty segments included), then the entry is
// read with that index straight from the kernel arguments: a scan that
// carried every field through a chain of selects held the whole table in
// scalar registers, which overflowed into vector-register lanes (a few
// hundred v_writelane/v_readlane per wavefront).
struct Seg {
  const uint8_t* codes;
  const uint8_t* scales;
  const float* gscale;
  float* y;
  int64_t N;
  int64_t unit;   // unit index inside the segment
  int index;      // segment number
};

__device__ __forceinline__ Seg find_seg(const SegTable& t, int64_t u) {
  int k = 0;
#pragma unroll
  for (int j = 1; j < kMaxSegments; ++j) k += (j < t.n && u >= t.start[j]) ? 1 : 0;
  return Seg{t.codes[k], t.scales[k], t.gscale[k], t.y[k], t.N[k], u - t.start[k], k};
}

// The same for a launch whose units number below 2^31 (its launcher checks):
// the comparisons are 32-bit and stay on the scalar unit.
__device__ __forceinline__ Seg find_seg32(const SegTable& t, int u) {
  int k = 0;
#pragma unroll
  for (int j = 1; j < kMaxSegments; ++j) k += (j < t.n && u >= (int)t.start[j]) ? 1 : 0;
  return Seg{t.codes[k], t.scales[k], t.gscale[k], t.y[k], t.N[k], (int64_t)(u - (int)t.start[k]), k};
}
#endif

}  // namespace nvfp4
