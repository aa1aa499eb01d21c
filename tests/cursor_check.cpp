// Host check of the segment cursor (nvfp4::SegCursor in segments.h) that the
// split-K GEMV kernel walks: random segment tables (empty segments included),
// every workgroup range of several grids, each tile checked against a plain
// scan of the table, and a step past the last tile that must leave the cursor
// on the last segment. Prints "ok <tables>" or the first failure.
#include <cstdio>
#include <cstdint>
#include <initializer_list>

#include "segments.h"

using nvfp4::SegCursor;
using nvfp4::SegDesc;
using nvfp4::SegTable;

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32() {
  rng = rng * 6364136223846793005ull + 1442695040888963407ull;
  return (uint32_t)(rng >> 33);
}

// plain scan: the segment holding unit u (u < total)
static int scan(const SegTable& t, int64_t u) {
  for (int k = 0; k < t.n; ++k)
    if (u >= t.start[k] && u < t.start[k + 1]) return k;
  return -1;
}

static bool check_cursor(const SegTable& t, const SegCursor& c, int64_t u, const char* what) {
  const int64_t total = t.start[nvfp4::kMaxSegments];
  if (c.k < 0 || c.k >= t.n) {
    std::printf("FAIL %s: k=%d outside [0, %d) at unit %lld\n", what, c.k, t.n, (long long)u);
    return false;
  }
  if (c.first != t.start[c.k] || c.end != t.start[c.k + 1]) {
    std::printf("FAIL %s: range [%lld, %lld) is not segment %d's\n", what, (long long)c.first,
                (long long)c.end, c.k);
    return false;
  }
  if (u < total) {
    const int k = scan(t, u);
    if (k != c.k) {
      std::printf("FAIL %s: unit %lld in segment %d, cursor on %d\n", what, (long long)u, k, c.k);
      return false;
    }
  } else if (c.k != t.n - 1) {
    std::printf("FAIL %s: past the end (%lld >= %lld) but k=%d of %d\n", what, (long long)u,
                (long long)total, c.k, t.n);
    return false;
  }
  return true;
}

int main() {
  int tables = 0;
  for (int rep = 0; rep < 4000; ++rep) {
    const int n = 1 + (int)(next_u32() % nvfp4::kMaxSegments);
    SegDesc d[nvfp4::kMaxSegments] = {};
    int64_t rows = 0;
    for (int s = 0; s < n; ++s) {
      const uint32_t kind = next_u32() % 4;
      d[s].N = kind == 0 ? 0 : kind == 1 ? 1 + next_u32() % 16 : 1 + next_u32() % 700;
      rows += d[s].N;
    }
    if (rows == 0) d[next_u32() % n].N = 1 + next_u32() % 40;
    const SegTable t = nvfp4::make_seg_table(d, n, 16);
    const int64_t tiles = t.start[nvfp4::kMaxSegments];
    ++tables;
    for (int64_t grid : {(int64_t)1, (int64_t)3, (int64_t)7, tiles, tiles + 5}) {
      for (int64_t b = 0; b < grid; ++b) {
        const int64_t t0 = tiles * b / grid;
        const int64_t nt = tiles * (b + 1) / grid - t0;
        if (nt <= 0) continue;
        SegCursor c;
        c.begin(t, t0);
        if (!check_cursor(t, c, t0, "begin")) return 1;
        for (int64_t u = t0 + 1; u <= t0 + nt; ++u) {
          c.seek(t, u);   // u = t0 + nt: one past the range (possibly past the total)
          if (!check_cursor(t, c, u, "seek")) return 1;
        }
        c.seek(t, tiles + 1000);
        if (!check_cursor(t, c, tiles + 1000, "far seek")) return 1;
      }
    }
  }
  std::printf("ok %d\n", tables);
  return 0;
}
