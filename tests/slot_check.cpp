// Host model check of the split-K GEMV's slot protocol (splitk_slots.h): W
// wavefronts deliver a partial of every tile of a workgroup's range in order,
// under random interleavings, through kSkSlots slots with arrival and
// release counters, using the same decision functions as the kernel.
//
// Checked, with an unbounded wait: every tile is summed exactly once, by the
// last of its W arrivals, from the W partials of that tile (no partial was
// overwritten before it was read), and no wavefront ever gives up. With a
// tiny wait bound and a schedule that lets one wavefront run ahead, waits are
// given up and the bookkeeping can break (a tile summed twice, never, or from
// another tile's partial): then the fault must have been recorded, so that
// no wrong result goes unreported. Prints "ok <cases>" or the first failure.
#include <cstdio>
#include <cstdint>
#include <vector>

#include "splitk_slots.h"

using namespace nvfp4;

static uint64_t rng = 0x2545F4914F6CDD1Dull;
static uint32_t next_u32() {
  rng ^= rng << 13;
  rng ^= rng >> 7;
  rng ^= rng << 17;
  return (uint32_t)(rng >> 16);
}

struct Partial {
  int tile = -1;
  bool poisoned = false;   // delivered by a wavefront that gave up its wait
};

struct Wave {
  int tl = 0;        // local tile being delivered
  int phase = 0;     // 0: math, 1: slot wait, 2: write, 3: arrive
  long spins = 0;
  bool give_up = false;
};

struct Result {
  bool ok = true;         // every tile summed exactly once from its own partials
  bool fault = false;     // some wavefront gave up a wait
  bool stuck = false;     // the model made no progress (a livelock)
  const char* why = "";
};

// One workgroup: W wavefronts, nt tiles, wait bound `limit` polls; `lead`
// >= 0 favours that wavefront (it runs ahead of the others).
static Result run(int W, int nt, long limit, int lead) {
  Result res;
  uint32_t cnt[kSkSlots] = {}, done[kSkSlots] = {};
  std::vector<std::vector<Partial>> slot(kSkSlots, std::vector<Partial>(W));
  std::vector<int> summed(nt, 0);
  std::vector<Wave> wv(W);
  int finished = 0;
  long steps = 0;
  while (finished < W) {
    if (++steps > 50000000L) {
      res.stuck = true;
      res.ok = false;
      res.why = "no progress";
      return res;
    }
    int w = (int)(next_u32() % W);
    if (lead >= 0 && next_u32() % 4 != 0) w = lead;
    Wave& a = wv[w];
    if (a.tl >= nt) continue;
    const int s = sk_slot(a.tl);
    const uint32_t round = sk_round(a.tl);
    switch (a.phase) {
      case 0:
        a.phase = 1;
        a.spins = 0;
        a.give_up = false;
        break;
      case 1:
        if (sk_slot_free(done[s], round)) {
          a.phase = 2;
        } else if (++a.spins >= limit) {
          a.give_up = true;
          res.fault = true;
          a.phase = 2;
        }
        break;
      case 2:
        slot[s][w].tile = a.tl;
        slot[s][w].poisoned = a.give_up;
        a.phase = 3;
        break;
      case 3: {
        const uint32_t old = cnt[s]++;
        if (sk_last_arrival(old, round, W)) {
          for (int v = 0; v < W; ++v)
            if (slot[s][v].tile != a.tl) {
              res.ok = false;
              res.why = "a tile summed from another tile's partial";
            }
          ++summed[a.tl];
          done[s] = round + 1;
        }
        a.phase = 0;
        if (++a.tl == nt) ++finished;
        break;
      }
    }
  }
  for (int t = 0; t < nt; ++t)
    if (summed[t] != 1) {
      res.ok = false;
      res.why = "a tile not summed exactly once";
    }
  return res;
}

int main() {
  int cases = 0;
  // normal operation: any interleaving, generous bound
  for (int W : {1, 2, 3, 5, 8, 16})
    for (int nt : {1, 3, 4, 5, 17, 64})
      for (int rep = 0; rep < 20; ++rep, ++cases) {
        const Result r = run(W, nt, 1L << 40, rep % 3 == 0 ? (int)(next_u32() % W) : -1);
        if (!r.ok || r.fault) {
          printf("FAIL normal W=%d nt=%d rep=%d: %s fault=%d\n", W, nt, rep, r.why,
                 (int)r.fault);
          return 1;
        }
      }
  // a tiny bound with one wavefront running ahead: waits are given up; any
  // wrong result must come with the fault recorded, and the model must not
  // livelock (every wait is bounded)
  int faults = 0;
  for (int W : {2, 4, 8, 16})
    for (int rep = 0; rep < 50; ++rep, ++cases) {
      const Result r = run(W, 40, 1, (int)(next_u32() % W));
      if (r.stuck || (!r.ok && !r.fault)) {
        printf("FAIL bounded W=%d rep=%d: %s fault=%d\n", W, rep, r.why, (int)r.fault);
        return 1;
      }
      faults += r.fault;
    }
  if (faults == 0) {
    printf("FAIL the bounded runs never gave up a wait\n");
    return 1;
  }
  printf("ok %d\n", cases);
  return 0;
}
