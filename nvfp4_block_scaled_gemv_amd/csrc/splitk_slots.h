// splitk_slots.h -- the slot protocol of the split-K GEMV's cross-wavefront
// reduction, as plain functions shared by the kernel (gemv_splitk.hip) and a
// host model check.
//
// A workgroup's W wavefronts each produce a partial of every tile of its
// range, local tile tl = 0, 1, ... in order. Tile tl uses LDS slot
// tl % kSkSlots in round tl / kSkSlots. Per slot there are two counters:
// arrivals (cnt, all rounds) and rounds summed (done). A wavefront
//   1. waits until done >= round (the slot's previous round has been read),
//      at most a bounded number of polls;
//   2. writes its partial into the slot and then adds 1 to cnt;
//   3. if the count before its add was round * W + W - 1 it is the last of
//      the W: it sums the W partials in wavefront order, sets done to
//      round + 1 and stores the tile.
// A wavefront that gives up in step 1 has found the protocol broken (a
// wavefront kSkSlots tiles ahead of one that does not progress): it records
// a fault and still arrives (so that no other wavefront waits for it without
// bound), with a NaN partial. From then on the counters may no longer match
// the tiles, so the call's results are invalid; the fault word says so
// whenever that can have happened (tiles summed from the NaN partial also
// show it).
#pragma once

#include <stdint.h>

#include "segments.h"   // NVFP4_HD

namespace nvfp4 {

constexpr int kSkSlots = 4;

NVFP4_HD inline int sk_slot(int tl) { return tl % kSkSlots; }
NVFP4_HD inline uint32_t sk_round(int tl) { return (uint32_t)(tl / kSkSlots); }

// The slot of a tile in `round` may be written once `done` (rounds summed)
// has reached it.
NVFP4_HD inline bool sk_slot_free(uint32_t done, uint32_t round) { return done >= round; }

// `old` is the slot's arrival count before this wavefront's add: true for the
// last of the W arrivals of `round`.
NVFP4_HD inline bool sk_last_arrival(uint32_t old, uint32_t round, int W) {
  return old == round * (uint32_t)W + (uint32_t)(W - 1);
}

}  // namespace nvfp4
