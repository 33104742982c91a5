// pipeline.hpp -- bookkeeping shared by the persistent, wave-specialised
// kernels (flat scan, segmented scan, compaction).
//
// A workgroup holds one control wave and D data waves and moves each tile
// through three phases: loads issued (phase k-1), scanned and parked in LDS
// with its aggregate published (phase k), looked back for two phases after
// its aggregate went out and stored (phase k+2).  PipeTiles is the window of
// tile ids the workgroup works on in one phase.
#pragma once

#include <stdint.h>

namespace dwps {

// LDS park slots: the tiles parked during phases k, k+1 and k+2.
constexpr int kParkSlots = 3;

// Tile ids of the pipeline, identical in every wave of the workgroup
// (num_tiles = none): prev2 waits for its prefix, prev and cur are parked or
// being parked, f1 and f2 are in flight.  Every value comes from LDS through
// readfirstlane, so the compiler keeps them in scalar registers and branches
// on them with scalar branches.
struct PipeTiles {
    uint32_t prev2, prev, cur, f1, f2;
    __device__ __forceinline__ bool drained(uint32_t num_tiles) const {
        return prev < num_tiles ? false : (cur >= num_tiles && f1 >= num_tiles && f2 >= num_tiles);
    }
    __device__ __forceinline__ void advance(uint32_t after, uint32_t num_tiles) {
        prev2 = prev;
        prev = cur;
        cur = f1;
        f1 = f2;
        f2 = (f2 < num_tiles) ? after : num_tiles;
    }
};

__device__ __forceinline__ uint32_t uniform(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ uint32_t next_slot(uint32_t slot) { return slot == kParkSlots - 1 ? 0u : slot + 1u; }

// The tile after f2: the next one of its group of G, or the first tile of a
// new group claimed with a ticket (`ticket` is the claimed group index).
template <int G>
__device__ __forceinline__ bool needs_ticket(uint32_t f2, uint32_t num_tiles) {
    return f2 < num_tiles && (f2 + 1u) % G == 0u;
}
template <int G>
__device__ __forceinline__ uint32_t tile_after(uint32_t f2, uint32_t num_tiles, bool ticketed, uint32_t ticket) {
    if (ticketed) return (ticket < (num_tiles + G - 1u) / G) ? ticket * G : num_tiles;
    return (f2 < num_tiles && f2 + 1u < num_tiles) ? f2 + 1u : num_tiles;
}

}  // namespace dwps
