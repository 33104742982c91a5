// pipeline.hpp -- bookkeeping shared by the persistent, wave-specialised
// kernels (flat scan, segmented scan, compaction).
//
// A workgroup holds one control wave and D data waves and moves each tile
// through a fixed sequence of phases: loads issued, scanned (aggregate
// published after the phase's barrier B), parked in LDS, looked back for and
// stored -- two phases after the park (LAG 2: segmented scan), or three
// with the look-back resolved the phase before (LAG 3: flat scan,
// compaction; in compaction and the two-word flat kernels the last tiles
// are stored together after a closing phase).
// PipeTiles is the window of tile ids the workgroup works on in one phase.
#pragma once

#include <stdint.h>

#include "dwps_device.hpp"
#include "ws_device.hpp"

namespace dwps {

// LDS park slots: the tiles parked during the last three phases.
constexpr int kParkSlots = 3;

// Tile ids of the pipeline, identical in every wave of the workgroup
// (num_tiles = none): f2 and f1 are in flight and being scanned, cur is
// being made tile-relative or parked, prev, prev2 (and prev3) are parked;
// the tile stored in a phase is prev2 (LAG 2) or prev3 (LAG 3).  Every value
// comes from LDS through readfirstlane, so the compiler keeps them in scalar
// registers and branches on them with scalar branches.
struct PipeTiles {
    uint32_t prev3, prev2, prev, cur, f1, f2;
    // nothing left after this phase's store
    template <int LAG>
    __device__ __forceinline__ bool drained(uint32_t num_tiles) const {
        return (LAG == 3 ? prev2 >= num_tiles : true) && prev >= num_tiles && cur >= num_tiles &&
               f1 >= num_tiles && f2 >= num_tiles;
    }
    __device__ __forceinline__ bool drained(uint32_t num_tiles) const { return drained<2>(num_tiles); }
    __device__ __forceinline__ void advance(uint32_t after, uint32_t num_tiles) {
        prev3 = prev2;
        prev2 = prev;
        prev = cur;
        cur = f1;
        f1 = f2;
        f2 = (f2 < num_tiles) ? after : num_tiles;
    }
};

__device__ __forceinline__ uint32_t uniform(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

// Per-tile statistics rows of the instrumented builds: kStatsWords uint32.
// Words 0-3: the tile's look-back (polls, windows, time, stalled polls).
// Words 4-7: the phase that scanned the tile, as the control wave saw it --
// from the start of the phase to reaching barrier B, waiting at B, from
// leaving B to reaching barrier A, waiting at A -- which add up to the
// phase's length: a long wait means the data waves came later.
// Words 8-12, a timeline (low 32 bits of the counter): [8] start of the
// tile's scan phase, [9] start of the phase that stored it, [10] the
// workgroup, [11] the workgroup's start, [12] (last tile a workgroup
// stored only) the time its control wave finished.  Words 13-14: when the
// phase that stored the tile scanned none (the drain), that phase's parts
// as in 4-7, 16 bits each.  Word 15: in the flat kernel data wave 0's view
// of the phase that scanned the tile (DataClock), in the segmented kernel
// the data waves' arrivals at barrier B of that phase (record_arrivals in
// segscan.hip).  Times in ticks of the 100 MHz real-time counter.
constexpr int kStatsWords = 16;

__device__ __forceinline__ uint32_t realtime32() { return (uint32_t)__builtin_amdgcn_s_memrealtime(); }

template <bool STATS>
struct PhaseClock {
    uint64_t start = 0, t_reach_b = 0, t_leave_b = 0, t_reach_a = 0;
    __device__ __forceinline__ void begin() {
        if (STATS) start = __builtin_amdgcn_s_memrealtime();
    }
    __device__ __forceinline__ void reach_b() {
        if (STATS) t_reach_b = __builtin_amdgcn_s_memrealtime();
    }
    __device__ __forceinline__ void leave_b() {
        if (STATS) t_leave_b = __builtin_amdgcn_s_memrealtime();
    }
    __device__ __forceinline__ void reach_a() {
        if (STATS) t_reach_a = __builtin_amdgcn_s_memrealtime();
    }
    // after barrier A, by lane 0 of the control wave: the phase of the tile
    // scanned (f1) and the start of the store phase of the tile stored (s)
    __device__ __forceinline__ void record(uint32_t *stats, uint32_t f1, uint32_t s, uint32_t num_tiles,
                                           uint32_t entry, bool writer) {
        if (STATS && writer) {
            const uint64_t t = __builtin_amdgcn_s_memrealtime();
            if (f1 < num_tiles) {
                uint32_t *row = stats + (uint64_t)kStatsWords * f1;
                uint4 r;
                r.x = (uint32_t)(t_reach_b - start);
                r.y = (uint32_t)(t_leave_b - t_reach_b);
                r.z = (uint32_t)(t_reach_a - t_leave_b);
                r.w = (uint32_t)(t - t_reach_a);
                reinterpret_cast<uint4 *>(row)[1] = r;
                row[8] = (uint32_t)start;
                row[10] = blockIdx.x;
                row[11] = entry;
            }
            if (s < num_tiles) {
                uint32_t *row = stats + (uint64_t)kStatsWords * s;
                row[9] = (uint32_t)start;
                if (f1 >= num_tiles) {
                    // a phase that scanned nothing (the drain): its parts,
                    // two per word (16 bits each)
                    row[13] = (uint32_t)(t_reach_b - start) | ((uint32_t)(t_leave_b - t_reach_b) << 16);
                    row[14] = (uint32_t)(t_reach_a - t_leave_b) | ((uint32_t)(t - t_reach_a) << 16);
                }
            }
        }
    }
    // after the last phase: the store phase of the last tile and the end
    __device__ __forceinline__ void finish(uint32_t *stats, uint32_t s, uint32_t num_tiles, bool writer) {
        if (STATS && writer && s < num_tiles) {
            stats[(uint64_t)kStatsWords * s + 9] = (uint32_t)start;
            stats[(uint64_t)kStatsWords * s + 12] = realtime32();
        }
    }
    // a tile of the closing store step (after the last barrier): its store
    // step's start, and for the workgroup's last tile the end
    __device__ __forceinline__ void closing(uint32_t *stats, uint32_t s, uint32_t num_tiles, bool last,
                                            bool writer) {
        if (STATS && writer && s < num_tiles) {
            const uint32_t t = realtime32();
            stats[(uint64_t)kStatsWords * s + 9] = t;
            if (last) stats[(uint64_t)kStatsWords * s + 12] = t;
        }
    }
};

// Data wave 0's view of a phase (instrumented flat scan), word 15 of the
// scanned tile's row, three 10-bit fields in ticks (saturating at 1023):
// bits 0-9 from the start of the phase (leaving barrier A of the phase
// before) to the end of the scan, just before barrier B; bits 10-19 from
// leaving barrier B to the last store of the stored tile issued; bits 20-29
// from leaving barrier B to reaching barrier A (the park and the next tile's
// id included).
template <bool STATS>
struct DataClock {
    uint32_t start = 0, scanned = 0, left_b = 0, stored = 0;
    __device__ __forceinline__ void begin() {
        if (STATS) start = realtime32();
    }
    __device__ __forceinline__ void scan_done() {
        if (STATS) scanned = realtime32();
    }
    __device__ __forceinline__ void leave_b() {
        if (STATS) left_b = realtime32();
    }
    __device__ __forceinline__ void store_done() {
        if (STATS) stored = realtime32();
    }
    __device__ __forceinline__ void reach_a(uint32_t *stats, uint32_t f1, uint32_t num_tiles, bool writer) {
        if (STATS && writer && f1 < num_tiles) {
            const uint32_t t = realtime32();
            auto sat = [](uint32_t v) { return v < 1023u ? v : 1023u; };
            stats[(uint64_t)kStatsWords * f1 + 15] =
                sat(scanned - start) | (sat(stored - left_b) << 10) | (sat(t - left_b) << 20);
        }
    }
};

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

// The closing phase of a LAG 3 pipeline built with CLOSE (its data waves
// must be built to match: they store after it when after_closing holds):
// the first phase with no tile to load or scan.  Its control wave resolves
// the prefixes of all three tiles still waiting (prev2, prev and cur, in
// that order; cur was scanned in the phase before, so every aggregate they
// need is out), publishes them, and leaves their exclusive prefixes in
// `close_prefix`; after its barrier A both kinds of wave leave the loop and
// the data waves store those three tiles from their park slots at once
// (closing_slot) instead of one per phase over three more phases.  The
// look-backs of prev and cur run one and two phases earlier than in the
// steady state, when a predecessor is a little more likely to be
// unpublished: a stalled poll costs a round trip.
__device__ __forceinline__ bool closing_phase(const PipeTiles &pt, uint32_t num_tiles) {
    return pt.f1 >= num_tiles && pt.f2 >= num_tiles && pt.cur < num_tiles;
}
// After barrier A of the closing phase (the tiles advanced, `slot` moved on):
// the park slot of prev3, prev2 and prev (i = 0, 1, 2).
__device__ __forceinline__ uint32_t closing_slot(uint32_t slot, int i) {
    return (slot + (uint32_t)i) % (uint32_t)kParkSlots;
}
__device__ __forceinline__ bool after_closing(const PipeTiles &pt, uint32_t num_tiles) {
    return pt.cur >= num_tiles && pt.f1 >= num_tiles && pt.f2 >= num_tiles;
}

// Control wave of the LAG 3 pipeline (the data waves store prev3): the
// look-back of prev2 is resolved one phase before its tile is stored, and
// its poll straddles barrier B.  Per phase: hand the data waves prev3's
// prefix (resolved in the phase before), issue the first poll of prev2's
// look-back, pass barrier B at once -- the data waves store while the poll
// is in flight -- then finish the look-back, publish prev2's prefix and
// f1's aggregate, and meet the data waves at barrier A.  The poll is as
// fresh as in the two-phase pipeline (issued at the start of the phase that
// resolves it); only its round trip moves off the path to barrier B.
template <class Op, int D, int LB_K, int G, bool STATS, bool PAIR_PREFIX, bool BLOCKED = true, bool CLOSE = false,
          class Shared, class FB>
__device__ __forceinline__ void control_loop3(PipeTiles pt, Shared &sh, uint32_t num_tiles, uint32_t *ctr,
                                              uint64_t *desc, typename Op::T *total, uint32_t *stats,
                                              int aggregate_only, LookbackCfg cfg, const FB &fb, uint32_t lane,
                                              uint32_t t_entry = 0) {
    using T = typename Op::T;
    using W = WordsFor<Op>;
    T agg_prev = Op::id(), agg_prev2 = Op::id(), agg_prev3 = Op::id();
    T incl_last = Op::id();   // inclusive prefix of the tile resolved one phase ago
    T excl_next = Op::id();   // exclusive prefix of prev3, resolved one phase ago
    T agg_next = Op::id();    // aggregate of cur, published at the end of the phase before
    constexpr bool kPairPrefix = PAIR_PREFIX && G > 1;
    for (int par = 0;; par ^= 1) {
        PhaseClock<STATS> clk;
        clk.begin();
        const T agg = agg_next;
        if (lane == 0) {
            sh.prefix = excl_next;
            if (total && pt.prev3 == num_tiles - 1) *total = Op::op(excl_next, agg_prev3);
        }
        const bool have = pt.prev2 < num_tiles && pt.prev2 != 0;
        const bool look = have && (pt.prev2 % G == 0u || (STATS && aggregate_only));
        const bool closing = CLOSE && closing_phase(pt, num_tiles);
        Window<LB_K, W::WORDS> win;
        if (look) window_load<Op, LB_K, BLOCKED>(desc, (int64_t)pt.prev2 - 1, lane, win);
        clk.reach_b();
        __syncthreads();  // B: prev3's prefix is in LDS
        clk.leave_b();
        LookbackStats st;
        uint64_t t0 = 0;
        if (STATS) t0 = __builtin_amdgcn_s_memrealtime();
        T excl = Op::id();
        if (look)
            excl = lookback<Op, LB_K, STATS, BLOCKED>(desc, pt.prev2, lane, st, ctr, cfg, agg_prev2, true, fb, &win);
        else if (have)
            excl = incl_last;
        if (lane == 0) {
            if (STATS && pt.prev2 < num_tiles) {
                const uint64_t t1 = __builtin_amdgcn_s_memrealtime();
                reinterpret_cast<uint4 *>(stats)[(kStatsWords / 4) * pt.prev2] =
                    make_uint4(st.polls, st.windows, (uint32_t)(t1 - t0), st.stalls);
            }
            if (!(STATS && aggregate_only)) {
                const bool early = kPairPrefix && pt.prev2 % G != 0u && pt.prev2 - 1u != 0u;
                if (have && !early) W::publish(desc, pt.prev2, cfg.tf, ST_PREFIX, Op::op(excl, agg_prev2));
                if (kPairPrefix && look && pt.prev == pt.prev2 + 1u && pt.prev < num_tiles)
                    W::publish(desc, pt.prev, cfg.tf, ST_PREFIX, Op::op(Op::op(excl, agg_prev2), agg_prev));
            }
        }
        // the wave totals of f1 are complete: its aggregate goes out now
        agg_next = Op::id();
        if (pt.f1 < num_tiles) {
#pragma unroll
            for (int w = 0; w < D; ++w) agg_next = Op::op(agg_next, sh.wt[par ^ 1][w]);
            // (a debug setting withholds aggregates, so that look-backs
            // reaching this tile stall and its aggregate comes from a fallback)
            const bool withhold = pt.f1 != 0 && (cfg.flags & kDbgWithholdAggregates);
            if (lane == 0 && !withhold)
                W::publish(desc, pt.f1, cfg.tf, pt.f1 == 0 ? ST_PREFIX : ST_AGGREGATE, agg_next);
        }
        if constexpr (CLOSE) {
          if (closing) {
            // prev and cur resolved now as well (see closing_phase), in one
            // loop, so that the look-back is not inlined twice
            T ex1 = Op::id(), ex2 = Op::id();
            T incl = Op::op(excl, agg_prev2);  // prev2's inclusive prefix, when it exists
#pragma unroll 1
            for (int i = 0; i < 2; ++i) {
                const uint32_t u = i == 0 ? pt.prev : pt.cur;
                const T au = i == 0 ? agg_prev : agg;
                if (u >= num_tiles) continue;
                const bool u_look = u != 0 && (u % G == 0u || (STATS && aggregate_only));
                LookbackStats su;
                uint64_t u0 = 0;
                if (STATS) u0 = __builtin_amdgcn_s_memrealtime();
                // a tile that is not the first of its group follows its
                // group's previous tile in this workgroup
                T e = Op::id();
                if (u_look)
                    e = lookback<Op, LB_K, STATS, BLOCKED>(desc, u, lane, su, ctr, cfg, au, true, fb);
                else if (u != 0)
                    e = incl;
                if (i == 0)
                    ex1 = e;
                else
                    ex2 = e;
                incl = Op::op(e, au);
                if (lane == 0) {
                    if (STATS) {
                        const uint64_t u1 = __builtin_amdgcn_s_memrealtime();
                        reinterpret_cast<uint4 *>(stats)[(kStatsWords / 4) * u] =
                            make_uint4(su.polls, su.windows, (uint32_t)(u1 - u0), su.stalls);
                    }
                    // prev's prefix went out already with prev2's (pair prefix)
                    const bool sent = i == 0 && kPairPrefix && look && pt.prev == pt.prev2 + 1u;
                    if (u != 0 && !sent && !(STATS && aggregate_only))
                        W::publish(desc, u, cfg.tf, ST_PREFIX, incl);
                    if (total && u == num_tiles - 1u) *total = incl;
                }
            }
            if (total && lane == 0 && pt.prev2 == num_tiles - 1u) *total = Op::op(excl, agg_prev2);
            if (lane == 0) {
                sh.close_prefix[0] = excl;
                sh.close_prefix[1] = ex1;
                sh.close_prefix[2] = ex2;
            }
            clk.reach_a();
            __syncthreads();  // A: the closing prefixes are in LDS
            clk.record(stats, pt.f1, pt.prev3, num_tiles, t_entry, lane == 0);
            // cur is the workgroup's last tile
            clk.closing(stats, pt.prev2, num_tiles, false, lane == 0);
            clk.closing(stats, pt.prev, num_tiles, false, lane == 0);
            clk.closing(stats, pt.cur, num_tiles, true, lane == 0);
            break;
          }
        }
        excl_next = excl;
        incl_last = Op::op(excl, agg_prev2);
        agg_prev3 = agg_prev2;
        agg_prev2 = agg_prev;
        agg_prev = agg;
        if (pt.template drained<3>(num_tiles)) {
            clk.finish(stats, pt.prev3, num_tiles, lane == 0);
            break;
        }
        clk.reach_a();
        __syncthreads();  // A: the next tile id is in LDS
        clk.record(stats, pt.f1, pt.prev3, num_tiles, t_entry, lane == 0);
        pt.advance(uniform(sh.next), num_tiles);
    }
}

}  // namespace dwps
