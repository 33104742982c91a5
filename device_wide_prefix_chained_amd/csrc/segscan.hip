// segscan.hip -- segmented uint32 sum scan over CSR offsets, single pass.
//
// Contract: "GPUSegmentedScan", sections "Prefix scans and segmented scans",
// "Contract" and "Limitations" (segment s is [offsets[s], offsets[s+1]), the
// running total restarts at every segment, empty segments write nothing,
// offsets are trusted on the hot path).  The scan itself is the chained scan
// with the operator of the carried segment flag ("Parallel Prefix Sum (Scan),
// in depth", section "What scan builds"):
//     (f1, v1) (+) (f2, v2) = (f1 | f2,  f2 ? v2 : v1 + v2).
//
// Strategy selection by segment size, inside one pass (the segmented-scan
// page's "Performance notes" call for it without building it):
//   * a segment that starts and ends inside one lane's 4 elements, one wave's
//     span or one tile is finished by the lane-serial, DPP wave or LDS block
//     layer -- it never waits on another workgroup;
//   * a tile that contains a segment start knows its carry-out without
//     looking back (the sum since its last start), so it publishes PREFIX
//     together with its aggregate and cuts every look-back chain that
//     reaches it;
//   * only a tile whose first element is not a segment start needs a carry,
//     and only the first tile of a ticket group looks back for it -- long
//     segments chain through start-free tiles exactly like the flat scan.
//
// One launch per call: the persistent, wave-specialised pipeline of the
// flat scan (one control wave, D data waves, look-back two phases behind the
// aggregate) on a workspace that keeps itself ready between calls.  The segment starts never go through memory as flags: while
// the data waves load a tile, the control wave reads the tile's offsets and
// sets the starts as bits of an LDS bitmap, which the data waves read when
// they scan the tile in the next phase.  To find those offsets, a sample of
// the offsets (every 512th, loaded into LDS once per workgroup) brackets the
// tile's first start within 512 entries, and one round of contiguous loads
// from there fetches the starts (repeated offsets -- empty segments -- set
// the same bit).
#include <hip/hip_runtime.h>

#include "dwps_device.hpp"
#include "host_common.hpp"
#include "pipeline.hpp"
#include "tile_io.hpp"

namespace dwps {

// Segment starts of one tile [tb, te) as bits of an LDS bitmap (bit i =
// element tb + i), found by one wave in the sorted offsets a[0, count).
//   * StartIndex: `sample` (LDS) holds every stride-th entry, a[k * stride]
//     for k < ns (ns <= kSampleMax); counting the sample entries below tb
//     brackets the first entry >= tb within one stride, and rounds of
//     64 * kStartProbes evenly spaced probes narrow the bracket further only
//     while it is wider than that (more than 2^19 offsets).
//   * Then batches of 64 * kStartProbes consecutive entries are loaded from
//     the bracket's start, and every loaded offset in [tb, te) sets its bit
//     (repeated offsets -- empty segments -- set the same bit), until an
//     entry at or past te or the end of the array.
// Loads are straight-line (out-of-range lanes read an in-range entry and are
// ignored), so reads stay inside [0, count) even if `a` is not sorted.
constexpr uint32_t kSampleMax = 1024u;
constexpr int kStartProbes = 8;
constexpr uint32_t kStartBatch = 64u * (uint32_t)kStartProbes;

struct StartIndex {
    const uint32_t *a;       // offsets
    uint32_t count;          // num_segments + 1
    uint32_t stride;         // sample stride (>= kStartBatch)
    uint32_t ns;             // sample entries
    const uint32_t *sample;  // LDS

    __device__ static StartIndex make(const uint32_t *offsets, uint32_t num_segments, const uint32_t *sample) {
        const uint32_t count = num_segments + 1u;  // < 2^32: checked on the host
        const uint32_t stride = max(kStartBatch, (uint32_t)(((uint64_t)count + kSampleMax - 1u) / kSampleMax));
        return StartIndex{offsets, count, stride, (uint32_t)(((uint64_t)count + stride - 1u) / stride), sample};
    }
    // Fill the sample, by the one wave that uses it (its own LDS writes are
    // visible to its later reads without a barrier).
    __device__ void load_sample(uint32_t *dst, uint32_t lane) const {
        for (uint32_t k = lane; k < ns; k += 64u) dst[k] = a[(uint64_t)k * stride];
    }
    // Index at or before the first entry >= tb, at most kStartBatch before it.
    __device__ uint32_t bracket(uint32_t tb, uint32_t lane) const {
        constexpr uint32_t P = kStartBatch;
        uint32_t c = 0;  // sample entries below tb: a prefix of the sample
        for (uint32_t k0 = 0; k0 < ns; k0 += 64u) {
            const uint32_t k = k0 + lane;
            c += (uint32_t)__builtin_popcountll(ballot(k < ns && sample[k < ns ? k : 0u] < tb));
        }
        // the first entry >= tb lies in [lo, hi]
        uint32_t lo = 0, hi = 0;
        if (c != 0u) {
            lo = (c - 1u) * stride + 1u;  // (c - 1) * stride < count
            hi = (uint32_t)min((uint64_t)count, (uint64_t)c * stride);
        }
        while (hi - lo > P) {
            const uint32_t s = (hi - lo + P - 1u) / P;
            uint32_t v[kStartProbes];
            bool in[kStartProbes];
#pragma unroll
            for (int j = 0; j < kStartProbes; ++j) {
                const uint64_t p = lo + (uint64_t)((uint32_t)j * 64u + lane) * s;
                in[j] = p < hi;
                v[j] = a[in[j] ? (uint32_t)p : lo];
            }
            uint32_t cp = 0;
#pragma unroll
            for (int j = 0; j < kStartProbes; ++j) cp += (uint32_t)__builtin_popcountll(ballot(in[j] && v[j] < tb));
            if (cp == 0u) {
                hi = lo;
            } else {
                const uint32_t b = lo;
                lo = b + (cp - 1u) * s + 1u;  // probe cp - 1 was in range
                hi = (uint32_t)min((uint64_t)hi, (uint64_t)b + (uint64_t)cp * s);
            }
        }
        return lo;
    }
    // The batch of entries from `base` (lane l, load j: entry base + 64 j + l).
    __device__ void load_batch(uint32_t base, uint32_t lane, uint32_t (&v)[kStartProbes]) const {
#pragma unroll
        for (int j = 0; j < kStartProbes; ++j) {
            const uint64_t idx = (uint64_t)base + (uint32_t)j * 64u + lane;
            v[j] = a[idx < count ? (uint32_t)idx : count - 1u];
        }
    }
    // Set the bits of the batch's offsets in [tb, te); true if the entries
    // after the batch may still hold starts of the tile.
    __device__ bool mark(const uint32_t (&v)[kStartProbes], uint32_t base, uint32_t tb, uint32_t te, uint32_t lane,
                         uint32_t *bits) const {
#pragma unroll
        for (int j = 0; j < kStartProbes; ++j) {
            const uint64_t idx = (uint64_t)base + (uint32_t)j * 64u + lane;
            if (idx < count && v[j] >= tb && v[j] < te) atomicOr(&bits[(v[j] - tb) >> 5], 1u << ((v[j] - tb) & 31u));
        }
        // entry base + kStartBatch - 1 is lane 63's last load
        return (uint64_t)base + kStartBatch < count &&
               (uint32_t)__builtin_amdgcn_readlane((int)v[kStartProbes - 1], 63) < te;
    }
    // Clear `words` bitmap words (16-byte aligned, a multiple of 4), then
    // mark the batches from `base` on (the first batch already loaded into v).
    __device__ void finish(uint32_t (&v)[kStartProbes], uint32_t base, uint32_t tb, uint32_t te, uint32_t lane,
                           uint32_t *bits, uint32_t words) const {
        // LDS operations of one wave complete in order: the clear before the marks
        for (uint32_t i = 4u * lane; i < words; i += 256u) *reinterpret_cast<v4u *>(bits + i) = v4u{0u, 0u, 0u, 0u};
        if (base >= count) return;
        while (mark(v, base, tb, te, lane, bits)) {
            base += kStartBatch;
            load_batch(base, lane, v);
        }
    }
};

struct SegPair {
    uint32_t f;  // 1 if the covered range contains a segment start
    uint32_t v;  // sum since the last start in the range (the whole range if none)
};
__device__ __forceinline__ SegPair seg_op(SegPair a, SegPair b) {
    return SegPair{a.f | b.f, b.f ? b.v : a.v + b.v};
}

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ void seg_dpp_step(uint32_t &f, uint32_t &v) {
    const uint32_t fl = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)f, CTRL, ROW_MASK, 0xF, false);
    const uint32_t vl = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, false);
    v = f ? v : vl + v;
    f = f | fl;
}

// Inclusive segmented scan of (f, v) pairs across the 64 lanes.
__device__ __forceinline__ void wave_seg_inclusive(uint32_t &f, uint32_t &v) {
    seg_dpp_step<0x111>(f, v);
    seg_dpp_step<0x112>(f, v);
    seg_dpp_step<0x114>(f, v);
    seg_dpp_step<0x118>(f, v);
    seg_dpp_step<0x142, 0xA>(f, v);
    seg_dpp_step<0x143, 0xC>(f, v);
}

// Segmented tile shape: D data waves x Q groups of four elements per lane.
// The segmented scan takes several times the vector instructions of the
// flat scan per element, and a SIMD issues its waves oldest first, so the
// last data wave on each SIMD reaches barrier B late.  Twelve data waves of
// four groups (13 waves per workgroup) spread the same 12 288-element tile
// over more waves than eight of six and shorten that wait.
#ifndef DWPS_SEG_D
#define DWPS_SEG_D 12
#endif
#ifndef DWPS_SEG_Q
#define DWPS_SEG_Q 4
#endif
constexpr int kSegD = DWPS_SEG_D;
constexpr int kSegQ = DWPS_SEG_Q;
#ifndef DWPS_SEG_G
#define DWPS_SEG_G 2
#endif
constexpr int kSegG = DWPS_SEG_G;  // tiles claimed per ticket
constexpr int kSegThreads = (kSegD + 1) * 64;
constexpr uint32_t kSegTile = (uint32_t)kSegD * kSegQ * 256u;
constexpr uint32_t kSegWords = kSegTile / 32u;  // bitmap words per tile

// ---------------------------------------------------------------------------
// the persistent pipeline
// ---------------------------------------------------------------------------
template <int D, int Q>
struct SegShared {
    v4u park[kParkSlots][D * Q * 64];  // tile-relative outputs (carry into the tile = 0)
    uint32_t park_first[kParkSlots];   // first segment start of each parked tile (tile-local; TILE if none)
    uint32_t wf[2][D], wv[2][D];       // wave totals (pairs), double-buffered by phase parity
    uint32_t wfirst[2][D];             // first segment start in each wave's span (TILE if none)
    alignas(16) uint32_t starts[2][kSegWords];  // start bitmaps of f2 (written) and f1 (read), by phase parity
    alignas(16) uint32_t fb_starts[kSegWords];  // start bitmap of a tile a fallback reduces
    uint32_t sample[kSampleMax];       // every stride-th offset (StartIndex)
    uint32_t next;
    uint32_t carry;                    // carry into prev2
    uint32_t arrive[2][D];             // instrumented builds: each data wave's arrival at barrier B, by parity
};

// Register state of one wave's span: the values.
template <int Q>
struct SegSpan {
    WaveSpan<SumU32, Q> x;
    template <bool VEC>
    __device__ __forceinline__ void load(const uint32_t *values, uint32_t tile, uint64_t lane_off, uint32_t n,
                                         bool valid) {
        const uint64_t base = (uint64_t)tile * kSegTile;
        x.template load<VEC>(values, base + lane_off, n, base + kSegTile <= n, valid);
    }
};

// A look-back's fallback: reduce tile p from scratch -- its start bitmap
// built from the offsets into `bits` (LDS), then values and start bits in
// rows of 256 elements, lane-serial pairs of four, the DPP pair scan across
// the lanes, rows folded in order -- and return the descriptor word its
// owner publishes first: PREFIX with the carry-out when the tile holds a
// start (or is tile 0), AGGREGATE with its sum otherwise.  Control wave,
// rarely.
struct SegFallback {
    const uint32_t *values;
    StartIndex idx;
    uint32_t *bits;
    uint32_t n;
    __device__ DescVal<uint32_t> operator()(uint32_t p, uint32_t lane) const {
        constexpr uint32_t ROWS = kSegTile / 256u;
        constexpr uint32_t BATCH = ROWS % 8u == 0u ? 8u : ROWS % 7u == 0u ? 7u : ROWS % 6u == 0u ? 6u
                                                                            : ROWS % 5u == 0u ? 5u : 4u;
        static_assert(ROWS % BATCH == 0, "whole batches of rows");
        {
            const uint32_t tb = p * kSegTile;
            const uint32_t te = (uint32_t)min((uint64_t)n, (uint64_t)tb + kSegTile);
            const uint32_t lo = idx.bracket(tb, lane);
            uint32_t v[kStartProbes];
            idx.load_batch(lo, lane, v);
            idx.finish(v, lo, tb, te, lane, bits, kSegWords);
        }
        const uint64_t base = (uint64_t)p * kSegTile + 4u * lane;
        const uint32_t wbase = lane >> 3;
        const uint32_t sh4 = 4u * (lane & 7u);
        SegPair acc{0u, 0u};
        for (uint32_t r = 0; r < ROWS; r += BATCH) {
            uint32_t x[BATCH][4], fl[BATCH];
#pragma unroll
            for (uint32_t k = 0; k < BATCH; ++k) {
                fl[k] = (bits[wbase + (r + k) * 8u] >> sh4) & 0xFu;
#pragma unroll
                for (uint32_t e = 0; e < 4; ++e) {
                    const uint64_t i = base + (uint64_t)(r + k) * 256u + e;
                    x[k][e] = i < n ? values[i] : 0u;
                }
            }
#pragma unroll
            for (uint32_t k = 0; k < BATCH; ++k) {
                uint32_t v = 0u;
#pragma unroll
                for (uint32_t e = 0; e < 4; ++e) v = ((fl[k] >> e) & 1u) ? x[k][e] : v + x[k][e];
                uint32_t f = fl[k] ? 1u : 0u;
                wave_seg_inclusive(f, v);
                acc = seg_op(acc, SegPair{(uint32_t)__builtin_amdgcn_readlane((int)f, 63),
                                          (uint32_t)__builtin_amdgcn_readlane((int)v, 63)});
            }
        }
        return DescVal<uint32_t>{(acc.f || p == 0) ? ST_PREFIX : ST_AGGREGATE, acc.v};
    }
};

// Instrumented builds: when the data waves reached barrier B in the phase
// that scanned tile f1, as word 15 of its statistics row -- bits 0-9 the
// first data wave and bits 10-19 the last one (ticks of the real-time
// counter after the control wave's phase start, 0 for a wave that came
// before it, at most 1023), bits 20-23 the last data wave's index, bits
// 24-27 the first one's.  The data waves' arrivals are spread by the order
// in which each SIMD issues its waves (oldest first).
template <int D>
__device__ __forceinline__ void record_arrivals(const uint32_t *arrive, uint64_t start, uint32_t *stats, uint32_t f1) {
    static_assert(D <= 16, "wave indices take four bits");
    uint32_t first = 0xFFFFFFFFu, last = 0u, who_first = 0u, who_last = 0u;
    for (int w = 0; w < D; ++w) {
        const int32_t dt = (int32_t)(arrive[w] - (uint32_t)start);
        const uint32_t t = dt < 0 ? 0u : (uint32_t)dt;
        if (t < first) {
            first = t;
            who_first = (uint32_t)w;
        }
        if (t >= last) {
            last = t;
            who_last = (uint32_t)w;
        }
    }
    first = first < 1023u ? first : 1023u;
    last = last < 1023u ? last : 1023u;
    stats[(uint64_t)kStatsWords * f1 + 15] = first | (last << 10) | (who_last << 20) | (who_first << 24);
}

// Control wave.  Phase k: issue the loads of the offsets around f2's first
// segment start (the tile the data waves load in this phase); find the carry
// into prev2 (a look-back only when prev2 heads a ticket group and its first
// element is not a segment start; the second tile of a group takes the
// carry-out of the first from this wave's registers) and publish PREFIX for
// prev2 if it had no start.  After barrier B: combine the wave pairs of f1
// (scanned in this phase) into its aggregate and first start and publish
// its descriptor at once -- PREFIX when it holds a start (or is tile 0),
// AGGREGATE otherwise -- most of a phase before it becomes cur (as in
// control_loop3).  f2's start bitmap is written before barrier B, while the
// data waves finalize, park and scan, into the buffer of this phase's
// parity; the data waves read it when they scan f2 in the next phase, and
// read the other buffer in this one.
template <int D, int Q, int LB_K, int G, bool STATS>
__device__ __forceinline__ void seg_control_loop(PipeTiles pt, SegShared<D, Q> &sh, uint32_t num_tiles, uint32_t n,
                                                 uint32_t *ctr, uint64_t *desc, LookbackCfg cfg,
                                                 const StartIndex &idx, const SegFallback &fb, uint32_t *stats,
                                                 uint32_t lane, uint32_t t_entry) {
    SegPair a_prev{0u, 0u}, a_prev2{0u, 0u};
    uint32_t fh_prev = kSegTile, fh_prev2 = kSegTile;
    uint32_t carry_out_last = 0;  // carry out of the tile handled one phase ago
    SegPair agg_next{0u, 0u};     // cur's aggregate and first start, published a phase ago
    uint32_t fh_next = kSegTile;
    for (int par = 0;; par ^= 1) {
        PhaseClock<STATS> clk;
        clk.begin();
        const SegPair agg = agg_next;
        const uint32_t fh = fh_next;
        // f2's starts: the first batch of offsets is in flight during the look-back
        const bool build = pt.f2 < num_tiles;
        const uint32_t tb = build ? pt.f2 * kSegTile : 0u;
        const uint32_t te = (uint32_t)min((uint64_t)n, (uint64_t)tb + kSegTile);
        const uint32_t s_lo = idx.bracket(tb, lane);
        uint32_t s_v[kStartProbes];
        idx.load_batch(s_lo, lane, s_v);
        uint32_t carry = 0;
        const bool have_prev2 = pt.prev2 < num_tiles && pt.prev2 != 0;
        LookbackStats st;
        uint64_t t0 = 0;
        if (STATS) t0 = __builtin_amdgcn_s_memrealtime();
        if (have_prev2) {
            if (pt.prev2 % G != 0u) {
                carry = carry_out_last;
            } else if (fh_prev2 != 0u) {
                // only a start-free tile's descriptor may turn PARTIAL (a
                // tile holding a start published PREFIX already)
                carry = lookback<SumU32, LB_K, STATS>(desc, pt.prev2, lane, st, ctr, cfg, a_prev2.v, !a_prev2.f, fb);
            }
        }
        if (STATS && lane == 0 && pt.prev2 < num_tiles) {
            const uint64_t t1 = __builtin_amdgcn_s_memrealtime();
            reinterpret_cast<uint4 *>(stats)[(kStatsWords / 4) * pt.prev2] =
                make_uint4(st.polls, st.windows, (uint32_t)(t1 - t0), st.stalls);
        }
        if (lane == 0) {
            sh.carry = carry;
            if (have_prev2 && !a_prev2.f)
                desc_publish(desc + pt.prev2, desc_word(ST_PREFIX | cfg.tf, carry + a_prev2.v));
        }
        if (build) idx.finish(s_v, s_lo, tb, te, lane, sh.starts[par], kSegWords);
        carry_out_last = a_prev2.f ? a_prev2.v : carry + a_prev2.v;
        a_prev2 = a_prev;
        fh_prev2 = fh_prev;
        a_prev = agg;
        fh_prev = fh;
        clk.reach_b();
        __syncthreads();  // B: the carry of prev2 is in LDS
        clk.leave_b();
        if (STATS && lane == 0 && pt.f1 < num_tiles) record_arrivals<D>(sh.arrive[par], clk.start, stats, pt.f1);
        agg_next = SegPair{0u, 0u};
        fh_next = kSegTile;
        if (pt.f1 < num_tiles) {
#pragma unroll
            for (int w = 0; w < D; ++w) {
                agg_next = seg_op(agg_next, SegPair{sh.wf[par ^ 1][w], sh.wv[par ^ 1][w]});
                fh_next = min(fh_next, sh.wfirst[par ^ 1][w]);
            }
            // a tile holding a start publishes PREFIX; the aggregate of a
            // start-free one may be withheld by a debug setting (look-backs
            // reaching it then take it from a fallback)
            const bool prefix = pt.f1 == 0 || agg_next.f;
            if (lane == 0 && (prefix || !(cfg.flags & kDbgWithholdAggregates)))
                desc_publish(desc + pt.f1, desc_word((prefix ? ST_PREFIX : ST_AGGREGATE) | cfg.tf, agg_next.v));
        }
        if (pt.drained(num_tiles)) {
            clk.finish(stats, pt.prev2, num_tiles, lane == 0);
            break;
        }
        clk.reach_a();
        __syncthreads();  // A: the next tile id is in LDS
        clk.record(stats, pt.f1, pt.prev2, num_tiles, t_entry, lane == 0);
        pt.advance(uniform(sh.next), num_tiles);
    }
}

// One phase of a data wave (the flat scan's phase with segment flags):
// finalize cur into LDS slot `slot` with carry 0, load the tile two ahead
// into the freed registers, scan f1; after barrier B add the carry to the
// elements of prev2 before its first segment start and store prev2.
template <int D, int Q, int G, bool INCL, bool VEC, bool STATS>
__device__ __forceinline__ bool seg_data_phase(SegSpan<Q> &cur, SegSpan<Q> &f1, int par, uint32_t &slot,
                                               PipeTiles &pt, uint32_t (&pre)[Q], uint32_t (&fl)[Q],
                                               SegShared<D, Q> &sh, const uint32_t *values, uint32_t *out, uint32_t n,
                                               uint32_t row_lo, uint32_t row_hi, uint32_t num_tiles,
                                               uint32_t *ctr, uint32_t lane, uint32_t d, uint64_t lane_off,
                                               uint32_t word_off) {
    constexpr uint32_t TILE = kSegTile;
    constexpr uint32_t WAVE_ELEMS = (uint32_t)Q * 256u;
    const bool need_ticket = needs_ticket<G>(pt.f2, num_tiles);
    uint32_t ticket = 0;
    if (need_ticket && d == 0 && lane == 0) ticket = take_ticket(ctr + kHdrTicket);
    const uint32_t old_slot = next_slot(slot);
    v4u *mine = &sh.park[slot][d * Q * 64u + lane];
    const v4u *theirs = &sh.park[old_slot][d * Q * 64u + lane];

    // cur: tile-relative segmented outputs, parked.  Work on absent tiles is
    // skipped (uniform branches, taken every phase but the pipeline's last
    // few): the loads stay straight-line, but nothing waits for the dummy
    // loads of an absent tile.
    if (pt.cur < num_tiles) {
        SegPair wave_prefix{0u, 0u};
        uint32_t first = TILE;
#pragma unroll
        for (int w = 0; w < D; ++w) {
            if ((uint32_t)w < d) wave_prefix = seg_op(wave_prefix, SegPair{sh.wf[par][w], sh.wv[par][w]});
            first = min(first, sh.wfirst[par][w]);
        }
        if (d == 0 && lane == 0) sh.park_first[slot] = first;
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            // the lane's prefix inside the wave, then the earlier waves' pair
            const uint32_t c = (fl[q] & 16u) ? pre[q] : wave_prefix.v + pre[q];
            uint32_t inc[4], o[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const bool seen = (fl[q] & ((2u << k) - 1u)) != 0u;  // a start among elements 0..k
                inc[k] = seen ? cur.x.v[q][k] : c + cur.x.v[q][k];
            }
            if (INCL) {
#pragma unroll
                for (int k = 0; k < 4; ++k) o[k] = inc[k];
            } else {
                o[0] = (fl[q] & 1u) ? 0u : c;
#pragma unroll
                for (int k = 1; k < 4; ++k) o[k] = (fl[q] & (1u << k)) ? 0u : inc[k - 1];
            }
            v4u w;
            w.x = o[0];
            w.y = o[1];
            w.z = o[2];
            w.w = o[3];
            mine[q * 64] = w;
        }
    }
    // the freed registers take the tile two ahead
    cur.template load<VEC>(values, pt.f2, lane_off, n, pt.f2 < num_tiles);
    // scan the next tile while the control wave looks back
    if (pt.f1 < num_tiles) {
        const uint64_t b1 = (uint64_t)pt.f1 * TILE;
        f1.x.pad(b1 + lane_off, n, b1 + TILE <= n);
        const uint32_t sh4 = 4u * (lane & 7u);
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            fl[q] = (sh.starts[par ^ 1][word_off + (uint32_t)q * 8u] >> sh4) & 0xFu;
            f1.x.v[q][1] = (fl[q] & 2u) ? f1.x.v[q][1] : f1.x.v[q][0] + f1.x.v[q][1];
            f1.x.v[q][2] = (fl[q] & 4u) ? f1.x.v[q][2] : f1.x.v[q][1] + f1.x.v[q][2];
            f1.x.v[q][3] = (fl[q] & 8u) ? f1.x.v[q][3] : f1.x.v[q][2] + f1.x.v[q][3];
        }
        SegPair run{0u, 0u};
        uint32_t wave_first = TILE;
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            uint32_t f = fl[q] ? 1u : 0u, v = f1.x.v[q][3];
            const uint64_t m = ballot(f != 0u);
            if (m != 0u && wave_first == TILE) {
                const uint32_t l0 = (uint32_t)__builtin_ctzll(m);
                const uint32_t bits = (uint32_t)__builtin_amdgcn_readlane((int)fl[q], (int)l0);
                wave_first = d * WAVE_ELEMS + (uint32_t)q * 256u + 4u * l0 + (uint32_t)__builtin_ctz(bits);
            }
            wave_seg_inclusive(f, v);
            // lane-exclusive pair within the row, combined at once with the
            // pair of the earlier rows of the span: bit 4 of fl marks a start
            // before the lane, pre holds the sum since it (or since the span
            // start)
            const uint32_t ef = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)f, 0x138, 0xF, 0xF, false);
            const uint32_t ev = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x138, 0xF, 0xF, false);
            const SegPair e = seg_op(run, SegPair{ef, ev});
            fl[q] |= e.f << 4;
            pre[q] = e.v;
            run = seg_op(run, SegPair{(uint32_t)__builtin_amdgcn_readlane((int)f, 63),
                                      (uint32_t)__builtin_amdgcn_readlane((int)v, 63)});
        }
        if (lane == 0) {
            sh.wf[par ^ 1][d] = run.f;
            sh.wv[par ^ 1][d] = run.v;
            sh.wfirst[par ^ 1][d] = wave_first;
        }
    }
    if (STATS && lane == 0) sh.arrive[par][d] = realtime32();
    __syncthreads();  // B
    if (pt.prev2 < num_tiles) {
        const uint64_t bp = (uint64_t)pt.prev2 * TILE;
        const uint32_t carry = sh.carry;
        const uint32_t first_start = sh.park_first[old_slot];
        const uint32_t span_local = d * WAVE_ELEMS + 4u * lane;
        const bool vec_store = VEC && bp >= row_lo && bp + TILE <= (uint64_t)row_hi;
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const v4u w = theirs[q * 64];
            const uint32_t li = span_local + (uint32_t)q * 256u;
            uint32_t o[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) o[k] = (li + k < first_start) ? o[k] + carry : o[k];
            if (vec_store) {
                v4u r;
                r.x = o[0];
                r.y = o[1];
                r.z = o[2];
                r.w = o[3];
                store16(out + bp + li, r);
            } else {
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const uint64_t i = bp + li + k;
                    if (i >= row_lo && i < row_hi) out[i] = o[k];
                }
            }
        }
    }
    if (pt.drained(num_tiles)) return true;
    if (d == 0 && lane == 0) sh.next = tile_after<G>(pt.f2, num_tiles, need_ticket, ticket);
    slot = old_slot;  // the slot just emptied takes the next tile
    __syncthreads();  // A
    pt.advance(uniform(sh.next), num_tiles);
    return false;
}

template <int D, int Q, int G, bool INCL, bool VEC, bool STATS>
__device__ __forceinline__ void seg_data_loop(PipeTiles pt, SegShared<D, Q> &sh, const uint32_t *values,
                                              uint32_t *out, uint32_t n, uint32_t row_lo,
                                              uint32_t row_hi, uint32_t num_tiles, uint32_t *ctr, uint32_t lane,
                                              uint32_t d) {
    const uint64_t lane_off = (uint64_t)d * Q * 256u + 4u * lane;
    const uint32_t word_off = d * Q * 8u + (lane >> 3);
    // two register buffers with alternating roles; the first two phases only
    // load, so every phase of the loop is the same instruction sequence
    SegSpan<Q> x, y;
    uint32_t pre[Q], fl[Q];
    uint32_t slot = 0;
    for (;;) {
        if (seg_data_phase<D, Q, G, INCL, VEC, STATS>(x, y, 0, slot, pt, pre, fl, sh, values,
                                               out, n, row_lo, row_hi, num_tiles, ctr, lane, d, lane_off,
                                               word_off))
            break;
        if (seg_data_phase<D, Q, G, INCL, VEC, STATS>(y, x, 1, slot, pt, pre, fl, sh, values,
                                               out, n, row_lo, row_hi, num_tiles, ctr, lane, d, lane_off,
                                               word_off))
            break;
    }
}

template <int D, int Q, int LB_K, int G, bool INCL, bool VEC, bool STATS>
__global__ __launch_bounds__((D + 1) * 64) void segscan_kernel(const uint32_t *values, uint32_t *out, uint32_t n,
                                                               const uint32_t *offsets, uint32_t num_segments,
                                                               uint32_t num_tiles, uint32_t *ctr, uint64_t *desc,
                                                               LookbackCfg cfg, uint32_t *stats) {
    __shared__ SegShared<D, Q> sh;
    __shared__ WsShared wsh;
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = uniform(threadIdx.x >> 6);
    const StartIndex idx = StartIndex::make(offsets, num_segments, sh.sample);
    uint32_t t0;
    const WsCall call = ws_start<G>(ctr, desc, num_tiles, num_tiles, wsh, t0);
    cfg.tf = tag_field(call.plan.tag);
    if (t0 < num_tiles) {
        const PipeTiles pt{num_tiles, num_tiles, num_tiles, num_tiles, num_tiles, t0};
        if (wave == 0) {
            // The control wave's own work (bracketing each tile's starts,
            // setting their bits, the look-back) is on the path to barrier
            // B in about half the phases, and its SIMD also runs three data
            // waves busy with the carried-flag scan: it issues first.  (The
            // flat scan's control wave mostly waits and gains nothing.)
            __builtin_amdgcn_s_setprio(3);
            // only the control wave reads the sample: the data waves' first
            // loads do not wait for it
            idx.load_sample(sh.sample, lane);
            ws_wait_clean(call, ctr);
            seg_control_loop<D, Q, LB_K, G, STATS>(pt, sh, num_tiles, n, ctr, desc, cfg, idx,
                                                   SegFallback{values, idx, sh.fb_starts, n}, stats, lane,
                                                   STATS ? wsh.entry : 0u);
        } else {
            // rows outside [offsets[0], offsets[N]) belong to no segment
            const uint32_t lo = offsets[0], hi = offsets[num_segments];
            seg_data_loop<D, Q, G, INCL, VEC, STATS>(pt, sh, values, out, n, uniform(lo < n ? lo : n),
                                              uniform(hi < n ? hi : n), num_tiles, ctr, lane, wave - 1);
        }
    }
    if (wave == 0) ws_done(wsh, num_tiles, ctr, lane);
}

// Workspace: header and descriptors as for the flat scan.
inline size_t seg_ws_bytes(uint64_t tiles) { return ws_bytes_for_tiles(tiles); }

}  // namespace dwps

using namespace dwps;

namespace dwps {

template <bool STATS>
ps_status launch_segmented(void *ws, size_t *ws_bytes, const uint32_t *values, uint64_t n, const uint32_t *offsets,
                           uint32_t num_segments, uint32_t *out, int inclusive, uint32_t *stats, void *stream) {
    // the offsets' count, num_segments + 1, must fit 32 bits
    if (n >= (1ull << 32) || num_segments == UINT32_MAX) return PS_ERR_SIZE;
    const uint64_t tiles = ceil_div(n, kSegTile);
    bool query = false;
    ps_status st = workspace_protocol(ws, ws_bytes, seg_ws_bytes(tiles), &query);
    if (st != PS_OK || query) return st;
    if (n == 0 || num_segments == 0) return PS_OK;
    if (!values || !offsets || !out) return PS_ERR_NULL;
    if (STATS && !stats) return PS_ERR_NULL;
    if (!aligned(values, 4) || !aligned(offsets, 4) || !aligned(out, 4) || !aligned(ws, 16))
        return PS_ERR_ALIGNMENT;
    if (ranges_overlap(out, n * 4, values, n * 4) ||
        ranges_overlap(out, n * 4, offsets, ((size_t)num_segments + 1) * 4))
        return PS_ERR_ALIAS;
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint32_t *ctr = ws_counter(ws);
    uint64_t *desc = ws_desc(ws);
    const uint32_t n32 = (uint32_t)n, nt = (uint32_t)tiles;
    const bool vec = aligned(values, 16) && aligned(out, 16);
    if (STATS && !vec) return PS_ERR_ALIGNMENT;  // instrumented for the vector path only
    auto launch = [&](auto kernel) -> ps_status {
        const uint32_t grid = persistent_grid(reinterpret_cast<const void *>(kernel), kSegThreads, nt);
        if (!grid) return PS_ERR_HIP;
        timing_begin(s);
        const LookbackCfg cfg = lookback_cfg(false);
        hipLaunchKernelGGL(kernel, dim3(grid), dim3(kSegThreads), 0, s, values, out, n32, offsets,
                           num_segments, nt, ctr, desc, cfg, stats);
        return PS_OK;
    };
    ps_status r;
    if constexpr (STATS) {
        r = inclusive ? launch(segscan_kernel<kSegD, kSegQ, DWPS_LOOKBACK_K, kSegG, true, true, true>)
                      : launch(segscan_kernel<kSegD, kSegQ, DWPS_LOOKBACK_K, kSegG, false, true, true>);
    } else if (inclusive) {
        r = vec ? launch(segscan_kernel<kSegD, kSegQ, DWPS_LOOKBACK_K, kSegG, true, true, false>)
                : launch(segscan_kernel<kSegD, kSegQ, DWPS_LOOKBACK_K, kSegG, true, false, false>);
    } else {
        r = vec ? launch(segscan_kernel<kSegD, kSegQ, DWPS_LOOKBACK_K, kSegG, false, true, false>)
                : launch(segscan_kernel<kSegD, kSegQ, DWPS_LOOKBACK_K, kSegG, false, false, false>);
    }
    if (r != PS_OK) return r;
    timing_end(s);
    return launch_status();
}

}  // namespace dwps

extern "C" ps_status ps_segmented_scan_u32(void *ws, size_t *ws_bytes, const uint32_t *values, uint64_t n,
                                           const uint32_t *offsets, uint32_t num_segments, uint32_t *out,
                                           int inclusive, void *stream) {
    return launch_segmented<false>(ws, ws_bytes, values, n, offsets, num_segments, out, inclusive, nullptr, stream);
}

extern "C" ps_status ps_segmented_lookback_stats_u32(void *ws, size_t *ws_bytes, const uint32_t *values, uint64_t n,
                                                     const uint32_t *offsets, uint32_t num_segments, uint32_t *out,
                                                     int inclusive, uint32_t *stats, void *stream) {
    return launch_segmented<true>(ws, ws_bytes, values, n, offsets, num_segments, out, inclusive, stats, stream);
}

extern "C" uint32_t ps_segmented_tile_elements(void) { return kSegTile; }
