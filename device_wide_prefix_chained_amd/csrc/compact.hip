// compact.hip -- stable stream compaction fused with its scan, single pass.
//
// "Prefix scans and compaction", sections "Scan as an index generator" and
// "Worked example: Stable stream compaction", and "Parallel Prefix Sum (Scan),
// in depth", section "What scan builds": the destination of a kept record is
// the exclusive scan of the keep flags at its position, so kept records land
// densely and in input order; the count is the last offset plus the last
// flag.  The offsets are never written to memory (the page's advice to avoid
// materialising the flags and prefixes).
//
// The flat scan's persistent, wave-specialised pipeline with a count as the
// scanned value: a tile is D waves x Q loads of 16 bytes per lane (E = 16 /
// record_bytes records per load), 48 KiB of records.  Per phase a data wave
//   * issues the loads of the tile two ahead into the free registers;
//   * ranks the next tile (the rank of a record is a ballot plus a
//     lane-masked popcount, v_mbcnt, over its row of 64 lanes; the wave's
//     count goes to the control wave);
//   * after barrier B, copies its run of kept records of the tile parked
//     three phases earlier, whose output base the look-back has returned,
//     from its part of the LDS slot to out[base + offset ...] -- contiguous,
//     so every store instruction writes 64 consecutive records -- and parks
//     the kept records of the current tile, compacted, in the same place.
// The control wave is the flat scan's (tile counts instead of sums).
#include <hip/hip_runtime.h>

#include "dwps_device.hpp"
#include "host_common.hpp"
#include "pipeline.hpp"
#include "tile_io.hpp"

namespace dwps {

typedef unsigned int v2u __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t lane_rank(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Record k of a 16-byte load, for each record width.
template <class Rec>
__device__ __forceinline__ Rec record_at(const v4u &raw, int k);
template <>
__device__ __forceinline__ uint32_t record_at<uint32_t>(const v4u &raw, int k) {
    return raw[k];
}
template <>
__device__ __forceinline__ v2u record_at<v2u>(const v4u &raw, int k) {
    v2u r;
    r.x = raw[2 * k];
    r.y = raw[2 * k + 1];
    return r;
}
template <>
__device__ __forceinline__ v4u record_at<v4u>(const v4u &raw, int k) {
    (void)k;
    return raw;
}

// Register state of one wave's span of a tile: Q 16-byte loads per lane and
// the keep flags of their records (byte k of fw[q] is the flag of record k).
// Load q of lane l covers records q*64*E + l*E ... + E-1 of the span, so one
// load instruction of the wave reads 1 KiB of consecutive records and the
// flags it needs are 64*E consecutive bytes.
template <class Rec, int Q>
struct RecSpan {
    static constexpr int E = 16 / (int)sizeof(Rec);
    v4u raw[Q];
    uint32_t fw[Q];

    // Straight-line loads as in the flat scan: past-the-end groups are
    // clamped to the last group that starts below n (it never leaves the page
    // of record n-1, nor does the flag word of that group), !valid reads the
    // first group again; pad() drops the flags at or past n.
    // VEC: records 16-byte aligned and flags E-byte aligned -- one 16-byte
    // record load and one E-byte flag load per group; otherwise one load per
    // record and flag byte.
    template <bool VEC>
    __device__ __forceinline__ void load(const Rec *records, const uint8_t *flags, uint64_t span, uint32_t n,
                                         bool full, bool valid) {
        if (VEC) {
            const uint64_t last_group = ((uint64_t)n - 1u) / E * E;
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                uint64_t g = span + (uint64_t)q * 64u * E;
                if (!full) g = g < last_group ? g : last_group;
                if (!valid) g = 0;
                raw[q] = load16(records + g);
                if (E == 4)
                    fw[q] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(flags + g));
                else if (E == 2)
                    fw[q] = __builtin_nontemporal_load(reinterpret_cast<const uint16_t *>(flags + g));
                else
                    fw[q] = __builtin_nontemporal_load(flags + g);
            }
        } else {
            const uint64_t last = (uint64_t)n - 1u;
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                uint32_t w[4];
                uint32_t f = 0;
#pragma unroll
                for (int k = 0; k < E; ++k) {
                    uint64_t i = span + (uint64_t)q * 64u * E + k;
                    i = i < last ? i : last;
                    if (!valid) i = 0;
                    const uint32_t *r = reinterpret_cast<const uint32_t *>(records + i);
#pragma unroll
                    for (int j = 0; j < 4 / E; ++j) w[k * (4 / E) + j] = r[j];
                    f |= (uint32_t)flags[i] << (8 * k);
                }
                raw[q].x = w[0];
                raw[q].y = w[1];
                raw[q].z = w[2];
                raw[q].w = w[3];
                fw[q] = f;
            }
        }
    }

    __device__ __forceinline__ void pad(uint64_t span, uint32_t n, bool full) {
        if (full) return;
#pragma unroll
        for (int q = 0; q < Q; ++q)
#pragma unroll
            for (int k = 0; k < E; ++k) {
                const uint64_t i = span + (uint64_t)q * 64u * E + k;
                fw[q] = (i < n) ? fw[q] : (fw[q] & ~(0xFFu << (8 * k)));
            }
    }
};

template <int D, int Q>
struct CompactShared {
    v4u park[kParkSlots][D * Q * 64];  // kept records of each wave's span, compacted, in the wave's part
    uint2 park_wave[kParkSlots][D];    // per wave, (offset in the tile's output, count) of its parked run
    uint32_t wt[2][D];                 // wave counts, double-buffered by phase parity
    uint32_t next;
    uint32_t prefix;                   // output base of the tile stored in the phase
    uint32_t close_prefix[3];          // the closing phase's output bases (closing_phase in pipeline.hpp)
};

// Copy this wave's parked run of tile `tile` (slot `slot`) to its place
// after the output base `prefix`; the last tile's last wave also writes the
// count.
template <class Rec, int D, int Q>
__device__ __forceinline__ void store_run(CompactShared<D, Q> &sh, uint32_t slot, uint32_t tile, uint32_t prefix,
                                          Rec *out, uint64_t *num_selected, uint32_t num_tiles, uint32_t lane,
                                          uint32_t d) {
    const Rec *run = reinterpret_cast<const Rec *>(&sh.park[slot][(uint32_t)d * Q * 64u]);
    const uint2 meta = sh.park_wave[slot][d];
    const uint64_t base = (uint64_t)prefix + meta.x;
    for (uint32_t j = lane; j < meta.y; j += 64u) __builtin_nontemporal_store(run[j], out + base + j);
    if (tile == num_tiles - 1u && d == (uint32_t)D - 1u && lane == 0) *num_selected = base + meta.y;
}

// One phase of a data wave (the flat scan's phase, data_phase3 in scan.hip,
// with a count as the scanned value).  Each wave parks the kept
// records of its own span, compacted, in its own part of the slot, so after
// barrier B a wave can copy prev3's run out of its part and write cur's run
// into it without waiting on the other waves.  The wave's run of a tile goes
// to out[base + (kept records of the earlier waves of the tile) ...]; both
// numbers travel with the parked run (park_wave).  kb/pos of `hold` come
// from its ranking in the phase before; the ranking of `sc` fills new ones.
template <class Rec, int D, int Q, int G, bool VEC>
__device__ __forceinline__ bool compact_phase3(RecSpan<Rec, Q> &hold, RecSpan<Rec, Q> &sc, RecSpan<Rec, Q> &ld,
                                               int par, uint32_t &slot, PipeTiles &pt, uint32_t (&kb)[Q],
                                               uint32_t (&pos)[Q], CompactShared<D, Q> &sh, const Rec *records,
                                               const uint8_t *flags, Rec *out, uint64_t *num_selected, uint32_t n,
                                               uint32_t num_tiles, uint32_t *ctr, uint32_t lane, uint32_t d,
                                               uint64_t lane_off) {
    constexpr int E = RecSpan<Rec, Q>::E;
    constexpr uint32_t TILE = (uint32_t)D * Q * 64u * E;
    const bool need_ticket = needs_ticket<G>(pt.f2, num_tiles);
    uint32_t ticket = 0;
    if (need_ticket && d == 0 && lane == 0) ticket = take_ticket(ctr + kHdrTicket);
    // cur: the wave's offset in the tile and its count
    uint32_t wave_prefix = 0u;
#pragma unroll
    for (int w = 0; w < D; ++w) wave_prefix += ((uint32_t)w < d) ? sh.wt[par][w] : 0u;
    const uint32_t wave_cnt = sh.wt[par][d];
    // the free registers take the tile two ahead
    const uint64_t b2 = (uint64_t)pt.f2 * TILE;
    ld.template load<VEC>(records, flags, b2 + lane_off, n, b2 + TILE <= n, pt.f2 < num_tiles);
    // rank the next tile while the control wave looks back (work on absent
    // tiles is skipped by uniform branches: nothing waits for their dummy
    // loads)
    uint32_t kb_n[Q], pos_n[Q];
    {
        // (also when f1 is absent: its flags are all padding, and a branch
        // here measured slower than ranking the padding)
        const uint64_t b1 = (uint64_t)pt.f1 * TILE;
        sc.pad(b1 + lane_off, n, b1 + TILE <= n);
        uint32_t run = 0u;
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            uint32_t bits = 0u;
#pragma unroll
            for (int k = 0; k < E; ++k) bits |= ((sc.fw[q] >> (8 * k)) & 0xFFu) ? (1u << k) : 0u;
            kb_n[q] = bits;
            uint32_t before = 0u, total = 0u;
#pragma unroll
            for (int k = 0; k < E; ++k) {
                const uint64_t m = ballot(((bits >> k) & 1u) != 0u);
                before += lane_rank(m);
                total += (uint32_t)__builtin_popcountll(m);
            }
            pos_n[q] = run + before;
            run += total;
        }
        if (lane == 0) sh.wt[par ^ 1][d] = run;
    }
    __syncthreads();  // B
    Rec *mine = reinterpret_cast<Rec *>(&sh.park[slot][(uint32_t)d * Q * 64u]);
    if (pt.prev3 < num_tiles)
        store_run<Rec, D, Q>(sh, slot, pt.prev3, sh.prefix, out, num_selected, num_tiles, lane, d);
    // park cur's kept records where prev3's were
    if (pt.cur < num_tiles) {
#pragma unroll
        for (int q = 0; q < Q; ++q) {
#pragma unroll
            for (int k = 0; k < E; ++k)
                if ((kb[q] >> k) & 1u) mine[pos[q] + (uint32_t)__builtin_popcount(kb[q] & ((1u << k) - 1u))] =
                    record_at<Rec>(hold.raw[q], k);
        }
        if (lane == 0) sh.park_wave[slot][d] = make_uint2(wave_prefix, wave_cnt);
    }
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        kb[q] = kb_n[q];
        pos[q] = pos_n[q];
    }
    if (pt.template drained<3>(num_tiles)) return true;
    if (d == 0 && lane == 0) sh.next = tile_after<G>(pt.f2, num_tiles, need_ticket, ticket);
    slot = next_slot(slot);
    __syncthreads();  // A
    pt.advance(uniform(sh.next), num_tiles);
    if (after_closing(pt, num_tiles)) {
        // the closing phase resolved the three parked tiles: store them all
        // now (the control wave has left the loop; no barrier follows)
#pragma unroll 1
        for (int i = 0; i < 3; ++i) {
            const uint32_t t = i == 0 ? pt.prev3 : i == 1 ? pt.prev2 : pt.prev;
            if (t < num_tiles)
                store_run<Rec, D, Q>(sh, closing_slot(slot, i), t, sh.close_prefix[i], out, num_selected, num_tiles,
                                     lane, d);
        }
        return true;
    }
    return false;
}

template <class Rec, int D, int Q, int G, bool VEC>
__device__ __forceinline__ void compact_data_loop3(PipeTiles pt, CompactShared<D, Q> &sh, const Rec *records,
                                                   const uint8_t *flags, Rec *out, uint64_t *num_selected,
                                                   uint32_t n, uint32_t num_tiles, uint32_t *ctr, uint32_t lane,
                                                   uint32_t d) {
    constexpr int E = RecSpan<Rec, Q>::E;
    const uint64_t lane_off = (uint64_t)d * Q * 64u * E + (uint64_t)lane * E;
    RecSpan<Rec, Q> x, y, z;
    // no keep bits before the first ranking: the first phases park nothing
    uint32_t kb[Q], pos[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) kb[q] = pos[q] = 0u;
    uint32_t slot = 0;
    int par = 0;
    for (;;) {
        if (compact_phase3<Rec, D, Q, G, VEC>(x, y, z, par, slot, pt, kb, pos, sh, records, flags, out,
                                              num_selected, n, num_tiles, ctr, lane, d, lane_off))
            break;
        par ^= 1;
        if (compact_phase3<Rec, D, Q, G, VEC>(y, z, x, par, slot, pt, kb, pos, sh, records, flags, out,
                                              num_selected, n, num_tiles, ctr, lane, d, lane_off))
            break;
        par ^= 1;
        if (compact_phase3<Rec, D, Q, G, VEC>(z, x, y, par, slot, pt, kb, pos, sh, records, flags, out,
                                              num_selected, n, num_tiles, ctr, lane, d, lane_off))
            break;
        par ^= 1;
    }
}

// A look-back's fallback: count the kept flags of tile p from scratch (rows
// of 64 flags, a ballot each) and return the descriptor word its owner
// publishes first.  Runs on the control wave, rarely.
template <uint32_t TILE>
struct CompactFallback {
    const uint8_t *flags;
    uint32_t n;
    __device__ DescVal<uint32_t> operator()(uint32_t p, uint32_t lane) const {
        constexpr uint32_t ROWS = TILE / 64u, BATCH = 8u;
        static_assert(ROWS % BATCH == 0, "whole batches of rows");
        const uint64_t base = (uint64_t)p * TILE + lane;
        uint32_t count = 0;
        for (uint32_t r = 0; r < ROWS; r += BATCH) {
            uint32_t f[BATCH];
#pragma unroll
            for (uint32_t k = 0; k < BATCH; ++k) {
                const uint64_t i = base + (uint64_t)(r + k) * 64u;
                f[k] = i < n ? flags[i] : 0u;
            }
#pragma unroll
            for (uint32_t k = 0; k < BATCH; ++k) count += (uint32_t)__builtin_popcountll(ballot(f[k] != 0u));
        }
        return DescVal<uint32_t>{p == 0 ? ST_PREFIX : ST_AGGREGATE, count};
    }
};

template <class Rec, int D, int Q, int LB_K, int G, bool VEC, bool STATS>
__global__ __launch_bounds__((D + 1) * 64) void compact_kernel(const Rec *records, const uint8_t *flags,
                                                               uint32_t n, Rec *out, uint64_t *num_selected,
                                                               uint32_t num_tiles, uint32_t *ctr, uint64_t *desc,
                                                               LookbackCfg cfg, uint32_t *stats) {
    __shared__ CompactShared<D, Q> sh;
    __shared__ WsShared wsh;
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = uniform(threadIdx.x >> 6);
    uint32_t t0;
    const WsCall call = ws_start<G>(ctr, desc, num_tiles, num_tiles, wsh, t0);
    cfg.tf = tag_field(call.plan.tag);
    if (t0 < num_tiles) {
        const PipeTiles pt{num_tiles, num_tiles, num_tiles, num_tiles, num_tiles, t0};
        using Fb = CompactFallback<(uint32_t)D * Q * 64u * (16u / sizeof(Rec))>;
        if (wave == 0) {
            ws_wait_clean(call, ctr);
            control_loop3<SumU32, D, LB_K, G, STATS, false, true, true>(pt, sh, num_tiles, ctr, desc, (uint32_t *)nullptr,
                                                                  stats, 0, cfg, Fb{flags, n}, lane,
                                                                  STATS ? wsh.entry : 0u);
        } else {
            compact_data_loop3<Rec, D, Q, G, VEC>(pt, sh, records, flags, out, num_selected, n, num_tiles, ctr, lane,
                                                  wave - 1);
        }
    }
    if (wave == 0) ws_done(wsh, num_tiles, ctr, lane);
}

__global__ void write_count_zero(uint64_t *p) { *p = 0ull; }

// Compaction tile shape: D data waves x Q 16-byte loads per lane.
#ifndef DWPS_COMPACT_D
#define DWPS_COMPACT_D 8
#endif
#ifndef DWPS_COMPACT_Q
#define DWPS_COMPACT_Q 6
#endif
constexpr int kCompactD = DWPS_COMPACT_D;
constexpr int kCompactQ = DWPS_COMPACT_Q;
constexpr int kCompactG = 2;
constexpr int kCompactThreads = (kCompactD + 1) * 64;

template <class Rec, bool STATS>
ps_status launch_compact(void *ws, size_t *ws_bytes, const void *records, const uint8_t *flags, uint64_t n,
                         void *out, uint64_t *num_selected, uint32_t *stats, hipStream_t s) {
    constexpr uint32_t TILE = (uint32_t)kCompactD * kCompactQ * 64u * (16u / sizeof(Rec));
    const uint64_t tiles = ceil_div(n, TILE);
    bool query = false;
    ps_status st = workspace_protocol(ws, ws_bytes, ws_bytes_for_tiles(tiles), &query);
    if (st != PS_OK || query) return st;
    if (!num_selected) return PS_ERR_NULL;
    if (!aligned(num_selected, 8)) return PS_ERR_ALIGNMENT;
    if (n == 0) {
        hipLaunchKernelGGL(write_count_zero, dim3(1), dim3(1), 0, s, num_selected);
        return launch_status();
    }
    if (!records || !flags || !out) return PS_ERR_NULL;
    if (STATS && !stats) return PS_ERR_NULL;
    if (!aligned(records, sizeof(Rec)) || !aligned(out, sizeof(Rec)) || !aligned(ws, 16)) return PS_ERR_ALIGNMENT;
    const size_t bytes = n * sizeof(Rec);
    if (ranges_overlap(out, bytes, records, bytes) || ranges_overlap(out, bytes, flags, n) ||
        ranges_overlap(num_selected, 8, out, bytes))
        return PS_ERR_ALIAS;
    const bool vec = aligned(records, 16) && aligned(flags, 16 / sizeof(Rec));
    if (STATS && !vec) return PS_ERR_ALIGNMENT;  // instrumented for the vector path only
    const Rec *rin = static_cast<const Rec *>(records);
    Rec *rout = static_cast<Rec *>(out);
    const uint32_t n32 = (uint32_t)n, nt = (uint32_t)tiles;
    uint32_t *ctr = ws_counter(ws);
    uint64_t *desc = ws_desc(ws);
    auto launch = [&](auto kernel) -> ps_status {
        const uint32_t grid = persistent_grid(reinterpret_cast<const void *>(kernel), kCompactThreads, nt);
        if (!grid) return PS_ERR_HIP;
        timing_begin(s);
        const LookbackCfg cfg = lookback_cfg(false);
        hipLaunchKernelGGL(kernel, dim3(grid), dim3(kCompactThreads), 0, s, rin, flags, n32, rout, num_selected,
                           nt, ctr, desc, cfg, stats);
        return PS_OK;
    };
    ps_status r;
    if constexpr (STATS)
        r = launch(compact_kernel<Rec, kCompactD, kCompactQ, DWPS_LOOKBACK_K, kCompactG, true, true>);
    else
        r = vec ? launch(compact_kernel<Rec, kCompactD, kCompactQ, DWPS_LOOKBACK_K, kCompactG, true, false>)
                : launch(compact_kernel<Rec, kCompactD, kCompactQ, DWPS_LOOKBACK_K, kCompactG, false, false>);
    if (r != PS_OK) return r;
    timing_end(s);
    return launch_status();
}

}  // namespace dwps

using namespace dwps;

extern "C" ps_status ps_compact(void *ws, size_t *ws_bytes, const void *records, uint32_t record_bytes,
                                const uint8_t *flags, uint64_t n, void *out, uint64_t *num_selected,
                                void *stream) {
    if (n >= (1ull << 32)) return PS_ERR_SIZE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    switch (record_bytes) {
    case 4: return launch_compact<uint32_t, false>(ws, ws_bytes, records, flags, n, out, num_selected, nullptr, s);
    case 8: return launch_compact<v2u, false>(ws, ws_bytes, records, flags, n, out, num_selected, nullptr, s);
    case 16: return launch_compact<v4u, false>(ws, ws_bytes, records, flags, n, out, num_selected, nullptr, s);
    default: return PS_ERR_UNSUPPORTED;
    }
}

extern "C" ps_status ps_compact_lookback_stats(void *ws, size_t *ws_bytes, const void *records,
                                               uint32_t record_bytes, const uint8_t *flags, uint64_t n, void *out,
                                               uint64_t *num_selected, uint32_t *stats, void *stream) {
    if (n >= (1ull << 32)) return PS_ERR_SIZE;
    if (record_bytes != 16) return PS_ERR_UNSUPPORTED;
    return launch_compact<v4u, true>(ws, ws_bytes, records, flags, n, out, num_selected, stats,
                                     static_cast<hipStream_t>(stream));
}

extern "C" uint32_t ps_compact_tile_records(uint32_t record_bytes) {
    if (record_bytes != 4 && record_bytes != 8 && record_bytes != 16) return 0;
    return (uint32_t)kCompactD * kCompactQ * 64u * (16u / record_bytes);
}
