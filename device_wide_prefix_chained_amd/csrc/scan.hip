// scan.hip -- flat device-wide scan: single pass, chained scan with decoupled
// look-back ("Single-Pass Prefix Scan with Decoupled Look-Back"; "Parallel
// Prefix Sum (Scan), in depth", section "Scanning a whole array: three grid
// strategies").
//
// Persistent, wave-specialised workgroups.  The grid holds as many
// workgroups as the GPU keeps resident; each one loops over tiles of
// D * Q * 256 elements taken from the atomic tile counter (two consecutive
// tiles per ticket).  A workgroup has one control wave and D data waves and
// moves each tile through these phases:
//   phase k-1  its loads are issued (into a register buffer);
//   phase k    it is scanned; after barrier B its aggregate is published;
//   phase k+1  it is made tile-relative and, after B, parked in LDS;
//   phase k+3  its look-back (first tile of a ticket) polls at the start of
//              the phase -- three phases after the aggregate went out, so
//              the poll normally finds every word it needs -- and finishes
//              after barrier B, while the data waves store;
//   phase k+4  the data waves add its prefix and store it.
// Control wave (per phase): hand the data waves the prefix resolved in the
// phase before, issue the first poll of the next look-back, pass barrier B,
// finish the look-back and publish its prefix, publish the aggregate of the
// tile just scanned.  Its vector-memory queue holds only descriptor traffic,
// so a poll never waits behind a tile load.  Data waves (per phase):
// finalize cur in registers, issue the loads of f2, scan f1; after barrier
// B store prev3 from LDS and park cur in its slot.  Up to two tiles of loads
// per workgroup are in flight while look-backs are resolved two phases
// behind (a persistent grid-stride loop, as in "Where the algorithm meets
// the hardware", with the look-back joining the tiles inside one launch).
// In the two-word kernels, a workgroup that runs out of tiles ends with a
// closing phase that resolves the prefixes of the three tiles still parked,
// and they are stored together (closing_phase in pipeline.hpp) rather than
// one per phase.
// Tickets come from an atomic counter, so every tile a look-back can wait on
// was handed out earlier to a running workgroup, which finishes it without
// waiting on anything later ("Scanning a whole array: three grid
// strategies"); forward progress follows by induction on the smallest
// unfinished tile.
#include <hip/hip_runtime.h>

#include <mutex>

#include "dwps_device.hpp"
#include "host_common.hpp"
#include "pipeline.hpp"
#include "tile_io.hpp"
#include "twolevel.hpp"

namespace dwps {

template <class Op, int D, int Q>
struct ScanShared {
    using T = typename Op::T;
    static constexpr int PW = (int)sizeof(T) / 4;  // 16-byte vectors per group of four outputs
    v4u park[kParkSlots][D * Q * 64 * PW];       // tile-relative outputs
    uint32_t next;
    T wt[2][D];  // wave totals, double-buffered by phase parity
    T prefix;
    T close_prefix[3];  // the closing phase's prefixes (closing_phase in pipeline.hpp)
};

// Store tile `tile`, parked in slot `slot`, with its exclusive prefix `pre`:
// each wave its own part of the slot (the closing phase's stores; the
// steady-state store in data_phase3 is the same code inline).
template <class Op, int D, int Q, bool VEC>
__device__ __forceinline__ void store_parked(ScanShared<Op, D, Q> &sh, uint32_t slot, uint32_t tile,
                                             typename Op::T pre, typename IoOf<Op>::Dst out, uint32_t n,
                                             uint32_t lane, uint32_t d, uint64_t lane_off) {
    using T = typename Op::T;
    constexpr uint32_t TILE = (uint32_t)D * (uint32_t)Q * 256u;
    constexpr int PW = ScanShared<Op, D, Q>::PW;
    const v4u *mine = &sh.park[slot][(uint32_t)d * Q * PW * 64u + lane];
    const uint64_t bp = (uint64_t)tile * TILE;
    const bool full = bp + TILE <= n;
    if constexpr (PW == 2 && VEC && std::is_pointer<typename IoOf<Op>::Dst>::value) {
        if (full) {
            // 8-byte outputs read back regrouped (see data_phase)
            const v4u *wp = &sh.park[slot][(uint32_t)d * Q * PW * 64u];
            T *row = out + bp + (uint64_t)d * Q * 256u + 2u * lane;
#pragma unroll
            for (int q = 0; q < Q; ++q)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const v4u w = wp[(q * 2 + (int)(lane & 1u)) * 64 + h * 32 + (int)(lane >> 1)];
                    const uint64_t a = to_bits64(Op::op(pre, from_bits64<T>(((uint64_t)w.y << 32) | w.x)));
                    const uint64_t b = to_bits64(Op::op(pre, from_bits64<T>(((uint64_t)w.w << 32) | w.z)));
                    v4u r;
                    r.x = (uint32_t)a;
                    r.y = (uint32_t)(a >> 32);
                    r.z = (uint32_t)b;
                    r.w = (uint32_t)(b >> 32);
                    store16(row + q * 256 + h * 128, r);
                }
            return;
        }
    }
    WaveSpan<Op, Q> old;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        v4u w[PW];
#pragma unroll
        for (int h = 0; h < PW; ++h) w[h] = mine[(q * PW + h) * 64];
        unpack16<T>(w, old.v[q]);
    }
    store_final<Op, Q, VEC>(old, pre, out, bp + lane_off, n, full);
}

// One phase of a data wave.  A tile is stored three phases after its park:
// cur is finalized (made tile-relative) in registers at the start of the
// phase and held until after barrier B; then the wave stores prev3 from slot
// `slot` and parks cur in the same slot (each wave reads and writes only its
// own part of a slot, in program order), so three slots and three register
// buffers cover the pipeline.  Buffers: `hold` = cur, `sc` = f1 (scanned
// now), `ld` = free, takes the loads of f2.  Straight-line code whether or
// not the tiles exist (absent tiles are dummy loads of the first group and
// harmless arithmetic), so that the compiler sees one fixed sequence of
// loads and keeps two tiles in flight.  Data wave 0 also takes the tickets:
// the atomic goes out at the start of the phase, ahead of the wave's tile
// loads, and its value is needed only after barrier B.
template <class Op, int D, int Q, int G, bool INCL, bool VEC, bool STATS, bool CLOSE>
__device__ __forceinline__ bool data_phase3(WaveSpan<Op, Q> &hold, WaveSpan<Op, Q> &sc, WaveSpan<Op, Q> &ld, int par,
                                            uint32_t &slot, PipeTiles &pt, typename Op::T (&lane_excl)[Q],
                                            typename Op::T (&row_prefix)[Q], ScanShared<Op, D, Q> &sh,
                                            typename IoOf<Op>::Src in, typename IoOf<Op>::Dst out, uint32_t n,
                                            uint32_t num_tiles, uint32_t *ctr, uint32_t lane, uint32_t d,
                                            uint64_t lane_off, uint32_t *stats) {
    using T = typename Op::T;
    constexpr uint32_t TILE = (uint32_t)D * (uint32_t)Q * 256u;
    constexpr int PW = ScanShared<Op, D, Q>::PW;
    DataClock<STATS> clk;
    clk.begin();
    const bool need_ticket = needs_ticket<G>(pt.f2, num_tiles);
    uint32_t ticket = 0;
    if (need_ticket && d == 0 && lane == 0) ticket = take_ticket(ctr + kHdrTicket);
    // cur tile-relative, in registers (its wave totals are in wt[par]).
    // Work on absent tiles is skipped (uniform branches, taken every phase
    // but the pipeline's last few): the loads stay straight-line, but
    // nothing waits for the dummy loads of an absent tile.
    if (pt.cur < num_tiles) {
        T wave_prefix = Op::id();
#pragma unroll
        for (int w = 0; w < D; ++w)
            if ((uint32_t)w < d) wave_prefix = Op::op(wave_prefix, sh.wt[par][w]);
        finalize_span<Op, Q, INCL>(hold, lane_excl, row_prefix, wave_prefix);
    }
    // the free buffer takes the tile two ahead
    const uint64_t b2 = (uint64_t)pt.f2 * TILE;
    ld.template load<VEC>(in, b2 + lane_off, n, b2 + TILE <= n, pt.f2 < num_tiles);
    // scan the next tile while the control wave looks back
    if (pt.f1 < num_tiles) {
        const uint64_t b1 = (uint64_t)pt.f1 * TILE;
        sc.pad(b1 + lane_off, n, b1 + TILE <= n);
        const T wt = scan_span<Op, Q>(sc, lane_excl, row_prefix);
        if (lane == 0) sh.wt[par ^ 1][d] = wt;
    }
    clk.scan_done();
    __syncthreads();  // B
    clk.leave_b();
    v4u *mine = &sh.park[slot][(uint32_t)d * Q * PW * 64u + lane];
    if (pt.prev3 < num_tiles) {
        const uint64_t bp = (uint64_t)pt.prev3 * TILE;
        const bool full = bp + TILE <= n;
        bool stored = false;
        if constexpr (PW == 2 && VEC && std::is_pointer<typename IoOf<Op>::Dst>::value) {
            if (full) {
                // 8-byte outputs read back regrouped (see data_phase)
                const v4u *wp = &sh.park[slot][(uint32_t)d * Q * PW * 64u];
                T *row = out + bp + (uint64_t)d * Q * 256u + 2u * lane;
                const T pre = sh.prefix;
#pragma unroll
                for (int q = 0; q < Q; ++q)
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const v4u w = wp[(q * 2 + (int)(lane & 1u)) * 64 + h * 32 + (int)(lane >> 1)];
                        const uint64_t a = to_bits64(Op::op(pre, from_bits64<T>(((uint64_t)w.y << 32) | w.x)));
                        const uint64_t b = to_bits64(Op::op(pre, from_bits64<T>(((uint64_t)w.w << 32) | w.z)));
                        v4u r;
                        r.x = (uint32_t)a;
                        r.y = (uint32_t)(a >> 32);
                        r.z = (uint32_t)b;
                        r.w = (uint32_t)(b >> 32);
                        store16(row + q * 256 + h * 128, r);
                    }
                stored = true;
            }
        }
        if (!stored) {
            WaveSpan<Op, Q> old;
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                v4u w[PW];
#pragma unroll
                for (int h = 0; h < PW; ++h) w[h] = mine[(q * PW + h) * 64];
                unpack16<T>(w, old.v[q]);
            }
            store_final<Op, Q, VEC>(old, sh.prefix, out, bp + lane_off, n, full);
        }
    }
    clk.store_done();
    // park cur where prev3 was
    if (pt.cur < num_tiles) {
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            v4u w[PW];
            pack16<T>(hold.v[q], w);
#pragma unroll
            for (int h = 0; h < PW; ++h) mine[(q * PW + h) * 64] = w[h];
        }
    }
    if (pt.template drained<3>(num_tiles)) return true;
    if (d == 0 && lane == 0) sh.next = tile_after<G>(pt.f2, num_tiles, need_ticket, ticket);
    slot = next_slot(slot);
    clk.reach_a(stats, pt.f1, num_tiles, d == 0 && lane == 0);
    __syncthreads();  // A
    pt.advance(uniform(sh.next), num_tiles);
    if (CLOSE && after_closing(pt, num_tiles)) {
        // the closing phase resolved the three parked tiles: store them all
        // now (the control wave has left the loop; no barrier follows)
#pragma unroll 1
        for (int i = 0; i < 3; ++i) {
            const uint32_t t = i == 0 ? pt.prev3 : i == 1 ? pt.prev2 : pt.prev;
            if (t < num_tiles)
                store_parked<Op, D, Q, VEC>(sh, closing_slot(slot, i), t, sh.close_prefix[i], out, n, lane, d,
                                            lane_off);
        }
        return true;
    }
    return false;
}

template <class Op, int D, int Q, int G, bool INCL, bool VEC, bool STATS, bool CLOSE>
__device__ __forceinline__ void data_loop3(PipeTiles pt, ScanShared<Op, D, Q> &sh, typename IoOf<Op>::Src in,
                                           typename IoOf<Op>::Dst out, uint32_t n, uint32_t num_tiles, uint32_t *ctr,
                                           uint32_t lane, uint32_t d, uint32_t *stats) {
    using T = typename Op::T;
    constexpr uint32_t WAVE_ELEMS = (uint32_t)Q * 256u;
    const uint64_t lane_off = (uint64_t)d * WAVE_ELEMS + 4u * lane;
    // three register buffers in rotating roles (cur, f1, free); the phase
    // parity alternates independently, so it stays a run-time value
    WaveSpan<Op, Q> x, y, z;
    T lane_excl[Q], row_prefix[Q];
    uint32_t slot = 0;
    int par = 0;
    for (;;) {
        if (data_phase3<Op, D, Q, G, INCL, VEC, STATS, CLOSE>(x, y, z, par, slot, pt, lane_excl, row_prefix, sh, in, out, n,
                                                num_tiles, ctr, lane, d, lane_off, stats))
            break;
        par ^= 1;
        if (data_phase3<Op, D, Q, G, INCL, VEC, STATS, CLOSE>(y, z, x, par, slot, pt, lane_excl, row_prefix, sh, in, out, n,
                                                num_tiles, ctr, lane, d, lane_off, stats))
            break;
        par ^= 1;
        if (data_phase3<Op, D, Q, G, INCL, VEC, STATS, CLOSE>(z, x, y, par, slot, pt, lane_excl, row_prefix, sh, in, out, n,
                                                num_tiles, ctr, lane, d, lane_off, stats))
            break;
        par ^= 1;
    }
}

// A look-back's fallback: reduce tile p of the input from scratch, in tile
// order (rows of 256 elements; each lane folds its four, the wave scan joins
// the lanes, the rows are folded in order), and return the descriptor word
// its owner publishes first.  Runs on the control wave, rarely.
template <class Op, uint32_t TILE>
struct FlatFallback {
    typename IoOf<Op>::Src in;
    uint32_t n;
    __device__ DescVal<typename Op::T> operator()(uint32_t p, uint32_t lane) const {
        using T = typename Op::T;
        constexpr uint32_t ROWS = TILE / 256u, BATCH = 8u;
        static_assert(ROWS % BATCH == 0, "whole batches of rows");
        const uint64_t base = (uint64_t)p * TILE + 4u * lane;
        T acc = Op::id();
        for (uint32_t r = 0; r < ROWS; r += BATCH) {
            T part[BATCH];
#pragma unroll
            for (uint32_t k = 0; k < BATCH; ++k) {
                T v = Op::id();
#pragma unroll
                for (uint32_t e = 0; e < 4; ++e) {
                    const uint64_t i = base + (uint64_t)(r + k) * 256u + e;
                    v = Op::op(v, i < n ? load_elem<T>(in, i) : Op::id());
                }
                part[k] = v;
            }
#pragma unroll
            for (uint32_t k = 0; k < BATCH; ++k) acc = Op::op(acc, read_lane(wave_inclusive<Op>(part[k]), 63));
        }
        return DescVal<T>{p == 0 ? ST_PREFIX : ST_AGGREGATE, acc};
    }
};

// Whether a flat kernel ends with the closing phase (closing_phase in
// pipeline.hpp).  Two-word kernels (the widening scan, the recurrence) do:
// 528.3 -> 526.7 us for the widening scan at 2^28.  One-word ones do not:
// their last stores are bound by the write bandwidth, and the u32 scan at
// 2^28 ran about 1 us slower with the closing code in the kernel, also with
// the closing switched off at run time.
template <class Op>
constexpr bool flat_close() {
    return WordsFor<Op>::WORDS == 2;
}

template <class Op, int D, int Q, int LB_K, int G, bool INCL, bool VEC, bool STATS>
__global__ __launch_bounds__((D + 1) * 64) void chained_scan_kernel(
    typename IoOf<Op>::Src in, typename IoOf<Op>::Dst out, uint32_t n, uint32_t num_tiles, uint32_t *hdr,
    uint64_t *desc, typename Op::T *total, uint32_t *stats, int aggregate_only, LookbackCfg cfg) {
    __shared__ ScanShared<Op, D, Q> sh;
    __shared__ WsShared wsh;
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = uniform(threadIdx.x >> 6);
    uint32_t t0;
    const WsCall call = ws_start<G>(hdr, desc, num_tiles * (uint32_t)WordsFor<Op>::WORDS, num_tiles, wsh, t0);
    cfg.tf = tag_field(call.plan.tag);
    if (t0 < num_tiles) {
        const PipeTiles pt{num_tiles, num_tiles, num_tiles, num_tiles, num_tiles, t0};
        if (wave == 0) {
            ws_wait_clean(call, hdr);
            control_loop3<Op, D, LB_K, G, STATS, WordsFor<Op>::WORDS == 1, true, flat_close<Op>()>(
                pt, sh, num_tiles, hdr, desc, total, stats, aggregate_only, cfg,
                FlatFallback<Op, (uint32_t)D * Q * 256u>{in, n}, lane, STATS ? wsh.entry : 0u);
        } else {
            data_loop3<Op, D, Q, G, INCL, VEC, STATS, flat_close<Op>()>(pt, sh, in, out, n, num_tiles, hdr, lane,
                                                                        wave - 1, stats);
        }
    }
    if (wave == 0) ws_done(wsh, num_tiles * (uint32_t)WordsFor<Op>::WORDS, hdr, lane);
}

template <class T>
__global__ void write_one(T *p, T v) {
    *p = v;
}

// Flat scan shape: D data waves x Q groups of four elements per lane, plus
// the control wave; look-back width 64 * K predecessors per poll.
#ifndef DWPS_FLAT_D
#define DWPS_FLAT_D 8
#endif
#ifndef DWPS_FLAT_Q
#define DWPS_FLAT_Q 6
#endif
constexpr int kFlatD = DWPS_FLAT_D;
constexpr int kFlatQ = DWPS_FLAT_Q;
constexpr int kLookbackK = DWPS_LOOKBACK_K;
// Tiles claimed per ticket: a workgroup scans G consecutive tiles in
// consecutive phases, and only the first of them looks back.
#ifndef DWPS_TILES_PER_TICKET
#define DWPS_TILES_PER_TICKET 2
#endif
constexpr int kTilesPerTicket = DWPS_TILES_PER_TICKET;
constexpr int kFlatThreads = (kFlatD + 1) * 64;
constexpr uint32_t kFlatTile = kFlatD * kFlatQ * 256;

// 8-byte outputs take half the groups per lane, so a parked tile keeps the
// same LDS footprint (48 KiB).
template <class Op>
constexpr int flat_q() {
    return sizeof(typename Op::T) == 8 ? kFlatQ / 2 : kFlatQ;
}
// Look-back width: every lane reads kLookbackK descriptor words per poll, so
// with two words per tile (64-bit payloads) a poll covers half as many tiles.
template <class Op>
constexpr int flat_k() {
    // the recurrence's phases are long enough for a poll of two tiles per
    // lane (four words); the widening scan's are not
    if (std::is_same<Op, LinRecF32>::value) return 2;
    return kLookbackK / WordsFor<Op>::WORDS > 0 ? kLookbackK / WordsFor<Op>::WORDS : 1;
}
template <class Op>
constexpr uint32_t flat_tile() {
    return (uint32_t)kFlatD * (uint32_t)flat_q<Op>() * 256u;
}
inline uint64_t flat_tiles(uint64_t n) { return ceil_div(n, kFlatTile); }

// Workspace: header + descriptor words (one or two per tile).
template <class Op>
inline size_t flat_ws_bytes(uint64_t tiles) {
    return kWsHeader + round_up(tiles * 8u * (uint64_t)WordsFor<Op>::WORDS, 256);
}

// Which form a flat call runs: the single-pass chained scan, the two-level
// one, or (kAuto) the two-level one for n up to the ps_small_n_config
// setting.  Inputs up to kSmallNCap elements get a workspace that fits
// either form, so that a size query stays valid whatever the setting.
enum class FlatForm { kAuto, kSinglePass, kTwoLevel };

template <class Op>
inline size_t flat_form_ws_bytes(uint64_t n, FlatForm form) {
    const size_t single = flat_ws_bytes<Op>(ceil_div(n, flat_tile<Op>()));
    const size_t two = tl_ws_bytes<Op>(n);
    if (form == FlatForm::kTwoLevel) return two;
    if (form == FlatForm::kAuto && n <= kSmallNCap) return single > two ? single : two;
    return single;
}
inline bool use_two_level(uint64_t n, FlatForm form) {
    return form == FlatForm::kTwoLevel || (form == FlatForm::kAuto && n <= small_n_max());
}

// Launch the flat kernel on validated arguments (n > 0); the workspace is
// prepared and keeps itself ready (ws_state.hpp).  VEC: every array 16-byte aligned.  An in-place call runs without
// the fallback: a fallback reduces a predecessor from its input, which in
// place may already hold that predecessor's outputs.
template <class Op, bool STATS>
ps_status launch_flat_kernel(void *ws, size_t ws_need, typename IoOf<Op>::Src in, typename IoOf<Op>::Dst out,
                             uint32_t n, typename Op::T *total, bool inclusive, bool vec, bool in_place,
                             uint32_t *stats, int aggregate_only, hipStream_t s) {
    constexpr int Q = flat_q<Op>();
    constexpr int K = flat_k<Op>();
    (void)ws_need;
    uint32_t *ctr = ws_counter(ws);
    uint64_t *desc = ws_desc(ws);
    const uint32_t nt = (uint32_t)ceil_div(n, flat_tile<Op>());
    const LookbackCfg cfg = lookback_cfg(in_place);
    auto launch = [&](auto kernel) -> ps_status {
        const uint32_t grid = persistent_grid(reinterpret_cast<const void *>(kernel), kFlatThreads, nt);
        if (!grid) return PS_ERR_HIP;
        timing_begin(s);
        hipLaunchKernelGGL(kernel, dim3(grid), dim3(kFlatThreads), 0, s, in, out, n, nt, ctr, desc, total, stats,
                           aggregate_only, cfg);
        return PS_OK;
    };
    ps_status r;
    if constexpr (STATS) {
        if (!vec) return PS_ERR_ALIGNMENT;  // instrumented for the vector path only
        r = inclusive ? launch(chained_scan_kernel<Op, kFlatD, Q, K, kTilesPerTicket, true, true, STATS>)
                      : launch(chained_scan_kernel<Op, kFlatD, Q, K, kTilesPerTicket, false, true, STATS>);
    } else if (inclusive) {
        r = vec ? launch(chained_scan_kernel<Op, kFlatD, Q, K, kTilesPerTicket, true, true, STATS>)
                : launch(chained_scan_kernel<Op, kFlatD, Q, K, kTilesPerTicket, true, false, STATS>);
    } else {
        r = vec ? launch(chained_scan_kernel<Op, kFlatD, Q, K, kTilesPerTicket, false, true, STATS>)
                : launch(chained_scan_kernel<Op, kFlatD, Q, K, kTilesPerTicket, false, false, STATS>);
    }
    if (r != PS_OK) return r;
    timing_end(s);
    return launch_status();
}

template <class Op, bool STATS>
ps_status launch_flat(void *ws, size_t *ws_bytes, const void *in_v, void *out_v, uint64_t n, void *total_v,
                      bool inclusive, uint32_t *stats, hipStream_t s, typename Op::T identity,
                      int aggregate_only = 0, FlatForm form = FlatForm::kAuto) {
    using T = typename Op::T;
    using In = typename InputOf<Op>::type;
    if (n >= (1ull << 32)) return PS_ERR_SIZE;
    if (STATS) form = FlatForm::kSinglePass;
    const size_t ws_need = flat_form_ws_bytes<Op>(n, form);
    bool query = false;
    ps_status st = workspace_protocol(ws, ws_bytes, ws_need, &query);
    if (st != PS_OK || query) return st;
    const In *in = static_cast<const In *>(in_v);
    T *out = static_cast<T *>(out_v);
    T *total = static_cast<T *>(total_v);
    if (n == 0) {
        if (!total) return PS_OK;
        if (!aligned(total, sizeof(T))) return PS_ERR_ALIGNMENT;
        hipLaunchKernelGGL(write_one<T>, dim3(1), dim3(1), 0, s, total, identity);
        return launch_status();
    }
    if (!in || !out) return PS_ERR_NULL;
    if (STATS && !stats) return PS_ERR_NULL;
    if (!aligned(in, sizeof(In)) || !aligned(out, sizeof(T)) || (total && !aligned(total, sizeof(T))) ||
        !aligned(ws, 16))
        return PS_ERR_ALIGNMENT;
    // exact in-place is allowed when input and output elements have one size
    const bool in_place = sizeof(In) == sizeof(T) && in_v == (const void *)out_v;
    if (!in_place && ranges_overlap(in, n * sizeof(In), out, n * sizeof(T))) return PS_ERR_ALIAS;
    const bool vec = aligned(in, 16) && aligned(out, 16);
    if (use_two_level(n, form)) return tl_launch<Op>(ws, in, out, (uint32_t)n, total, inclusive, vec, s);
    return launch_flat_kernel<Op, STATS>(ws, ws_need, in, out, (uint32_t)n, total, inclusive, vec, in_place, stats,
                                         aggregate_only, s);
}

// The recurrence pairs come in two float planes and go out in two (out_a
// optional).  Exact in-place use of either plane is allowed; any other
// overlap between an input and an output, or between the outputs, is not.
template <bool STATS>
ps_status launch_linrec(void *ws, size_t *ws_bytes, const float *a, const float *b, float *out_a, float *out_b,
                        uint64_t n, bool inclusive, float *total, uint32_t *stats, hipStream_t s) {
    if (n >= (1ull << 32)) return PS_ERR_SIZE;
    const size_t ws_need = flat_form_ws_bytes<LinRecF32>(n, FlatForm::kAuto);
    bool query = false;
    ps_status st = workspace_protocol(ws, ws_bytes, ws_need, &query);
    if (st != PS_OK || query) return st;
    F2 *tot = reinterpret_cast<F2 *>(total);
    if (n == 0) {
        if (!total) return PS_OK;
        if (!aligned(total, sizeof(float))) return PS_ERR_ALIGNMENT;
        hipLaunchKernelGGL(write_one<F2>, dim3(1), dim3(1), 0, s, tot, F2{1.0f, 0.0f});
        return launch_status();
    }
    if (!a || !b || !out_b || (STATS && !stats)) return PS_ERR_NULL;
    if (!aligned(a, 4) || !aligned(b, 4) || !aligned(out_b, 4) || (out_a && !aligned(out_a, 4)) ||
        (total && !aligned(total, 4)) || !aligned(ws, 16))
        return PS_ERR_ALIGNMENT;
    const uint64_t bytes = n * sizeof(float);
    const float *ins[2] = {a, b};
    float *outs[2] = {out_a, out_b};
    bool in_place = false;
    for (int o = 0; o < 2; ++o) {
        if (!outs[o]) continue;
        for (int i = 0; i < 2; ++i) {
            if (ins[i] == outs[o] && i == o) {
                in_place = true;
                continue;
            }
            if (ranges_overlap(ins[i], bytes, outs[o], bytes)) return PS_ERR_ALIAS;
        }
    }
    if (out_a && ranges_overlap(out_a, bytes, out_b, bytes)) return PS_ERR_ALIAS;
    const bool vec = aligned(a, 16) && aligned(b, 16) && aligned(out_b, 16) && (!out_a || aligned(out_a, 16));
    if (!STATS && use_two_level(n, FlatForm::kAuto))
        return tl_launch<LinRecF32>(ws, PlanesIn{a, b}, PlanesOut{out_a, out_b}, (uint32_t)n, tot, inclusive, vec, s);
    return launch_flat_kernel<LinRecF32, STATS>(ws, ws_need, PlanesIn{a, b}, PlanesOut{out_a, out_b}, (uint32_t)n,
                                                tot, inclusive, vec, in_place, stats, 0, s);
}

}  // namespace dwps

using namespace dwps;

extern "C" ps_status ps_scan_exclusive_u32(void *ws, size_t *ws_bytes, const uint32_t *in, uint32_t *out,
                                           uint64_t n, uint32_t *total, void *stream) {
    return launch_flat<SumU32, false>(ws, ws_bytes, in, out, n, total, false, nullptr,
                                      static_cast<hipStream_t>(stream), 0u);
}

extern "C" ps_status ps_scan_inclusive_u32(void *ws, size_t *ws_bytes, const uint32_t *in, uint32_t *out,
                                           uint64_t n, uint32_t *total, void *stream) {
    return launch_flat<SumU32, false>(ws, ws_bytes, in, out, n, total, true, nullptr,
                                      static_cast<hipStream_t>(stream), 0u);
}

extern "C" ps_status ps_scan_exclusive_u32_u64(void *ws, size_t *ws_bytes, const uint32_t *in, uint64_t *out,
                                               uint64_t n, uint64_t *total, void *stream) {
    return launch_flat<SumU32toU64, false>(ws, ws_bytes, in, out, n, total, false, nullptr,
                                           static_cast<hipStream_t>(stream), 0ull);
}

extern "C" ps_status ps_scan_inclusive_u32_u64(void *ws, size_t *ws_bytes, const uint32_t *in, uint64_t *out,
                                               uint64_t n, uint64_t *total, void *stream) {
    return launch_flat<SumU32toU64, false>(ws, ws_bytes, in, out, n, total, true, nullptr,
                                           static_cast<hipStream_t>(stream), 0ull);
}

extern "C" ps_status ps_scan_exclusive_f32(void *ws, size_t *ws_bytes, const float *in, float *out, uint64_t n,
                                           float *total, void *stream) {
    return launch_flat<SumF32, false>(ws, ws_bytes, in, out, n, total, false, nullptr,
                                      static_cast<hipStream_t>(stream), 0.0f);
}

extern "C" ps_status ps_scan_inclusive_f32(void *ws, size_t *ws_bytes, const float *in, float *out, uint64_t n,
                                           float *total, void *stream) {
    return launch_flat<SumF32, false>(ws, ws_bytes, in, out, n, total, true, nullptr,
                                      static_cast<hipStream_t>(stream), 0.0f);
}

extern "C" ps_status ps_scan_linrec_f32(void *ws, size_t *ws_bytes, const float *a, const float *b, float *out_a,
                                        float *out_b, uint64_t n, int inclusive, float *total, void *stream) {
    return launch_linrec<false>(ws, ws_bytes, a, b, out_a, out_b, n, inclusive != 0, total, nullptr,
                                static_cast<hipStream_t>(stream));
}

extern "C" ps_status ps_linrec_lookback_stats(void *ws, size_t *ws_bytes, const float *a, const float *b,
                                             float *out_a, float *out_b, uint64_t n, int inclusive, uint32_t *stats,
                                             void *stream) {
    return launch_linrec<true>(ws, ws_bytes, a, b, out_a, out_b, n, inclusive != 0, nullptr, stats,
                               static_cast<hipStream_t>(stream));
}

extern "C" uint32_t ps_linrec_tile_elements(void) { return flat_tile<LinRecF32>(); }

// ---------------------------------------------------------------------------
// Staged compaction: the ablation of the fused kernel in compact.hip.  Two
// launches of separate passes over the whole array, the composition of
// "Prefix scans and compaction", section "Worked example: Stable stream
// compaction": an exclusive scan of the keep flags (uint8 -> uint32
// offsets, the flat scan above), then a scatter of every kept record to its
// offset.  Traffic per record: 1 + 4 bytes for the scan, 1 + 4 + R for the
// scatter, R per kept record, against the fused kernel's 1 + R and R per
// kept record.
// ---------------------------------------------------------------------------
template <class Rec>
__global__ __launch_bounds__(256) void scatter_kept_kernel(const Rec *rec, const uint8_t *flags,
                                                          const uint32_t *offsets, uint32_t n, Rec *out,
                                                          const uint32_t *count, uint64_t *num_selected,
                                                          uint32_t *hdr, uint32_t dirty_a, uint32_t dirty_b) {
    const uint64_t i = (uint64_t)blockIdx.x * 256u + threadIdx.x;
    if (i == 0) {
        const uint32_t c = *count;
        *num_selected = c < n ? c : n;
        // the offsets and the count are plain data in descriptor words
        uint32_t lo = hdr[kHdrDirtyLo], hi = hdr[kHdrDirtyHi];
        ws_mark_dirty(lo, hi, dirty_a, dirty_b);
        hdr[kHdrDirtyLo] = lo;
        hdr[kHdrDirtyHi] = hi;
    }
    if (i < n && flags[i] != 0) {
        const uint32_t o = offsets[i];
        if (o < n) out[o] = rec[i];
    }
}

__global__ void write_count_zero_staged(uint64_t *p) { *p = 0ull; }

template <class Rec>
ps_status launch_compact_staged(void *ws, size_t *ws_bytes, const void *records, const uint8_t *flags, uint64_t n,
                                void *out, uint64_t *num_selected, hipStream_t s) {
    // workspace: [scan workspace][offsets: n uint32][count]
    size_t scan_bytes = flat_form_ws_bytes<CountFlags>(n, FlatForm::kAuto);
    const size_t off_at = round_up(scan_bytes, 256), cnt_at = off_at + round_up(n * 4u, 256);
    bool query = false;
    ps_status st = workspace_protocol(ws, ws_bytes, cnt_at + 256, &query);
    if (st != PS_OK || query) return st;
    if (!num_selected) return PS_ERR_NULL;
    if (!aligned(num_selected, 8)) return PS_ERR_ALIGNMENT;
    if (n == 0) {
        hipLaunchKernelGGL(write_count_zero_staged, dim3(1), dim3(1), 0, s, num_selected);
        return launch_status();
    }
    if (!records || !flags || !out) return PS_ERR_NULL;
    if (!aligned(records, sizeof(Rec)) || !aligned(out, sizeof(Rec)) || !aligned(ws, 16)) return PS_ERR_ALIGNMENT;
    const size_t bytes = n * sizeof(Rec);
    if (ranges_overlap(out, bytes, records, bytes) || ranges_overlap(out, bytes, flags, n) ||
        ranges_overlap(num_selected, 8, out, bytes))
        return PS_ERR_ALIAS;
    char *base = static_cast<char *>(ws);
    uint32_t *offsets = reinterpret_cast<uint32_t *>(base + off_at);
    uint32_t *count = reinterpret_cast<uint32_t *>(base + cnt_at);
    st = launch_flat<CountFlags, false>(ws, &scan_bytes, flags, offsets, n, count, false, nullptr, s, 0u);
    if (st != PS_OK) return st;
    timing_begin(s);
    // descriptor words holding the offsets and the count, left dirty
    const uint32_t dirty_a = (uint32_t)((off_at - kWsHeader) / 8u);
    const uint32_t dirty_b = (uint32_t)((cnt_at + 256u - kWsHeader) / 8u);
    hipLaunchKernelGGL(scatter_kept_kernel<Rec>, dim3((uint32_t)ceil_div(n, 256)), dim3(256), 0, s,
                       static_cast<const Rec *>(records), flags, offsets, (uint32_t)n, static_cast<Rec *>(out), count,
                       num_selected, ws_counter(ws), dirty_a, dirty_b);
    timing_end(s);
    return launch_status();
}

namespace {

template <class Op>
ps_status generic(void *ws, size_t *ws_bytes, const void *in, void *out, uint64_t n, void *total, bool inc,
                  hipStream_t s, typename Op::T identity, FlatForm form) {
    return launch_flat<Op, false>(ws, ws_bytes, in, out, n, total, inc, nullptr, s, identity, 0, form);
}

ps_status scan_any(void *ws, size_t *ws_bytes, ps_op op, ps_dtype dtype, int inclusive, const void *in, void *out,
                   uint64_t n, void *total, hipStream_t s, FlatForm form) {
    const bool inc = inclusive != 0;
    if (dtype == PS_U32) {
        switch (op) {
        case PS_OP_SUM: return generic<SumU32>(ws, ws_bytes, in, out, n, total, inc, s, 0u, form);
        case PS_OP_MAX: return generic<MaxU32>(ws, ws_bytes, in, out, n, total, inc, s, 0u, form);
        case PS_OP_MIN: return generic<MinU32>(ws, ws_bytes, in, out, n, total, inc, s, 0xFFFFFFFFu, form);
        case PS_OP_AND: return generic<AndU32>(ws, ws_bytes, in, out, n, total, inc, s, 0xFFFFFFFFu, form);
        case PS_OP_OR: return generic<OrU32>(ws, ws_bytes, in, out, n, total, inc, s, 0u, form);
        case PS_OP_XOR: return generic<XorU32>(ws, ws_bytes, in, out, n, total, inc, s, 0u, form);
        case PS_OP_AFFINE16: return generic<Affine16>(ws, ws_bytes, in, out, n, total, inc, s, 0x00010000u, form);
        }
        return PS_ERR_UNSUPPORTED;
    }
    if (dtype == PS_U64) {
        if (op != PS_OP_SUM) return PS_ERR_UNSUPPORTED;
        return generic<SumU32toU64>(ws, ws_bytes, in, out, n, total, inc, s, 0ull, form);
    }
    if (dtype == PS_F32) {
        switch (op) {
        case PS_OP_SUM: return generic<SumF32>(ws, ws_bytes, in, out, n, total, inc, s, 0.0f, form);
        case PS_OP_MAX: return generic<MaxF32>(ws, ws_bytes, in, out, n, total, inc, s, -__builtin_huge_valf(), form);
        case PS_OP_MIN: return generic<MinF32>(ws, ws_bytes, in, out, n, total, inc, s, __builtin_huge_valf(), form);
        default: return PS_ERR_UNSUPPORTED;
        }
    }
    return PS_ERR_UNSUPPORTED;
}

}  // namespace

extern "C" ps_status ps_scan(void *ws, size_t *ws_bytes, ps_op op, ps_dtype dtype, int inclusive, const void *in,
                             void *out, uint64_t n, void *total, void *stream) {
    return scan_any(ws, ws_bytes, op, dtype, inclusive, in, out, n, total, static_cast<hipStream_t>(stream),
                    FlatForm::kAuto);
}

// ---------------------------------------------------------------------------
// ps_scan_noalloc: ps_scan on a workspace that lives in the library itself,
// for callers that cannot allocate device memory.  The array below is that
// workspace, one copy per device; its address is looked up once per device
// (in host code its name is not a device address) and the header is
// prepared by the same first call, on its stream.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = (size_t)4 << 20;
static __device__ __align__(256) uint64_t scratch[kScratchBytes / 8];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];  // per device; null until set up

ps_status scratch_for_current_device(hipStream_t s, void **ptr) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PS_ERR_HIP;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return PS_ERR_HIP;
        if (launch_ws_init(p, kScratchBytes, s) != hipSuccess) return PS_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return PS_OK;
}
}  // namespace

extern "C" ps_status ps_scan_noalloc(ps_op op, ps_dtype dtype, int inclusive, const void *in, void *out, uint64_t n,
                                     void *total, void *stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    size_t need = 0;
    const ps_status q = scan_any(nullptr, &need, op, dtype, inclusive, in, out, n, total, s, FlatForm::kAuto);
    if (q != PS_OK) return q;
    if (need > kScratchBytes) return PS_ERR_SIZE;
    void *ws = nullptr;
    const ps_status st = scratch_for_current_device(s, &ws);
    if (st != PS_OK) return st;
    size_t have = kScratchBytes;
    return scan_any(ws, &have, op, dtype, inclusive, in, out, n, total, s, FlatForm::kAuto);
}

extern "C" size_t ps_scan_noalloc_bytes(void) { return kScratchBytes; }

extern "C" ps_status ps_scan_single_pass(void *ws, size_t *ws_bytes, ps_op op, ps_dtype dtype, int inclusive,
                                         const void *in, void *out, uint64_t n, void *total, void *stream) {
    return scan_any(ws, ws_bytes, op, dtype, inclusive, in, out, n, total, static_cast<hipStream_t>(stream),
                    FlatForm::kSinglePass);
}

extern "C" ps_status ps_scan_two_level(void *ws, size_t *ws_bytes, ps_op op, ps_dtype dtype, int inclusive,
                                       const void *in, void *out, uint64_t n, void *total, void *stream) {
    return scan_any(ws, ws_bytes, op, dtype, inclusive, in, out, n, total, static_cast<hipStream_t>(stream),
                    FlatForm::kTwoLevel);
}

extern "C" uint32_t ps_two_level_tile_elements(void) { return kTlTile; }

extern "C" ps_status ps_lookback_stats_u32(void *ws, size_t *ws_bytes, const uint32_t *in, uint32_t *out,
                                           uint64_t n, uint32_t *stats, int aggregate_only, void *stream) {
    return launch_flat<SumU32, true>(ws, ws_bytes, in, out, n, nullptr, false, stats,
                                     static_cast<hipStream_t>(stream), 0u, aggregate_only);
}

extern "C" ps_status ps_scan_lookback_stats(void *ws, size_t *ws_bytes, ps_op op, ps_dtype dtype, int inclusive,
                                            const void *in, void *out, uint64_t n, uint32_t *stats, void *stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool inc = inclusive != 0;
    if (op == PS_OP_SUM && dtype == PS_U32)
        return launch_flat<SumU32, true>(ws, ws_bytes, in, out, n, nullptr, inc, stats, s, 0u);
    if (op == PS_OP_SUM && dtype == PS_F32)
        return launch_flat<SumF32, true>(ws, ws_bytes, in, out, n, nullptr, inc, stats, s, 0.0f);
    if (op == PS_OP_MAX && dtype == PS_F32)
        return launch_flat<MaxF32, true>(ws, ws_bytes, in, out, n, nullptr, inc, stats, s, -__builtin_huge_valf());
    return PS_ERR_UNSUPPORTED;
}

extern "C" uint64_t ps_lookback_tiles(uint64_t n) { return flat_tiles(n); }

extern "C" uint32_t ps_lookback_window(void) { return 64u * (uint32_t)kLookbackK; }

extern "C" uint32_t ps_lookback_group(void) { return (uint32_t)kTilesPerTicket; }

extern "C" uint32_t ps_tile_elements(ps_dtype dtype) {
    return dtype == PS_U64 ? flat_tile<SumU32toU64>() : kFlatTile;
}

extern "C" ps_status ps_compact_staged(void *ws, size_t *ws_bytes, const void *records, uint32_t record_bytes,
                                       const uint8_t *flags, uint64_t n, void *out, uint64_t *num_selected,
                                       void *stream) {
    if (n >= (1ull << 32)) return PS_ERR_SIZE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    switch (record_bytes) {
    case 4: return launch_compact_staged<uint32_t>(ws, ws_bytes, records, flags, n, out, num_selected, s);
    case 8: return launch_compact_staged<uint2>(ws, ws_bytes, records, flags, n, out, num_selected, s);
    case 16: return launch_compact_staged<uint4>(ws, ws_bytes, records, flags, n, out, num_selected, s);
    default: return PS_ERR_UNSUPPORTED;
    }
}
