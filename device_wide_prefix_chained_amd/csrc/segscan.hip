// segscan.hip -- segmented uint32 sum scan over CSR offsets, single pass.
//
// Contract: "GPUSegmentedScan", sections "Prefix scans and segmented scans",
// "Contract" and "Limitations" (segment s is [offsets[s], offsets[s+1]), the
// running total restarts at every segment, empty segments write nothing,
// offsets are trusted on the hot path).  The scan itself is the flat chained
// scan with the operator of the carried segment flag ("Parallel Prefix Sum
// (Scan), in depth", section "What scan builds"):
//     (f1, v1) (+) (f2, v2) = (f1 | f2,  f2 ? v2 : v1 + v2).
//
// Strategy selection by segment size, inside one launch (the page's
// "Performance notes" call for it without building it):
//   * a segment that starts and ends inside one lane's 4 elements, one wave's
//     span or one tile is finished by the lane-serial, DPP wave or LDS block
//     layer -- it never waits on another workgroup;
//   * a tile that contains a segment head knows its carry-out without looking
//     back (the sum since its last head), so it publishes PREFIX at once and
//     cuts every look-back chain that reaches it;
//   * only tiles without a head (inside a segment longer than a tile) publish
//     AGGREGATE and wait, exactly like the flat scan; a tile whose first
//     element is a head needs no carry and does not look back at all.
// Heads are found per tile without host readback: two 64-way searches of the
// offsets give the range of segment starts inside the tile, and those starts
// set bits in an LDS bitmap (duplicate offsets -- empty segments -- set the
// same bit).
#include <hip/hip_runtime.h>

#include "dwps_device.hpp"
#include "host_common.hpp"

namespace dwps {

// First index s in [0, count) with a[s] >= key (count if none), searched by
// one full wave: 64 probes per round narrow the range 64-fold, so 65 537
// offsets take three dependent rounds.  Reads stay inside [0, count) even if
// `a` is not sorted.
__device__ __forceinline__ uint32_t wave_lower_bound(const uint32_t *a, uint32_t count, uint32_t key,
                                                     uint32_t lane) {
    uint32_t lo = 0, hi = count;
    while (hi - lo > 64u) {
        const uint32_t step = (hi - lo + 63u) / 64u;
        const uint32_t p = lo + lane * step;
        const bool less = (p < hi) && (a[p] < key);
        const uint32_t c = (uint32_t)__builtin_popcountll(ballot(less));
        if (c == 0) return lo;
        const uint32_t old_lo = lo;
        lo = old_lo + (c - 1u) * step + 1u;
        const uint32_t next_probe = old_lo + c * step;
        hi = next_probe < hi ? next_probe : hi;
    }
    const uint32_t p = lo + lane;
    const bool less = (p < hi) && (a[p] < key);
    return lo + (uint32_t)__builtin_popcountll(ballot(less));
}

struct SegPair {
    uint32_t f;  // 1 if the covered range contains a segment head
    uint32_t v;  // sum since the last head in the range (the whole range if none)
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

template <int NT, int Q, bool INCL, bool VEC>
__global__ __launch_bounds__(NT) void segscan_kernel(const uint32_t *values, uint32_t *out, uint32_t n,
                                                     const uint32_t *offsets, uint32_t num_segments,
                                                     uint32_t *ctr, uint64_t *desc) {
    static_assert(NT >= 128, "two waves run the two offset searches");
    constexpr int NW = NT / 64;
    constexpr uint32_t WAVE_ELEMS = (uint32_t)Q * 256u;
    constexpr uint32_t TILE = (uint32_t)NT * (uint32_t)Q * 4u;
    constexpr uint32_t BITWORDS = TILE / 32u;

    __shared__ uint32_t s_tile, s_lo, s_hi, s_carry;
    __shared__ uint32_t s_heads[BITWORDS];
    __shared__ uint32_t s_wf[NW], s_wv[NW];

    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & 63u;
    const uint32_t wave = tid >> 6;

    if (tid == 0) s_tile = take_ticket(ctr);
    for (uint32_t i = tid; i < BITWORDS; i += NT) s_heads[i] = 0u;
    __syncthreads();
    const uint32_t tile = s_tile;
    const uint64_t tile_base = (uint64_t)tile * TILE;
    const uint32_t tb = (uint32_t)tile_base;  // < n < 2^32
    const uint64_t tile_end64 = tile_base + TILE;
    const uint32_t te = tile_end64 < (uint64_t)n ? (uint32_t)tile_end64 : n;
    const bool full = tile_end64 <= (uint64_t)n;
    const uint64_t span = tile_base + (uint64_t)wave * WAVE_ELEMS + 4u * lane;

    // values first, so their latency overlaps the offset searches
    uint32_t x[Q][4];
    if (VEC && full) {
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const uint4 r = *reinterpret_cast<const uint4 *>(values + span + (uint64_t)q * 256u);
            x[q][0] = r.x;
            x[q][1] = r.y;
            x[q][2] = r.z;
            x[q][3] = r.w;
        }
    } else {
#pragma unroll
        for (int q = 0; q < Q; ++q)
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint64_t i = span + (uint64_t)q * 256u + k;
                x[q][k] = (i < n) ? values[i] : 0u;
            }
    }
    uint32_t row_lo = offsets[0];
    uint32_t row_hi = offsets[num_segments];
    row_lo = row_lo < n ? row_lo : n;
    row_hi = row_hi < n ? row_hi : n;

    if (wave == 0) {
        const uint32_t r = wave_lower_bound(offsets, num_segments + 1u, tb, lane);
        if (lane == 0) s_lo = r;
    } else if (wave == 1) {
        const uint32_t r = wave_lower_bound(offsets, num_segments + 1u, te, lane);
        if (lane == 0) s_hi = r;
    }
    __syncthreads();
    {
        const uint32_t lo = s_lo, hi = s_hi;
        for (uint32_t s = lo + tid; s < hi; s += NT) {
            const uint32_t o = offsets[s];
            if (o >= tb && o < te) atomicOr(&s_heads[(o - tb) >> 5], 1u << ((o - tb) & 31u));
        }
    }
    __syncthreads();

    // lane-serial segmented scan of each group of four
    uint32_t fl[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const uint32_t li = wave * WAVE_ELEMS + (uint32_t)q * 256u + 4u * lane;
        fl[q] = (s_heads[li >> 5] >> (li & 31u)) & 0xFu;
        x[q][1] = (fl[q] & 2u) ? x[q][1] : x[q][0] + x[q][1];
        x[q][2] = (fl[q] & 4u) ? x[q][2] : x[q][1] + x[q][2];
        x[q][3] = (fl[q] & 8u) ? x[q][3] : x[q][2] + x[q][3];
    }
    // wave scans of the group pairs, then the wave pairs through LDS
    SegPair lane_excl[Q], group_prefix[Q];
    SegPair run{0u, 0u};
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        uint32_t f = fl[q] ? 1u : 0u, v = x[q][3];
        wave_seg_inclusive(f, v);
        lane_excl[q].f = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)f, 0x138, 0xF, 0xF, false);
        lane_excl[q].v = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x138, 0xF, 0xF, false);
        group_prefix[q] = run;
        run = seg_op(run, SegPair{(uint32_t)__builtin_amdgcn_readlane((int)f, 63),
                                  (uint32_t)__builtin_amdgcn_readlane((int)v, 63)});
    }
    if (lane == 0) {
        s_wf[wave] = run.f;
        s_wv[wave] = run.v;
    }
    __syncthreads();
    SegPair wave_prefix{0u, 0u}, agg{0u, 0u};
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const SegPair t{s_wf[w], s_wv[w]};
        if ((uint32_t)w < wave) wave_prefix = seg_op(wave_prefix, t);
        agg = seg_op(agg, t);
    }

    // grid level: heads publish at once; head-free tiles chain like the flat scan
    if (wave == 0) {
        LookbackStats st;
        uint32_t carry = 0u;
        const bool first_is_head = (s_heads[0] & 1u) != 0u;
        if (tile == 0) {
            if (lane == 0) desc_publish(desc, desc_word(ST_PREFIX, agg.v));
        } else if (agg.f) {
            if (lane == 0) desc_publish(desc + tile, desc_word(ST_PREFIX, agg.v));
            if (!first_is_head) carry = lookback<SumU32, DWPS_LOOKBACK_K, false>(desc, tile, lane, st, ctr + 1);
        } else {
            if (lane == 0) desc_publish(desc + tile, desc_word(ST_AGGREGATE, agg.v));
            carry = lookback<SumU32, DWPS_LOOKBACK_K, false>(desc, tile, lane, st, ctr + 1);
            if (lane == 0) desc_publish(desc + tile, desc_word(ST_PREFIX, carry + agg.v));
        }
        if (lane == 0) s_carry = carry;
    }
    __syncthreads();

    const SegPair base = seg_op(SegPair{0u, s_carry}, wave_prefix);
    const bool vec_store = VEC && full && tb >= row_lo && tile_end64 <= (uint64_t)row_hi;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const uint32_t c = seg_op(seg_op(base, group_prefix[q]), lane_excl[q]).v;
        uint32_t inc[4], o[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const bool seen = (fl[q] & ((2u << k) - 1u)) != 0u;  // a head among elements 0..k
            inc[k] = seen ? x[q][k] : c + x[q][k];
        }
        if (INCL) {
#pragma unroll
            for (int k = 0; k < 4; ++k) o[k] = inc[k];
        } else {
            o[0] = (fl[q] & 1u) ? 0u : c;
#pragma unroll
            for (int k = 1; k < 4; ++k) o[k] = (fl[q] & (1u << k)) ? 0u : inc[k - 1];
        }
        if (vec_store) {
            *reinterpret_cast<uint4 *>(out + span + (uint64_t)q * 256u) = make_uint4(o[0], o[1], o[2], o[3]);
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint64_t i = span + (uint64_t)q * 256u + k;
                if (i >= row_lo && i < row_hi) out[i] = o[k];
            }
        }
    }
}

constexpr int kSegNT = 256;
constexpr int kSegQ = 4;
constexpr uint32_t kSegTile = kSegNT * kSegQ * 4;

}  // namespace dwps

using namespace dwps;

extern "C" ps_status ps_segmented_scan_u32(void *ws, size_t *ws_bytes, const uint32_t *values, uint64_t n,
                                           const uint32_t *offsets, uint32_t num_segments, uint32_t *out,
                                           int inclusive, void *stream) {
    if (n >= (1ull << 32)) return PS_ERR_SIZE;
    const uint64_t tiles = ceil_div(n, kSegTile);
    bool query = false;
    ps_status st = workspace_protocol(ws, ws_bytes, ws_bytes_for_tiles(tiles), &query);
    if (st != PS_OK || query) return st;
    if (n == 0 || num_segments == 0) return PS_OK;
    if (!values || !offsets || !out) return PS_ERR_NULL;
    if (!aligned(values, 4) || !aligned(offsets, 4) || !aligned(out, 4)) return PS_ERR_ALIGNMENT;
    if (ranges_overlap(out, n * 4, values, n * 4) ||
        ranges_overlap(out, n * 4, offsets, ((size_t)num_segments + 1) * 4))
        return PS_ERR_ALIAS;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (launch_clear(ws, ws_bytes_for_tiles(tiles), s) != hipSuccess) return PS_ERR_HIP;
    const bool vec = aligned(values, 16) && aligned(out, 16);
    const dim3 grid((unsigned)tiles), block(kSegNT);
    uint32_t *ctr = ws_counter(ws);
    uint64_t *desc = ws_desc(ws);
    const uint32_t n32 = (uint32_t)n;
    timing_begin(s);
    if (inclusive) {
        if (vec)
            hipLaunchKernelGGL((segscan_kernel<kSegNT, kSegQ, true, true>), grid, block, 0, s, values, out, n32,
                               offsets, num_segments, ctr, desc);
        else
            hipLaunchKernelGGL((segscan_kernel<kSegNT, kSegQ, true, false>), grid, block, 0, s, values, out, n32,
                               offsets, num_segments, ctr, desc);
    } else {
        if (vec)
            hipLaunchKernelGGL((segscan_kernel<kSegNT, kSegQ, false, true>), grid, block, 0, s, values, out, n32,
                               offsets, num_segments, ctr, desc);
        else
            hipLaunchKernelGGL((segscan_kernel<kSegNT, kSegQ, false, false>), grid, block, 0, s, values, out,
                               n32, offsets, num_segments, ctr, desc);
    }
    timing_end(s);
    return launch_status();
}
