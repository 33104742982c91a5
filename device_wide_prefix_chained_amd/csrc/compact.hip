// compact.hip -- stable stream compaction fused with its scan, single pass.
//
// "Prefix scans and compaction", sections "Scan as an index generator" and
// "Worked example: Stable stream compaction", and "Parallel Prefix Sum (Scan),
// in depth", section "What scan builds": the destination of a kept record is
// the exclusive scan of the keep flags at its position, so kept records land
// densely and in input order; the count is the last offset plus the last
// flag.  The offsets are never written to memory (the page's advice to avoid
// materialising the flags and prefixes): each tile scans its flags in
// registers, takes its output base from the chained look-back over per-tile
// counts, and writes its kept records straight to their destinations.
//
// Tile: NT threads x R records.  Wave w owns 64*R consecutive records; step r
// of lane l handles record (w*64*R + r*64 + l), so every step of a wave reads
// 64 consecutive flag bytes and up to 64 consecutive records.  Within a step
// the flag scan is a ballot plus a lane-masked popcount (v_mbcnt), the
// rank of a kept record among the kept records of earlier lanes.
#include <hip/hip_runtime.h>

#include "dwps_device.hpp"
#include "host_common.hpp"

namespace dwps {

__device__ __forceinline__ uint32_t lane_rank(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

template <class Rec, int NT, int R>
__global__ __launch_bounds__(NT) void compact_kernel(const Rec *records, const uint8_t *flags, uint32_t n,
                                                     Rec *out, uint64_t *num_selected, uint32_t num_tiles,
                                                     uint32_t *ctr, uint64_t *desc) {
    constexpr int NW = NT / 64;
    constexpr uint32_t WAVE_RECS = (uint32_t)R * 64u;
    constexpr uint32_t TILE = (uint32_t)NT * (uint32_t)R;

    __shared__ uint32_t s_tile;
    __shared__ uint32_t s_wave[NW];
    __shared__ uint32_t s_base;

    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & 63u;
    const uint32_t wave = tid >> 6;

    if (tid == 0) s_tile = take_ticket(ctr);
    __syncthreads();
    const uint32_t tile = s_tile;
    const uint64_t first = (uint64_t)tile * TILE + (uint64_t)wave * WAVE_RECS + lane;

    bool keep[R];
    Rec rec[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const uint64_t i = first + (uint64_t)r * 64u;
        keep[r] = (i < n) && flags[i] != 0;
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const uint64_t i = first + (uint64_t)r * 64u;
        if (keep[r]) rec[r] = records[i];
    }
    uint32_t rank[R], step_prefix[R];
    uint32_t run = 0u;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const uint64_t m = ballot(keep[r]);
        rank[r] = lane_rank(m);
        step_prefix[r] = run;
        run += (uint32_t)__builtin_popcountll(m);
    }
    if (lane == 0) s_wave[wave] = run;
    __syncthreads();
    uint32_t wave_prefix = 0u, count = 0u;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const uint32_t t = s_wave[w];
        if ((uint32_t)w < wave) wave_prefix += t;
        count += t;
    }
    if (wave == 0) {
        LookbackStats st;
        uint32_t excl = 0u;
        if (tile == 0) {
            if (lane == 0) desc_publish(desc, desc_word(ST_PREFIX, count));
        } else {
            if (lane == 0) desc_publish(desc + tile, desc_word(ST_AGGREGATE, count));
            excl = lookback<SumU32, DWPS_LOOKBACK_K, false>(desc, tile, lane, st, ctr + 1);
            if (lane == 0) desc_publish(desc + tile, desc_word(ST_PREFIX, excl + count));
        }
        if (lane == 0) {
            s_base = excl;
            if (tile == num_tiles - 1) *num_selected = (uint64_t)(excl + count);
        }
    }
    __syncthreads();
    const uint32_t base = s_base + wave_prefix;
#pragma unroll
    for (int r = 0; r < R; ++r)
        if (keep[r]) out[base + step_prefix[r] + rank[r]] = rec[r];
}

__global__ void write_count_zero(uint64_t *p) { *p = 0ull; }

constexpr int kCompactNT = 256;

template <class Rec, int R>
ps_status launch_compact(void *ws, size_t *ws_bytes, const void *records, const uint8_t *flags, uint64_t n,
                         void *out, uint64_t *num_selected, hipStream_t s) {
    constexpr uint32_t TILE = kCompactNT * R;
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
    if (!aligned(records, sizeof(Rec)) || !aligned(out, sizeof(Rec))) return PS_ERR_ALIGNMENT;
    const size_t bytes = n * sizeof(Rec);
    if (ranges_overlap(out, bytes, records, bytes) || ranges_overlap(out, bytes, flags, n) ||
        ranges_overlap(num_selected, 8, out, bytes))
        return PS_ERR_ALIAS;
    if (launch_clear(ws, ws_bytes_for_tiles(tiles), s) != hipSuccess) return PS_ERR_HIP;
    timing_begin(s);
    hipLaunchKernelGGL((compact_kernel<Rec, kCompactNT, R>), dim3((unsigned)tiles), dim3(kCompactNT), 0, s,
                       static_cast<const Rec *>(records), flags, (uint32_t)n, static_cast<Rec *>(out),
                       num_selected, (uint32_t)tiles, ws_counter(ws), ws_desc(ws));
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
    case 4: return launch_compact<uint32_t, 16>(ws, ws_bytes, records, flags, n, out, num_selected, s);
    case 8: return launch_compact<uint2, 16>(ws, ws_bytes, records, flags, n, out, num_selected, s);
    case 16: return launch_compact<uint4, 8>(ws, ws_bytes, records, flags, n, out, num_selected, s);
    default: return PS_ERR_UNSUPPORTED;
    }
}
