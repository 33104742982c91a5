// twolevel.hpp -- the two-level (reduce-then-scan) device-wide scan in three
// launches ("Single-Pass Prefix Scan with Decoupled Look-Back", sections on
// the two-level form and "When not to use it"; "Parallel Prefix Sum (Scan),
// in depth", section "Scanning a whole array: three grid strategies"):
//   pass 1  every workgroup folds one tile and writes the tile's total;
//   pass 2  one workgroup scans the tile totals in place (exclusive) and
//           writes the fold of everything;
//   pass 3  every workgroup scans its tile again and adds the tile's prefix.
// Up to 1024 tiles, pass 3 folds the earlier tile totals itself and pass 2
// is dropped; a single tile is pass 3 alone.  The input is read twice (12 bytes of traffic per 32-bit element against
// the chained scan's 8), but there are no descriptors, no look-back and no
// workspace clear, and each pass is one short wave of workgroups.  It serves
// small inputs, where the persistent chained pipeline's fixed latency (a tile
// passes through several phases, each waiting on a load) outweighs the
// second read, and it is the baseline the single-pass scan is measured
// against.
#pragma once

#include <hip/hip_runtime.h>

#include "dwps_device.hpp"
#include "host_common.hpp"
#include "pipeline.hpp"
#include "tile_io.hpp"

namespace dwps {

// Passes 1 and 3: 4 waves x 4 groups of four elements per lane = 4096
// elements per tile; a wave owns 1024 consecutive elements.
constexpr int kTlWaves = 4;
constexpr int kTlQ = 4;
constexpr uint32_t kTlTile = (uint32_t)kTlWaves * kTlQ * 256u;
// Pass 2: one workgroup of 16 waves, four tile totals per lane per round.
constexpr int kTlScanWaves = 16;
constexpr uint32_t kTlScanChunk = (uint32_t)kTlScanWaves * 64u * 4u;

// Tile totals live in the descriptor area of the workspace (after its
// header, which they leave alone), one 64-bit word per 32 payload bits with
// the upper half zero: every word reads as an unpublished descriptor, so a
// later single-pass call on the same workspace never mistakes a total for
// a published tile.
template <class T>
__device__ __forceinline__ T tl_get(const uint64_t *w, uint32_t i) {
    if constexpr (sizeof(T) == 8)
        return from_bits64<T>(((uint64_t)(uint32_t)w[2u * i + 1u] << 32) | (uint32_t)w[2u * i]);
    else
        return from_bits<T>((uint32_t)w[i]);
}
template <class T>
__device__ __forceinline__ void tl_put(uint64_t *w, uint32_t i, T v) {
    if constexpr (sizeof(T) == 8) {
        const uint64_t b = to_bits64(v);
        w[2u * i] = (uint32_t)b;
        w[2u * i + 1u] = (uint32_t)(b >> 32);
    } else {
        w[i] = to_bits(v);
    }
}

template <class Op, bool VEC>
__global__ __launch_bounds__(kTlWaves * 64) void tl_reduce_kernel(typename IoOf<Op>::Src in, uint32_t n,
                                                                 uint64_t *sums) {
    using T = typename Op::T;
    __shared__ T wt[kTlWaves];
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t w = uniform(threadIdx.x >> 6);
    const uint64_t base = (uint64_t)blockIdx.x * kTlTile;
    const uint64_t span = base + (uint64_t)w * kTlQ * 256u + 4u * lane;
    const bool full = base + kTlTile <= n;
    WaveSpan<Op, kTlQ> s;
    s.template load<VEC>(in, span, n, full, true);
    s.pad(span, n, full);
    T lane_excl[kTlQ], row_prefix[kTlQ];
    const T tot = scan_span<Op, kTlQ>(s, lane_excl, row_prefix);  // rows folded in element order
    if (lane == 0) wt[w] = tot;
    __syncthreads();
    if (threadIdx.x == 0) {
        T acc = Op::id();
#pragma unroll
        for (int k = 0; k < kTlWaves; ++k) acc = Op::op(acc, wt[k]);
        tl_put<T>(sums, blockIdx.x, acc);
    }
}

// Exclusive scan of `num` tile totals in place; *total (optional) gets the
// fold of all of them.  Thread t holds totals 4t .. 4t+3 of each round.
template <class Op>
__global__ __launch_bounds__(kTlScanWaves * 64) void tl_scan_sums_kernel(uint64_t *sums, uint32_t num,
                                                                        typename Op::T *total) {
    using T = typename Op::T;
    __shared__ T wt[kTlScanWaves];
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t w = uniform(threadIdx.x >> 6);
    T carry = Op::id();
    for (uint32_t c = 0; c < num; c += kTlScanChunk) {
        T v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t i = c + 4u * threadIdx.x + (uint32_t)k;
            v[k] = i < num ? tl_get<T>(sums, i) : Op::id();
        }
        T inc[4];
        inc[0] = v[0];
#pragma unroll
        for (int k = 1; k < 4; ++k) inc[k] = Op::op(inc[k - 1], v[k]);
        const T winc = wave_inclusive<Op>(inc[3]);
        const T lex = wave_shift_right<Op>(winc);
        if (lane == 63) wt[w] = winc;
        __syncthreads();
        T wp = carry, all = carry;
#pragma unroll
        for (int k = 0; k < kTlScanWaves; ++k) {
            if ((uint32_t)k < w) wp = Op::op(wp, wt[k]);
            all = Op::op(all, wt[k]);
        }
        const T c0 = Op::op(wp, lex);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t i = c + 4u * threadIdx.x + (uint32_t)k;
            if (i < num) tl_put<T>(sums, i, k == 0 ? c0 : Op::op(c0, inc[k - 1]));
        }
        carry = all;
        __syncthreads();  // wt is rewritten by the next round
    }
    if (threadIdx.x == 0 && total) *total = carry;
}

// Where pass 3 takes its tile's prefix from.
enum TlPrefix {
    kTlFromScan = 0,  // the exclusive scan of the totals left by pass 2
    kTlFold = 1,      // folds the totals of the tiles before it itself (no pass 2)
    kTlAlone = 2,     // the only tile: no prefix, and it writes the total
};
// Tile counts up to which pass 3 folds the earlier totals itself: at most
// kTlFoldMax / 64 reads per lane of one wave, all issued at once.
constexpr uint32_t kTlFoldMax = 1024;

// Fold of totals[0 .. t) in index order by one wave: lane l folds a
// contiguous run of them, the wave scan joins the runs.
template <class Op>
__device__ __forceinline__ typename Op::T fold_before(const uint64_t *totals, uint32_t t, uint32_t lane) {
    using T = typename Op::T;
    constexpr uint32_t PER = kTlFoldMax / 64u;
    const uint32_t per = (t + 63u) / 64u;  // <= PER
    T v = Op::id();
#pragma unroll
    for (uint32_t k = 0; k < PER; ++k) {
        const uint32_t i = lane * per + k;
        const bool in = k < per && i < t;
        const T x = tl_get<T>(totals, in ? i : 0u);
        v = in ? Op::op(v, x) : v;
    }
    return read_lane(wave_inclusive<Op>(v), 63);
}

template <class Op, bool INCL, bool VEC, int PREFIX>
__global__ __launch_bounds__(kTlWaves * 64) void tl_scan_kernel(typename IoOf<Op>::Src in,
                                                               typename IoOf<Op>::Dst out, uint32_t n,
                                                               const uint64_t *sums, typename Op::T *total) {
    using T = typename Op::T;
    __shared__ T wt[kTlWaves];
    __shared__ T tile_prefix_sh;
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t w = uniform(threadIdx.x >> 6);
    const uint64_t base = (uint64_t)blockIdx.x * kTlTile;
    const uint64_t span = base + (uint64_t)w * kTlQ * 256u + 4u * lane;
    const bool full = base + kTlTile <= n;
    WaveSpan<Op, kTlQ> s;
    s.template load<VEC>(in, span, n, full, true);
    if (PREFIX == kTlFold && w == 0) {
        const T p = fold_before<Op>(sums, blockIdx.x, lane);
        if (lane == 0) tile_prefix_sh = p;
    }
    s.pad(span, n, full);
    T lane_excl[kTlQ], row_prefix[kTlQ];
    const T tot = scan_span<Op, kTlQ>(s, lane_excl, row_prefix);
    if (lane == 0) wt[w] = tot;
    __syncthreads();
    T tile_prefix = Op::id();
    if (PREFIX == kTlFromScan) tile_prefix = tl_get<T>(sums, blockIdx.x);
    if (PREFIX == kTlFold) tile_prefix = tile_prefix_sh;
    if (PREFIX != kTlFromScan && total && threadIdx.x == 0 && blockIdx.x == gridDim.x - 1) {
        T all = tile_prefix;
#pragma unroll
        for (int k = 0; k < kTlWaves; ++k) all = Op::op(all, wt[k]);
        *total = all;
    }
    T wave_prefix = tile_prefix;
#pragma unroll
    for (int k = 0; k < kTlWaves; ++k)
        if ((uint32_t)k < w) wave_prefix = Op::op(wave_prefix, wt[k]);
    finalize_span<Op, kTlQ, INCL>(s, lane_excl, row_prefix, wave_prefix);
#pragma unroll
    for (int q = 0; q < kTlQ; ++q) {
        const uint64_t g = span + (uint64_t)q * 256u;
        if constexpr (std::is_same<typename IoOf<Op>::Dst, PlanesOut>::value) {
            v4u wa, wb;
            split_planes(s.v[q], wa, wb);
            store_planes(out, g, wa, wb, VEC && full, n);
        } else if (VEC && full) {
            store_group(out, g, s.v[q]);
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                if (g + k < n) store_elem(out, g + k, s.v[q][k]);
        }
    }
}

template <class T>
__global__ void tl_write_one(T *p, T v) {
    *p = v;
}

inline uint64_t tl_tiles(uint64_t n) { return ceil_div(n, kTlTile); }

template <class Op>
inline size_t tl_ws_bytes(uint64_t n) {
    return kWsHeader + round_up(tl_tiles(n) * sizeof(typename Op::T) * 2u, 256);
}

// The passes on validated arguments (n > 0); `sums` is the workspace.  One
// tile: pass 3 alone (one launch).  Up to kTlFoldMax tiles: pass 1, then
// pass 3 folding the earlier totals itself (two launches).  More: all three.
// The workspace needs no preparation for this form.
template <class Op, int PREFIX>
void tl_third(typename IoOf<Op>::Src in, typename IoOf<Op>::Dst out, uint32_t n, uint64_t *sums,
              typename Op::T *total, uint32_t tiles, bool inclusive, bool vec, hipStream_t s) {
    const dim3 grid(tiles), block(kTlWaves * 64);
    if (inclusive && vec)
        hipLaunchKernelGGL((tl_scan_kernel<Op, true, true, PREFIX>), grid, block, 0, s, in, out, n, sums, total);
    else if (inclusive)
        hipLaunchKernelGGL((tl_scan_kernel<Op, true, false, PREFIX>), grid, block, 0, s, in, out, n, sums, total);
    else if (vec)
        hipLaunchKernelGGL((tl_scan_kernel<Op, false, true, PREFIX>), grid, block, 0, s, in, out, n, sums, total);
    else
        hipLaunchKernelGGL((tl_scan_kernel<Op, false, false, PREFIX>), grid, block, 0, s, in, out, n, sums, total);
}

template <class Op>
ps_status tl_launch(void *ws, typename IoOf<Op>::Src in, typename IoOf<Op>::Dst out, uint32_t n,
                    typename Op::T *total, bool inclusive, bool vec, hipStream_t s) {
    uint64_t *sums = ws_desc(ws);
    const uint32_t tiles = (uint32_t)tl_tiles(n);
    timing_begin(s);
    if (tiles == 1) {
        tl_third<Op, kTlAlone>(in, out, n, sums, total, tiles, inclusive, vec, s);
    } else {
        if (vec)
            hipLaunchKernelGGL((tl_reduce_kernel<Op, true>), dim3(tiles), dim3(kTlWaves * 64), 0, s, in, n, sums);
        else
            hipLaunchKernelGGL((tl_reduce_kernel<Op, false>), dim3(tiles), dim3(kTlWaves * 64), 0, s, in, n, sums);
        if (tiles <= kTlFoldMax) {
            tl_third<Op, kTlFold>(in, out, n, sums, total, tiles, inclusive, vec, s);
        } else {
            hipLaunchKernelGGL(tl_scan_sums_kernel<Op>, dim3(1), dim3(kTlScanWaves * 64), 0, s, sums, tiles,
                               total);
            tl_third<Op, kTlFromScan>(in, out, n, sums, total, tiles, inclusive, vec, s);
        }
    }
    timing_end(s);
    return launch_status();
}

}  // namespace dwps
