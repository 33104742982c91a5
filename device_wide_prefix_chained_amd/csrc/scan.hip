// scan.hip -- flat device-wide scan: single pass, chained scan with decoupled
// look-back ("Single-Pass Prefix Scan with Decoupled Look-Back"; "Parallel
// Prefix Sum (Scan), in depth", section "Scanning a whole array: three grid
// strategies").
//
// One workgroup of NT threads scans one tile of NT * Q * 4 elements.
//   1. Ticket: thread 0 takes the tile index from an atomic counter, so every
//      tile it may wait on was handed out earlier and is already resident or
//      finished (blockIdx order is not a dispatch guarantee).
//   2. Load: wave w of the tile owns Q * 256 consecutive elements; load q of
//      lane l is the 16-byte group at element q*256 + 4*l of that span, so each
//      wave-wide load instruction reads 1 KiB of contiguous memory.
//   3. Thread-serial inclusive scan of each group of four, wave64 DPP scan of
//      the Q group totals, LDS scan of the NT/64 wave totals -> the tile
//      aggregate.
//   4. Wave 0 publishes the aggregate (tile 0: its inclusive prefix), looks
//      back over the predecessors' descriptors, publishes the tile's inclusive
//      prefix, and hands the exclusive prefix to the other waves through LDS.
//   5. Every lane combines tile prefix (+) wave prefix (+) group prefix (+)
//      lane prefix (+) its element prefix and stores 16 bytes per group.
#include <hip/hip_runtime.h>

#include "dwps_device.hpp"
#include "host_common.hpp"

namespace dwps {

template <class Op, int NT, int Q, bool INCL, bool VEC, bool STATS>
__global__ __launch_bounds__(NT) void scan_kernel(const typename Op::T *in, typename Op::T *out,
                                                  uint32_t n, uint32_t num_tiles, uint32_t *ctr,
                                                  uint64_t *desc, typename Op::T *total,
                                                  uint32_t *stats, int aggregate_only) {
    using T = typename Op::T;
    constexpr int NW = NT / 64;
    constexpr uint32_t WAVE_ELEMS = (uint32_t)Q * 256u;
    constexpr uint32_t TILE = (uint32_t)NT * (uint32_t)Q * 4u;

    __shared__ uint32_t s_tile;
    __shared__ T s_wave[NW];
    __shared__ T s_prefix;

    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & 63u;
    const uint32_t wave = tid >> 6;

    if (tid == 0) s_tile = take_ticket(ctr);
    __syncthreads();
    const uint32_t tile = s_tile;
    const uint64_t tile_base = (uint64_t)tile * TILE;
    const uint64_t span = tile_base + (uint64_t)wave * WAVE_ELEMS + 4u * lane;
    const bool full = tile_base + TILE <= (uint64_t)n;

    // ---- 2. load -----------------------------------------------------------
    T v[Q][4];
    if (VEC && full) {
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const uint4 r = *reinterpret_cast<const uint4 *>(in + span + (uint64_t)q * 256u);
            v[q][0] = from_bits<T>(r.x);
            v[q][1] = from_bits<T>(r.y);
            v[q][2] = from_bits<T>(r.z);
            v[q][3] = from_bits<T>(r.w);
        }
    } else {
#pragma unroll
        for (int q = 0; q < Q; ++q)
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint64_t i = span + (uint64_t)q * 256u + k;
                v[q][k] = (i < n) ? in[i] : Op::id();
            }
    }

    // ---- 3. thread-serial, wave and block scans ---------------------------------
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        v[q][1] = Op::op(v[q][0], v[q][1]);
        v[q][2] = Op::op(v[q][1], v[q][2]);
        v[q][3] = Op::op(v[q][2], v[q][3]);
    }
    T lane_excl[Q];
    T group_prefix[Q];
    T run = Op::id();
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const T inc = wave_inclusive<Op>(v[q][3]);
        lane_excl[q] = wave_shift_right<Op>(inc);
        group_prefix[q] = run;
        run = Op::op(run, read_lane(inc, 63));
    }
    if (lane == 0) s_wave[wave] = run;
    __syncthreads();
    T wave_prefix = Op::id();
    T agg = Op::id();
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const T t = s_wave[w];
        if ((uint32_t)w < wave) wave_prefix = Op::op(wave_prefix, t);
        agg = Op::op(agg, t);
    }

    // ---- 4. publish, look back, publish -------------------------------------
    if (wave == 0) {
        LookbackStats st;
        uint64_t t0 = 0;
        if (STATS) t0 = __builtin_amdgcn_s_memrealtime();
        T excl = Op::id();
        if (tile == 0) {
            if (lane == 0) desc_publish(desc, desc_word(ST_PREFIX, to_bits(agg)));
        } else {
            if (lane == 0) desc_publish(desc + tile, desc_word(ST_AGGREGATE, to_bits(agg)));
            excl = lookback<Op, STATS>(desc, tile, lane, st, ctr + 1);
            // (diagnostic build only: aggregate_only keeps every later tile in
            // AGGREGATE state so that each look-back walks back to tile 0)
            if (lane == 0 && !(STATS && aggregate_only))
                desc_publish(desc + tile, desc_word(ST_PREFIX, to_bits(Op::op(excl, agg))));
        }
        if (lane == 0) {
            s_prefix = excl;
            if (total && tile == num_tiles - 1) *total = Op::op(excl, agg);
            if (STATS) {
                const uint64_t t1 = __builtin_amdgcn_s_memrealtime();
                uint4 rec = make_uint4(st.polls, st.windows, (uint32_t)(t1 - t0), st.stalls);
                reinterpret_cast<uint4 *>(stats)[tile] = rec;
            }
        }
    }
    __syncthreads();

    // ---- 5. combine and store -------------------------------------------------
    const T base = Op::op(s_prefix, wave_prefix);
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const T c = Op::op(Op::op(base, group_prefix[q]), lane_excl[q]);
        T o[4];
        if (INCL) {
            o[0] = Op::op(c, v[q][0]);
            o[1] = Op::op(c, v[q][1]);
            o[2] = Op::op(c, v[q][2]);
            o[3] = Op::op(c, v[q][3]);
        } else {
            o[0] = c;
            o[1] = Op::op(c, v[q][0]);
            o[2] = Op::op(c, v[q][1]);
            o[3] = Op::op(c, v[q][2]);
        }
        if (VEC && full) {
            *reinterpret_cast<uint4 *>(out + span + (uint64_t)q * 256u) =
                make_uint4(to_bits(o[0]), to_bits(o[1]), to_bits(o[2]), to_bits(o[3]));
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint64_t i = span + (uint64_t)q * 256u + k;
                if (i < n) out[i] = o[k];
            }
        }
    }
}

template <class T>
__global__ void write_one(T *p, T v) {
    *p = v;
}

// Flat scan tile shape: 256 threads (4 waves) x 16 elements.
constexpr int kFlatNT = 256;
constexpr int kFlatQ = 4;
constexpr uint32_t kFlatTile = kFlatNT * kFlatQ * 4;

inline uint64_t flat_tiles(uint64_t n) { return ceil_div(n, kFlatTile); }

template <class Op, bool STATS>
ps_status launch_flat(void *ws, size_t *ws_bytes, const void *in_v, void *out_v, uint64_t n, void *total_v,
                      bool inclusive, uint32_t *stats, hipStream_t s, typename Op::T identity,
                      int aggregate_only = 0) {
    using T = typename Op::T;
    if (n >= (1ull << 32)) return PS_ERR_SIZE;
    const uint64_t tiles = flat_tiles(n);
    bool query = false;
    ps_status st = workspace_protocol(ws, ws_bytes, ws_bytes_for_tiles(tiles), &query);
    if (st != PS_OK || query) return st;
    const T *in = static_cast<const T *>(in_v);
    T *out = static_cast<T *>(out_v);
    T *total = static_cast<T *>(total_v);
    if (n == 0) {
        if (!total) return PS_OK;
        if (!aligned(total, 4)) return PS_ERR_ALIGNMENT;
        hipLaunchKernelGGL(write_one<T>, dim3(1), dim3(1), 0, s, total, identity);
        return launch_status();
    }
    if (!in || !out) return PS_ERR_NULL;
    if (STATS && !stats) return PS_ERR_NULL;
    if (!aligned(in, 4) || !aligned(out, 4) || (total && !aligned(total, 4))) return PS_ERR_ALIGNMENT;
    if (in != (const void *)out && ranges_overlap(in, n * 4, out, n * 4)) return PS_ERR_ALIAS;
    if (launch_clear(ws, ws_bytes_for_tiles(tiles), s) != hipSuccess) return PS_ERR_HIP;
    const bool vec = aligned(in, 16) && aligned(out, 16);
    const dim3 grid((unsigned)tiles), block(kFlatNT);
    uint32_t *ctr = ws_counter(ws);
    uint64_t *desc = ws_desc(ws);
    const uint32_t n32 = (uint32_t)n, nt = (uint32_t)tiles;
    timing_begin(s);
    if (inclusive) {
        if (vec)
            hipLaunchKernelGGL((scan_kernel<Op, kFlatNT, kFlatQ, true, true, STATS>), grid, block, 0, s, in, out,
                               n32, nt, ctr, desc, total, stats, aggregate_only);
        else
            hipLaunchKernelGGL((scan_kernel<Op, kFlatNT, kFlatQ, true, false, STATS>), grid, block, 0, s, in, out,
                               n32, nt, ctr, desc, total, stats, aggregate_only);
    } else {
        if (vec)
            hipLaunchKernelGGL((scan_kernel<Op, kFlatNT, kFlatQ, false, true, STATS>), grid, block, 0, s, in, out,
                               n32, nt, ctr, desc, total, stats, aggregate_only);
        else
            hipLaunchKernelGGL((scan_kernel<Op, kFlatNT, kFlatQ, false, false, STATS>), grid, block, 0, s, in,
                               out, n32, nt, ctr, desc, total, stats, aggregate_only);
    }
    timing_end(s);
    return launch_status();
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

extern "C" ps_status ps_scan(void *ws, size_t *ws_bytes, ps_op op, ps_dtype dtype, int inclusive, const void *in,
                             void *out, uint64_t n, void *total, void *stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool inc = inclusive != 0;
    if (dtype == PS_U32) {
        switch (op) {
        case PS_OP_SUM: return launch_flat<SumU32, false>(ws, ws_bytes, in, out, n, total, inc, nullptr, s, 0u);
        case PS_OP_MAX: return launch_flat<MaxU32, false>(ws, ws_bytes, in, out, n, total, inc, nullptr, s, 0u);
        case PS_OP_MIN:
            return launch_flat<MinU32, false>(ws, ws_bytes, in, out, n, total, inc, nullptr, s, 0xFFFFFFFFu);
        case PS_OP_AND:
            return launch_flat<AndU32, false>(ws, ws_bytes, in, out, n, total, inc, nullptr, s, 0xFFFFFFFFu);
        case PS_OP_OR: return launch_flat<OrU32, false>(ws, ws_bytes, in, out, n, total, inc, nullptr, s, 0u);
        case PS_OP_XOR: return launch_flat<XorU32, false>(ws, ws_bytes, in, out, n, total, inc, nullptr, s, 0u);
        case PS_OP_AFFINE16:
            return launch_flat<Affine16, false>(ws, ws_bytes, in, out, n, total, inc, nullptr, s, 0x00010000u);
        }
        return PS_ERR_UNSUPPORTED;
    }
    if (dtype == PS_F32) {
        switch (op) {
        case PS_OP_SUM: return launch_flat<SumF32, false>(ws, ws_bytes, in, out, n, total, inc, nullptr, s, 0.0f);
        case PS_OP_MAX:
            return launch_flat<MaxF32, false>(ws, ws_bytes, in, out, n, total, inc, nullptr, s,
                                              -__builtin_huge_valf());
        case PS_OP_MIN:
            return launch_flat<MinF32, false>(ws, ws_bytes, in, out, n, total, inc, nullptr, s,
                                              __builtin_huge_valf());
        default: return PS_ERR_UNSUPPORTED;
        }
    }
    return PS_ERR_UNSUPPORTED;
}

extern "C" ps_status ps_lookback_stats_u32(void *ws, size_t *ws_bytes, const uint32_t *in, uint32_t *out,
                                           uint64_t n, uint32_t *stats, int aggregate_only, void *stream) {
    return launch_flat<SumU32, true>(ws, ws_bytes, in, out, n, nullptr, false, stats,
                                     static_cast<hipStream_t>(stream), 0u, aggregate_only);
}

extern "C" uint64_t ps_lookback_tiles(uint64_t n) { return flat_tiles(n); }

extern "C" uint32_t ps_tile_elements(ps_dtype dtype) {
    (void)dtype;
    return kFlatTile;
}
