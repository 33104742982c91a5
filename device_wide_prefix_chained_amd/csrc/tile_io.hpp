// tile_io.hpp -- the data-wave side of a tile: 16-byte loads and stores of a
// wave's span and the register-level scan of that span.
//
// A data wave owns Q * 256 consecutive elements of its tile.  Load q of lane l
// is the group of four elements at q*256 + 4*l of the span, so one wave-wide
// load or store instruction covers 1 KiB of contiguous memory.  The elements a
// lane holds are scanned serially in groups of four, the Q group totals of the
// wave by the DPP wave scan, and the wave total is handed to the block layer
// ("Parallel Prefix Sum (Scan), in depth", section "A CUDA scan: warp, block,
// grid": thread-serial work first, then the warp layer, then the block layer).
#pragma once

#include "dwps_device.hpp"

namespace dwps {

typedef unsigned int v4u __attribute__((ext_vector_type(4)));

// Streaming accesses are marked non-temporal: every input element is read
// once and every output element written once, so they should not displace
// the look-back descriptors from the caches.
#ifndef DWPS_NONTEMPORAL
#define DWPS_NONTEMPORAL 1
#endif

__device__ __forceinline__ v4u load16(const void *p) {
    const v4u *q = static_cast<const v4u *>(p);
    if (DWPS_NONTEMPORAL) return __builtin_nontemporal_load(q);
    return *q;
}
__device__ __forceinline__ void store16(void *p, v4u v) {
    v4u *q = static_cast<v4u *>(p);
    if (DWPS_NONTEMPORAL)
        __builtin_nontemporal_store(v, q);
    else
        *q = v;
}

// Register state of one wave's span of a tile.
template <class Op, int Q>
struct WaveSpan {
    using T = typename Op::T;
    using In = typename InputOf<Op>::type;  // 4-byte input elements, widened to T on load
    static_assert(sizeof(In) == 4, "16-byte loads carry four input elements");
    T v[Q][4];  // elements, then their lane-local inclusive prefixes

    // Issue the loads of the span starting at element `span` (= tile base +
    // wave offset + 4*lane).  The loads are the same straight-line
    // instructions for every tile -- no branch, no use of the loaded values --
    // so several tiles of loads can stay in flight across the pipeline:
    // addresses past the end are clamped to the last in-range group (a
    // 16-byte aligned group that starts below n never leaves the page that
    // holds element n-1), and !valid (no tile) reads the first group again.
    // pad() later replaces the elements at or past n by the identity.
    // VEC: 16-byte aligned input, one 16-byte load per group; otherwise one
    // 4-byte load per element.
    template <bool VEC>
    __device__ __forceinline__ void load(const In *in, uint64_t span, uint32_t n, bool full, bool valid) {
        if (VEC) {
            const uint64_t last_group = ((uint64_t)n - 1u) & ~(uint64_t)3u;
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                uint64_t g = span + (uint64_t)q * 256u;
                if (!full) g = g < last_group ? g : last_group;
                if (!valid) g = 0;
                const v4u r = load16(in + g);
                v[q][0] = (T)from_bits<In>(r.x);
                v[q][1] = (T)from_bits<In>(r.y);
                v[q][2] = (T)from_bits<In>(r.z);
                v[q][3] = (T)from_bits<In>(r.w);
            }
        } else {
            const uint64_t last = (uint64_t)n - 1u;
#pragma unroll
            for (int q = 0; q < Q; ++q)
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    uint64_t i = span + (uint64_t)q * 256u + k;
                    i = i < last ? i : last;
                    if (!valid) i = 0;
                    v[q][k] = (T)in[i];
                }
        }
    }

    // Identity padding of a partial tile ("Parallel Prefix Sum (Scan), in
    // depth", section "Failure modes": the pad must be the identity).
    __device__ __forceinline__ void pad(uint64_t span, uint32_t n, bool full) {
        if (full) return;
#pragma unroll
        for (int q = 0; q < Q; ++q)
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint64_t i = span + (uint64_t)q * 256u + k;
                v[q][k] = (i < n) ? v[q][k] : Op::id();
            }
    }
};

// Scan of a loaded span: lane-local inclusive prefixes in place, the lane's
// exclusive prefix within each group-row of the wave, the wave-uniform prefix
// of each group-row, and the wave total (returned).
template <class Op, int Q>
__device__ __forceinline__ typename Op::T scan_span(WaveSpan<Op, Q> &s, typename Op::T (&lane_excl)[Q],
                                                    typename Op::T (&row_prefix)[Q]) {
    using T = typename Op::T;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        s.v[q][1] = Op::op(s.v[q][0], s.v[q][1]);
        s.v[q][2] = Op::op(s.v[q][1], s.v[q][2]);
        s.v[q][3] = Op::op(s.v[q][2], s.v[q][3]);
    }
    T run = Op::id();
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const T inc = wave_inclusive<Op>(s.v[q][3]);
        lane_excl[q] = wave_shift_right<Op>(inc);
        row_prefix[q] = run;
        run = Op::op(run, read_lane(inc, 63));
    }
    return run;
}

// Turn a scanned span into its outputs relative to the tile start:
// wave prefix (+) row prefix (+) lane prefix (+) element prefix, in the
// inclusive or exclusive form.  Afterwards only the tile's exclusive prefix
// is missing: out = tile_prefix (+) v.
template <class Op, int Q, bool INCL>
__device__ __forceinline__ void finalize_span(WaveSpan<Op, Q> &s, const typename Op::T (&lane_excl)[Q],
                                              const typename Op::T (&row_prefix)[Q], typename Op::T wave_prefix) {
    using T = typename Op::T;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const T c = Op::op(Op::op(wave_prefix, row_prefix[q]), lane_excl[q]);
        if (INCL) {
            s.v[q][0] = Op::op(c, s.v[q][0]);
            s.v[q][1] = Op::op(c, s.v[q][1]);
            s.v[q][2] = Op::op(c, s.v[q][2]);
            s.v[q][3] = Op::op(c, s.v[q][3]);
        } else {
            s.v[q][3] = Op::op(c, s.v[q][2]);
            s.v[q][2] = Op::op(c, s.v[q][1]);
            s.v[q][1] = Op::op(c, s.v[q][0]);
            s.v[q][0] = c;
        }
    }
}

// Four elements as 16-byte vectors: one for 4-byte T, two for 8-byte T.
template <class T>
__device__ __forceinline__ void pack16(const T (&o)[4], v4u (&w)[sizeof(T) / 4]) {
    if constexpr (sizeof(T) == 8) {
        w[0].x = (uint32_t)o[0];
        w[0].y = (uint32_t)(o[0] >> 32);
        w[0].z = (uint32_t)o[1];
        w[0].w = (uint32_t)(o[1] >> 32);
        w[1].x = (uint32_t)o[2];
        w[1].y = (uint32_t)(o[2] >> 32);
        w[1].z = (uint32_t)o[3];
        w[1].w = (uint32_t)(o[3] >> 32);
    } else {
        w[0].x = to_bits(o[0]);
        w[0].y = to_bits(o[1]);
        w[0].z = to_bits(o[2]);
        w[0].w = to_bits(o[3]);
    }
}
template <class T>
__device__ __forceinline__ void unpack16(const v4u (&w)[sizeof(T) / 4], T (&o)[4]) {
    if constexpr (sizeof(T) == 8) {
        o[0] = (T)(((uint64_t)w[0].y << 32) | w[0].x);
        o[1] = (T)(((uint64_t)w[0].w << 32) | w[0].z);
        o[2] = (T)(((uint64_t)w[1].y << 32) | w[1].x);
        o[3] = (T)(((uint64_t)w[1].w << 32) | w[1].z);
    } else {
        o[0] = from_bits<T>(w[0].x);
        o[1] = from_bits<T>(w[0].y);
        o[2] = from_bits<T>(w[0].z);
        o[3] = from_bits<T>(w[0].w);
    }
}

// Store a finalized span: out = prefix (+) v.
template <class Op, int Q, bool VEC>
__device__ __forceinline__ void store_final(const WaveSpan<Op, Q> &s, typename Op::T prefix, typename Op::T *out,
                                            uint64_t span, uint32_t n, bool full) {
    using T = typename Op::T;
    constexpr int PW = (int)sizeof(T) / 4;  // 16-byte vectors per group of four
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        T o[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) o[k] = Op::op(prefix, s.v[q][k]);
        if (VEC && full) {
            v4u w[PW];
            pack16<T>(o, w);
#pragma unroll
            for (int h = 0; h < PW; ++h) store16(out + span + (uint64_t)q * 256u + 4 / PW * h, w[h]);
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint64_t i = span + (uint64_t)q * 256u + k;
                if (i < n) out[i] = o[k];
            }
        }
    }
}

}  // namespace dwps
