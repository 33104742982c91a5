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

#include <type_traits>

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

// Where a flat scan reads and writes: one array of elements, or, for the
// recurrence pairs, two float planes a[] and b[] (the layout in which
// callers keep the coefficients of a linear recurrence).  Outputs go to the
// planes of PlanesOut; its `a` may be null, then only the b plane (h[t] of
// the inclusive scan) is written.
struct PlanesIn {
    const float *a, *b;
};
struct PlanesOut {
    float *a, *b;
};
template <class Op, bool PLANES = std::is_same<typename Op::T, F2>::value>
struct IoOf {
    using Src = const typename InputOf<Op>::type *;
    using Dst = typename Op::T *;
};
template <class Op>
struct IoOf<Op, true> {
    using Src = PlanesIn;
    using Dst = PlanesOut;
};

// Four consecutive elements from a 16-byte aligned group (index g).
template <class T, class In>
__device__ __forceinline__ void load_group(const In *in, uint64_t g, T (&v)[4]) {
    static_assert(sizeof(In) == 4, "16-byte loads carry four input elements");
    const v4u r = load16(in + g);
    v[0] = (T)from_bits<In>(r.x);
    v[1] = (T)from_bits<In>(r.y);
    v[2] = (T)from_bits<In>(r.z);
    v[3] = (T)from_bits<In>(r.w);
}
// Four keep flags: one 4-byte load (a group never leaves the 4-byte word
// that holds its first flag).
template <class T>
__device__ __forceinline__ void load_group(const Flag8 *in, uint64_t g, T (&v)[4]) {
    const uint32_t w = *reinterpret_cast<const uint32_t *>(in + g);
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = ((w >> (8 * k)) & 0xFFu) != 0u ? T(1) : T(0);
}
__device__ __forceinline__ void load_group(PlanesIn in, uint64_t g, F2 (&v)[4]) {
    const v4u ra = load16(in.a + g), rb = load16(in.b + g);
    v[0] = F2{__uint_as_float(ra.x), __uint_as_float(rb.x)};
    v[1] = F2{__uint_as_float(ra.y), __uint_as_float(rb.y)};
    v[2] = F2{__uint_as_float(ra.z), __uint_as_float(rb.z)};
    v[3] = F2{__uint_as_float(ra.w), __uint_as_float(rb.w)};
}
template <class T, class In>
__device__ __forceinline__ T load_elem(const In *in, uint64_t i) {
    return (T)in[i];
}
template <class T>
__device__ __forceinline__ T load_elem(PlanesIn in, uint64_t i) {
    return T{in.a[i], in.b[i]};
}

// Register state of one wave's span of a tile.
template <class Op, int Q>
struct WaveSpan {
    using T = typename Op::T;
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
    template <bool VEC, class Src>
    __device__ __forceinline__ void load(Src in, uint64_t span, uint32_t n, bool full, bool valid) {
        if (VEC) {
            const uint64_t last_group = ((uint64_t)n - 1u) & ~(uint64_t)3u;
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                uint64_t g = span + (uint64_t)q * 256u;
                if (!full) g = g < last_group ? g : last_group;
                if (!valid) g = 0;
                load_group(in, g, v[q]);
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
                    v[q][k] = load_elem<T>(in, i);
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
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint64_t e0 = to_bits64(o[2 * h]), e1 = to_bits64(o[2 * h + 1]);
            w[h].x = (uint32_t)e0;
            w[h].y = (uint32_t)(e0 >> 32);
            w[h].z = (uint32_t)e1;
            w[h].w = (uint32_t)(e1 >> 32);
        }
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
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            o[2 * h] = from_bits64<T>(((uint64_t)w[h].y << 32) | w[h].x);
            o[2 * h + 1] = from_bits64<T>(((uint64_t)w[h].w << 32) | w[h].z);
        }
    } else {
        o[0] = from_bits<T>(w[0].x);
        o[1] = from_bits<T>(w[0].y);
        o[2] = from_bits<T>(w[0].z);
        o[3] = from_bits<T>(w[0].w);
    }
}

// Four consecutive outputs to a 16-byte aligned group (index g), and one.
template <class T>
__device__ __forceinline__ void store_group(T *out, uint64_t g, const T (&o)[4]) {
    constexpr int PW = (int)sizeof(T) / 4;  // 16-byte vectors per group of four
    v4u w[PW];
    pack16<T>(o, w);
#pragma unroll
    for (int h = 0; h < PW; ++h) store16(out + g + 4 / PW * h, w[h]);
}
// Four consecutive pairs, already split into their planes (registers, not
// an array of pairs: one regrouped after a branch ends up in per-lane
// scratch memory, and waiting for a scratch load also waits for every load
// issued before it -- the next tile's, which the pipeline keeps in flight):
// 16-byte vectors when `whole`, else the elements below n.
__device__ __forceinline__ void store_planes(PlanesOut out, uint64_t g, v4u wa, v4u wb, bool whole, uint32_t n) {
    if (whole) {
        if (out.a) store16(out.a + g, wa);
        store16(out.b + g, wb);
        return;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        if (g + k < n) {
            if (out.a) out.a[g + k] = __uint_as_float(wa[k]);
            out.b[g + k] = __uint_as_float(wb[k]);
        }
    }
}
// A group of pairs split into the planes' vectors.
__device__ __forceinline__ void split_planes(const F2 (&o)[4], v4u &wa, v4u &wb) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        wa[k] = __float_as_uint(o[k].a);
        wb[k] = __float_as_uint(o[k].b);
    }
}
template <class T>
__device__ __forceinline__ void store_elem(T *out, uint64_t i, T v) {
    out[i] = v;
}

// Store a finalized span: out = prefix (+) v.
template <class Op, int Q, bool VEC, class Dst>
__device__ __forceinline__ void store_final(const WaveSpan<Op, Q> &s, typename Op::T prefix, Dst out,
                                            uint64_t span, uint32_t n, bool full) {
    using T = typename Op::T;
    if constexpr (std::is_same<Dst, PlanesOut>::value) {
        // the pairs split into their planes as they are computed (store_planes)
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            v4u wa, wb;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const F2 o = Op::op(prefix, s.v[q][k]);
                wa[k] = __float_as_uint(o.a);
                wb[k] = __float_as_uint(o.b);
            }
            store_planes(out, span + (uint64_t)q * 256u, wa, wb, VEC && full, n);
        }
    } else {
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            T o[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) o[k] = Op::op(prefix, s.v[q][k]);
            if (VEC && full) {
                store_group(out, span + (uint64_t)q * 256u, o);
            } else {
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const uint64_t i = span + (uint64_t)q * 256u + k;
                    if (i < n) store_elem(out, i, o[k]);
                }
            }
        }
    }
}

}  // namespace dwps
