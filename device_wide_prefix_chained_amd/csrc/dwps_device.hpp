// dwps_device.hpp -- device building blocks of the chained scan for gfx950.
//
// Layers, bottom to top (the warp / block / grid composition of
// "Parallel Prefix Sum (Scan), in depth", section "A CUDA scan: warp, block,
// grid", and "Prefix scans and compaction", section "Warp, block, and grid
// composition"), re-built for 64-lane CDNA4 wavefronts:
//   * thread-serial fold of the elements a lane holds in registers;
//   * wave64 Hillis-Steele scan with DPP row shifts and row broadcasts (no
//     LDS traffic, no barrier: the 64 lanes execute in lockstep);
//   * block scan over the per-wave totals staged in LDS;
//   * grid level: per-tile 64-bit descriptors with the three states of
//     "Single-Pass Prefix Scan with Decoupled Look-Back", section "Three
//     states in a per-block descriptor", published and read as single
//     agent-scope atomic words (section "The publication protocol in code"),
//     with a look-back that reads 64 predecessors per poll, one per lane.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "ws_state.hpp"

namespace dwps {

// ---------------------------------------------------------------------------
// Operators: op(a, b) with a the EARLIER and b the LATER operand.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t to_bits(uint32_t v) { return v; }
__device__ __forceinline__ uint32_t to_bits(float v) { return __float_as_uint(v); }
template <class T> __device__ __forceinline__ T from_bits(uint32_t b);
template <> __device__ __forceinline__ uint32_t from_bits<uint32_t>(uint32_t b) { return b; }
template <> __device__ __forceinline__ float from_bits<float>(uint32_t b) { return __uint_as_float(b); }

// (a, b) of the map h -> a h + b, the element of the linear recurrence.
struct F2 {
    float a, b;
};

// 64-bit values as bits, for moving them in two 32-bit halves (DPP, lane
// reads, two-word descriptors).
__device__ __forceinline__ uint64_t to_bits64(uint64_t v) { return v; }
__device__ __forceinline__ uint64_t to_bits64(F2 v) {
    return ((uint64_t)__float_as_uint(v.b) << 32) | (uint64_t)__float_as_uint(v.a);
}
template <class T> __device__ __forceinline__ T from_bits64(uint64_t b);
template <> __device__ __forceinline__ uint64_t from_bits64<uint64_t>(uint64_t b) { return b; }
template <> __device__ __forceinline__ F2 from_bits64<F2>(uint64_t b) {
    return F2{__uint_as_float((uint32_t)b), __uint_as_float((uint32_t)(b >> 32))};
}

struct SumU32 {
    using T = uint32_t;
    __device__ static T id() { return 0u; }
    __device__ static T op(T a, T b) { return a + b; }
};
struct MaxU32 {
    using T = uint32_t;
    __device__ static T id() { return 0u; }
    __device__ static T op(T a, T b) { return (b > a) ? b : a; }
};
struct MinU32 {
    using T = uint32_t;
    __device__ static T id() { return 0xFFFFFFFFu; }
    __device__ static T op(T a, T b) { return (b < a) ? b : a; }
};
struct AndU32 {
    using T = uint32_t;
    __device__ static T id() { return 0xFFFFFFFFu; }
    __device__ static T op(T a, T b) { return a & b; }
};
struct OrU32 {
    using T = uint32_t;
    __device__ static T id() { return 0u; }
    __device__ static T op(T a, T b) { return a | b; }
};
struct XorU32 {
    using T = uint32_t;
    __device__ static T id() { return 0u; }
    __device__ static T op(T a, T b) { return a ^ b; }
};
// h -> a*h + b over Z/2^16, packed (a << 16) | b; a first, then b:
// h -> a_b*(a_a*h + b_a) + b_b.
struct Affine16 {
    using T = uint32_t;
    __device__ static T id() { return 0x00010000u; }
    __device__ static T op(T x, T y) {
        const uint32_t xa = x >> 16, xb = x & 0xFFFFu;
        const uint32_t ya = y >> 16, yb = y & 0xFFFFu;
        return (((xa * ya) & 0xFFFFu) << 16) | ((ya * xb + yb) & 0xFFFFu);
    }
};
// Widening sum: uint32 inputs, uint64 running sums (no wrap below 2^64).
struct SumU32toU64 {
    using T = uint64_t;
    using In = uint32_t;
    __device__ static T id() { return 0ull; }
    __device__ static T op(T a, T b) { return a + b; }
};
struct SumF32 {
    using T = float;
    __device__ static T id() { return 0.0f; }
    __device__ static T op(T a, T b) { return a + b; }
};
struct MaxF32 {
    using T = float;
    __device__ static T id() { return -__builtin_huge_valf(); }
    __device__ static T op(T a, T b) { return (b > a) ? b : a; }
};
struct MinF32 {
    using T = float;
    __device__ static T id() { return __builtin_huge_valf(); }
    __device__ static T op(T a, T b) { return (b < a) ? b : a; }
};

// Linear recurrence h[t] = a[t] h[t-1] + b[t] in fp32 ("Parallel Prefix Sum
// (Scan), in depth", section "What scan builds"): x first, then y, is
// h -> y.a (x.a h + x.b) + y.b, i.e. (x.a y.a, y.a x.b + y.b).  Associative
// (up to rounding), not commutative.  The identity (1, 0) is exact on
// either side, so identity padding changes no bit.
struct LinRecF32 {
    using T = F2;
    __device__ static T id() { return F2{1.0f, 0.0f}; }
    __device__ static T op(T x, T y) { return F2{x.a * y.a, __builtin_fmaf(y.a, x.b, y.b)}; }
};

// A keep flag of a compaction: one byte, nonzero = keep; it converts to 1
// or 0 ("Prefix scans and compaction", "Scan as an index generator").
struct Flag8 {
    uint8_t v;
    __device__ explicit operator uint32_t() const { return v != 0 ? 1u : 0u; }
};
// Count of kept flags before each position: the offsets of a staged
// compaction.
struct CountFlags {
    using T = uint32_t;
    using In = Flag8;
    __device__ static T id() { return 0u; }
    __device__ static T op(T a, T b) { return a + b; }
};

// Element type of an operator's input: Op::In when it widens, else Op::T.
template <class Op, class = void>
struct InputOf {
    using type = typename Op::T;
};
template <class Op>
struct InputOf<Op, decltype((void)sizeof(typename Op::In))> {
    using type = typename Op::In;
};

// ---------------------------------------------------------------------------
// Wave64 primitives (DPP).  DPP control codes of the GFX9 ISA:
//   0x111..0x11F row_shr:1..15   (within each row of 16 lanes)
//   0x138        wave_shr:1      (whole wave, lane i <- lane i-1)
//   0x142        row_bcast:15    (lane 15 of a row -> every lane of the next row)
//   0x143        row_bcast:31    (lane 31 -> rows 2 and 3)
// A lane whose source is outside the row/wave, or that row_mask disables,
// keeps `old`, which is always the operator's identity here.
// ---------------------------------------------------------------------------
// 64-bit values move as two 32-bit halves.
template <class Op, int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ typename Op::T dpp_from(typename Op::T x) {
    using T = typename Op::T;
    if constexpr (sizeof(T) == 8) {
        const uint64_t id = to_bits64(Op::id()), v = to_bits64(x);
        const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp((int)(uint32_t)id, (int)(uint32_t)v, CTRL,
                                                                  ROW_MASK, 0xF, false);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp((int)(uint32_t)(id >> 32),
                                                                  (int)(uint32_t)(v >> 32), CTRL, ROW_MASK, 0xF,
                                                                  false);
        return from_bits64<T>(((uint64_t)hi << 32) | lo);
    } else {
        return from_bits<T>((uint32_t)__builtin_amdgcn_update_dpp((int)to_bits(Op::id()), (int)to_bits(x), CTRL,
                                                                  ROW_MASK, 0xF, false));
    }
}

// Inclusive scan across the 64 lanes, lane order = element order.
template <class Op>
__device__ __forceinline__ typename Op::T wave_inclusive(typename Op::T x) {
    x = Op::op(dpp_from<Op, 0x111>(x), x);
    x = Op::op(dpp_from<Op, 0x112>(x), x);
    x = Op::op(dpp_from<Op, 0x114>(x), x);
    x = Op::op(dpp_from<Op, 0x118>(x), x);
    x = Op::op(dpp_from<Op, 0x142, 0xA>(x), x);
    x = Op::op(dpp_from<Op, 0x143, 0xC>(x), x);
    return x;
}

// Inclusive -> exclusive: lane i takes lane i-1's value, lane 0 the identity.
template <class Op>
__device__ __forceinline__ typename Op::T wave_shift_right(typename Op::T x) {
    return dpp_from<Op, 0x138>(x);
}

template <class T>
__device__ __forceinline__ T read_lane(T x, int lane) {
    if constexpr (sizeof(T) == 8) {
        const uint64_t v = to_bits64(x);
        const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, lane);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), lane);
        return from_bits64<T>(((uint64_t)hi << 32) | lo);
    } else {
        return from_bits<T>((uint32_t)__builtin_amdgcn_readlane((int)to_bits(x), lane));
    }
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }

// ---------------------------------------------------------------------------
// Tile descriptors: state word in the high 32 bits, payload in the low 32
// bits, so one atomic store publishes both and one atomic load reads a
// consistent pair.  Agent (device) scope: readers are on other XCDs of the
// same GPU, never on the host or a peer device.  The ordering that matters
// -- the tile's own LDS/register scan before its publication -- is program
// order within the publishing lane after a workgroup barrier, so relaxed
// ordering suffices; no other memory is handed over through a descriptor.
// State word: bits 1..0 the state, bits 10..2 the tag of the call that
// wrote it, bits 31..11 the distance of a PARTIAL (ws_state.hpp); a word
// carrying another call's tag reads as INVALID.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t desc_word(uint32_t state, uint32_t payload) {
    return ((uint64_t)state << 32) | (uint64_t)payload;
}
__device__ __forceinline__ void desc_publish(uint64_t *d, uint64_t w) {
    __hip_atomic_store(d, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t desc_poll(const uint64_t *d) {
    return __hip_atomic_load(d, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Install a descriptor computed by another tile's fallback: only over a
// word that the call with tag field tf sees as INVALID (zero, or left by
// another call), so a word the owner (or an earlier fallback) published in
// this call stays.
__device__ __forceinline__ bool desc_install(uint64_t *d, uint64_t w, uint32_t tf) {
    uint64_t seen = desc_poll(d);
    if (state_seen((uint32_t)(seen >> 32), tf) != ST_INVALID) return false;
    return __hip_atomic_compare_exchange_strong(d, &seen, w, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t take_ticket(uint32_t *ctr) {
    return __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void count_event(uint32_t *word) {
    __hip_atomic_fetch_add(word, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A descriptor's content: the state word (state in bits 1..0, a PARTIAL's
// distance from bit kDistShift up; the tag is added on publication) and the
// payload.
template <class T>
struct DescVal {
    uint32_t state;
    T value;
};

// One 64-bit word per tile: state word high, 32-bit payload low.  read()
// returns the state word as the call with tag field tf sees it (0 when
// another call wrote it); publish() and install() add tf.
template <class Op>
struct Words1 {
    using T = typename Op::T;
    static constexpr int WORDS = 1;
    // load() only issues the read; decode() interprets it -- separately, so
    // that a window read ahead of a barrier is not waited for before it
    __device__ static void load(const uint64_t *desc, int64_t tile, uint64_t (&raw)[WORDS]) {
        raw[0] = desc_poll(desc + tile);
    }
    __device__ static void decode(const uint64_t (&raw)[WORDS], uint32_t tf, uint32_t &state, T &v) {
        state = state_seen((uint32_t)(raw[0] >> 32), tf);
        v = from_bits<T>((uint32_t)raw[0]);
    }
    __device__ static void publish(uint64_t *desc, uint32_t tile, uint32_t tf, uint32_t state, T v) {
        desc_publish(desc + tile, ((uint64_t)(state | tf) << 32) | to_bits(v));
    }
    __device__ static bool install(uint64_t *desc, uint32_t tile, uint32_t tf, uint32_t state, T v) {
        return desc_install(desc + tile, ((uint64_t)(state | tf) << 32) | to_bits(v), tf);
    }
};

// Two 64-bit words per tile for a 64-bit payload: word 0 = state word | low
// half, word 1 = state word | high half, each one atomic store.  A reader
// takes the tile only when both state words agree.  Every state word
// (state, tag and distance) is published with one payload only, so agreeing
// words hold the two halves of one value; a read that meets a publication
// half done sees two different state words and polls again.  The one
// exception is a fallback's install racing the owner's own first
// publication of the same state: a reader may then take one half from
// each.  Both are reductions of the same tile, equal for integers and each
// a valid fp32 evaluation for floating point.
template <class Op>
struct Words2 {
    using T = typename Op::T;
    static constexpr int WORDS = 2;
    __device__ static void load(const uint64_t *desc, int64_t tile, uint64_t (&raw)[WORDS]) {
        raw[0] = desc_poll(desc + 2 * tile);
        raw[1] = desc_poll(desc + 2 * tile + 1);
    }
    __device__ static void decode(const uint64_t (&raw)[WORDS], uint32_t tf, uint32_t &state, T &v) {
        const uint32_t s0 = state_seen((uint32_t)(raw[0] >> 32), tf), s1 = state_seen((uint32_t)(raw[1] >> 32), tf);
        state = (s0 == s1) ? s0 : ST_INVALID;
        v = from_bits64<T>(((uint64_t)(uint32_t)raw[1] << 32) | (uint32_t)raw[0]);
    }
    __device__ static void publish(uint64_t *desc, uint32_t tile, uint32_t tf, uint32_t state, T v) {
        const uint64_t b = to_bits64(v), sw = (uint64_t)(state | tf) << 32;
        desc_publish(desc + 2 * (uint64_t)tile, sw | (uint32_t)b);
        desc_publish(desc + 2 * (uint64_t)tile + 1, sw | (uint32_t)(b >> 32));
    }
    __device__ static bool install(uint64_t *desc, uint32_t tile, uint32_t tf, uint32_t state, T v) {
        const uint64_t b = to_bits64(v), sw = (uint64_t)(state | tf) << 32;
        const bool lo = desc_install(desc + 2 * (uint64_t)tile, sw | (uint32_t)b, tf);
        const bool hi = desc_install(desc + 2 * (uint64_t)tile + 1, sw | (uint32_t)(b >> 32), tf);
        return lo || hi;
    }
};

template <class Op>
using WordsFor = typename std::conditional<sizeof(typename Op::T) == 8, Words2<Op>, Words1<Op>>::type;

// A look-back that never computes a predecessor itself.
template <class T>
struct NoFallback {
    __device__ DescVal<T> operator()(uint32_t, uint32_t) const { return DescVal<T>{ST_INVALID, T{}}; }
};

struct LookbackStats {
    uint32_t polls = 0;    // poll rounds (64*K descriptor reads each)
    uint32_t windows = 0;  // windows of predecessors folded
    uint32_t stalls = 0;   // polls that found an unpublished predecessor
};

// What a look-back may do besides waiting: after `fallback_after` stalled
// polls in a row (0 = never) reduce the stalled predecessor's input itself;
// once it has walked `partial` windows without reaching an inclusive prefix
// (0 = never), publish a PARTIAL descriptor for its own tile after every
// further window.  `flags` are debug settings of the whole kernel (kDbg*);
// `tf` is the tag field of the call, filled in on the device.
struct LookbackCfg {
    uint32_t fallback_after;
    uint32_t partial;
    uint32_t flags;
    uint32_t tf;
};

// Debug setting: tiles never publish their AGGREGATE (only PREFIX, and
// PARTIALs), so every look-back that reaches a tile before its owner has
// resolved its prefix stalls there -- with a fallback configured, that
// fallback is what supplies the aggregate.
constexpr uint32_t kDbgWithholdAggregates = PS_DEBUG_WITHHOLD_AGGREGATES;

// Safety net of the spin: a wave that finds an unpublished predecessor this
// many times in a row (seconds of waiting; a healthy chain needs a few) gives
// up, raises the workspace error word and continues with a wrong prefix
// instead of hanging the GPU.  Progress is guaranteed by the protocol, so the
// limit only trips on a broken workspace or a faulting predecessor.
constexpr uint32_t kSpinLimit = 1u << 20;

// Descriptors read per lane per poll (the look-back window is 64 * K tiles).
#ifndef DWPS_LOOKBACK_K
#define DWPS_LOOKBACK_K 2
#endif

// One poll's worth of descriptor words, the 64*K predecessors from
// base = nearest - 64K + 1 on.  Two layouts: blocked, word j of lane l is
// tile base + 64j + l (each load instruction reads 64 consecutive
// descriptors); interleaved, it is tile base + Kl + j (each lane reads K
// consecutive ones, and a lane can fold its own words in tile order).
template <int K, int WORDS>
struct Window {
    uint64_t raw[K][WORDS];  // descriptor words as read, decoded when used
};

template <int K, bool BLOCKED>
__device__ __forceinline__ int64_t window_index(int64_t base, uint32_t lane, int j) {
    return BLOCKED ? base + 64 * j + (int64_t)lane : base + (int64_t)lane * K + j;
}

// Issue the loads of one window.  Every load is issued before any is used
// (no branch around a load, so one poll costs one round trip), and nothing
// is computed from them here, so a window read ahead of a barrier is only
// waited for where it is decoded; words before tile 0 read tile 0's and are
// replaced by the look-back.
template <class Op, int K, bool BLOCKED, class W = WordsFor<Op>>
__device__ __forceinline__ void window_load(const uint64_t *desc, int64_t nearest, uint32_t lane,
                                            Window<K, W::WORDS> &win) {
    const int64_t base = nearest - 64 * K + 1;
#pragma unroll
    for (int j = 0; j < K; ++j) {
        const int64_t idx = window_index<K, BLOCKED>(base, lane, j);
        W::load(desc, idx >= 0 ? idx : 0, win.raw[j]);
    }
}

// Decoupled look-back, executed by one full wave over windows of 64*K
// predecessors (BLOCKED or interleaved, see Window).  Indices below 0 read
// as a PREFIX carrying the identity.
//
// Walking back from the nearest predecessor, an AGGREGATE adds its payload
// and steps one tile, a PARTIAL adds its payload and jumps over the d tiles
// it covers, a PREFIX adds its payload and ends the walk, an INVALID waits.
// In a window: let s be the nearest word in PREFIX or PARTIAL state; if a
// word nearer than s is INVALID the window is polled again (each poll
// reloads every word); otherwise the payloads from s to the nearest
// predecessor are folded in tile order (blocked: one wave scan per block,
// the blocks in order; interleaved: each lane folds its own words, one wave
// scan joins the lanes).  At a PREFIX the fold is final; at a PARTIAL the
// next window ends just before the tiles it covers; with neither, the
// window slides 64*K tiles back.  Each time the walk continues, the tile's
// own descriptor becomes a PARTIAL covering everything folded so far and
// itself (once cfg.partial windows were walked, and when may_publish), so
// later look-backs over the same stretch jump it in one read -- the
// bounded-window variant of "Single-Pass Prefix Scan with Decoupled
// Look-Back", section "Why the work stays linear", with W = cfg.partial
// windows of 64*K predecessors.
//
// After cfg.fallback_after stalled polls in a row the wave reduces the
// nearest unpublished predecessor from its input (fb(tile, lane) returns the
// descriptor word that tile's owner would publish first) and installs it
// over INVALID with a compare-and-swap, so the first of several fallbacks on
// one tile wins and the owner's own later stores agree with it
// ("GPUPrefixSums", section "Decoupled Fallback").  After kSpinLimit stalled
// polls the unpublished words are folded as they are and the error word is
// set.  Returns the exclusive prefix of `tile` (the fold of every earlier
// tile).  Terminates because tile 0 publishes PREFIX without waiting and
// every tile only waits on tiles that took their ticket earlier, hence are
// resident or finished ("Single-Pass Prefix Scan with Decoupled Look-Back",
// sections "Three states in a per-block descriptor" and "Where the algorithm
// meets the hardware").  `pre`, when given, is the first window, read ahead
// of time (an older read of a descriptor is still a valid one: states only
// move forward, and an unpublished word just costs another poll).
template <class Op, int K, bool STATS, class FB, class W>
__device__ __forceinline__ typename Op::T lookback_blocked(uint64_t *desc, uint32_t tile, uint32_t lane,
                                                           LookbackStats &st, uint32_t *hdr, LookbackCfg cfg,
                                                           typename Op::T own, bool may_publish, const FB &fb,
                                                           const Window<K, W::WORDS> *pre) {
    using T = typename Op::T;
    T acc = Op::id();
    int64_t nearest = (int64_t)tile - 1;
    uint32_t spins = 0, stalled = 0, walked = 0;
    bool use_pre = pre != nullptr;  // a constant wherever lookback is inlined
    for (;;) {
        const int64_t base = nearest - 64 * K + 1;
        Window<K, W::WORDS> win;
        if (use_pre)
            win = *pre;
        else
            window_load<Op, K, true, W>(desc, nearest, lane, win);
        use_pre = false;
        uint32_t sw[K];  // state words
        T val[K];
#pragma unroll
        for (int j = 0; j < K; ++j) {
            W::decode(win.raw[j], cfg.tf, sw[j], val[j]);
            const bool before = window_index<K, true>(base, lane, j) < 0;
            sw[j] = before ? ST_PREFIX : sw[j];
            val[j] = before ? Op::id() : val[j];
        }
        // the nearest PREFIX/PARTIAL word: block js, lane ls (js = -1: none)
        int js = -1;
        uint64_t pm = 0;
#pragma unroll
        for (int j = 0; j < K; ++j) {
            const uint64_t m = ballot((sw[j] & 3u) >= ST_PREFIX);
            js = m ? j : js;
            pm = m ? m : pm;
        }
        const uint32_t ls = pm ? 63u - (uint32_t)__builtin_clzll(pm) : 0u;
        bool rel[K];  // nearer than the stopper, or the stopper itself
#pragma unroll
        for (int j = 0; j < K; ++j) rel[j] = j > js || (j == js && lane >= ls);
        // the nearest INVALID word among them: block ji, lane li
        int ji = -1;
        uint64_t imask = 0;
#pragma unroll
        for (int j = 0; j < K; ++j) {
            const uint64_t m = ballot(rel[j] && (sw[j] & 3u) == ST_INVALID);
            ji = m ? j : ji;
            imask = m ? m : imask;
        }
        if (STATS) st.polls++;
        if (ji >= 0) {
            if (STATS) st.stalls++;
            if (cfg.fallback_after && ++stalled >= cfg.fallback_after) {
                // reduce the nearest unpublished predecessor ourselves
                const uint32_t li = 63u - (uint32_t)__builtin_clzll(imask);
                const int64_t p = base + 64 * ji + (int64_t)li;
                const DescVal<T> dv = fb((uint32_t)p, lane);
                if (lane == 0 && W::install(desc, (uint32_t)p, cfg.tf, dv.state, dv.value)) count_event(hdr + kHdrFallbacks);
                stalled = 0;
                continue;
            }
            if (++spins < kSpinLimit) {
                __builtin_amdgcn_s_sleep(1);
                continue;
            }
            if (lane == 0) __hip_atomic_fetch_or(hdr + kHdrError, kErrSpin, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        spins = 0;
        stalled = 0;
        // fold the counted words in tile order: block by block, the lanes of
        // a block by the wave scan
        T wsum = Op::id();
#pragma unroll
        for (int j = 0; j < K; ++j) {
            if (j >= js) {
                const T v = wave_inclusive<Op>(rel[j] ? val[j] : Op::id());
                wsum = Op::op(wsum, read_lane(v, 63));
            }
        }
        acc = Op::op(wsum, acc);
        if (STATS) st.windows++;
        if (js >= 0) {
            // the stopper's state word, uniform
            uint32_t ss = sw[0];
#pragma unroll
            for (int j = 1; j < K; ++j) ss = (j == js) ? sw[j] : ss;
            const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)ss, (int)ls);
            if ((hi & 3u) == ST_PREFIX) break;
            const int64_t stop = base + 64 * js + (int64_t)ls;
            nearest = stop - (int64_t)(hi >> kDistShift);
        } else {
            nearest -= 64 * K;
        }
        if (nearest < 0) break;  // a PARTIAL reaching back to tile 0 ends the walk
        if (cfg.partial && ++walked >= cfg.partial && may_publish && lane == 0) {
            W::publish(desc, tile, cfg.tf, ((uint32_t)((int64_t)tile - nearest) << kDistShift) | ST_PARTIAL,
                       Op::op(acc, own));
            // counted by the instrumented build only: an atomic on one shared
            // word would queue ahead of this wave's next poll
            if (STATS) count_event(hdr + kHdrPartials);
        }
    }
    return acc;
}

template <class Op, int K, bool STATS, class FB, class W>
__device__ __forceinline__ typename Op::T lookback_interleaved(uint64_t *desc, uint32_t tile, uint32_t lane,
                                                               LookbackStats &st, uint32_t *hdr, LookbackCfg cfg,
                                                               typename Op::T own, bool may_publish, const FB &fb,
                                                               const Window<K, W::WORDS> *pre) {
    using T = typename Op::T;
    T acc = Op::id();
    int64_t nearest = (int64_t)tile - 1;
    uint32_t spins = 0, stalled = 0, walked = 0;
    bool use_pre = pre != nullptr;  // a constant wherever lookback is inlined
    for (;;) {
        const int64_t first = nearest - 64 * K + 1 + (int64_t)lane * K;
        uint32_t sw[K];  // state words
        T val[K];
        // the first window may have been read ahead of time (an older read
        // of a descriptor is still a valid one: states only move forward,
        // and an unpublished word just costs another poll)
        Window<K, W::WORDS> win;
        if (use_pre)
            win = *pre;
        else
            window_load<Op, K, false, W>(desc, nearest, lane, win);
        use_pre = false;
#pragma unroll
        for (int j = 0; j < K; ++j) W::decode(win.raw[j], cfg.tf, sw[j], val[j]);
#pragma unroll
        for (int j = 0; j < K; ++j) {
            const bool before = first + j < 0;
            sw[j] = before ? ST_PREFIX : sw[j];
            val[j] = before ? Op::id() : val[j];
        }
        // nearest PREFIX/PARTIAL word of this lane (-1 if none), and the
        // nearest INVALID word nearer than it (-1 if none)
        int jp = -1;
#pragma unroll
        for (int j = 0; j < K; ++j)
            if ((sw[j] & 3u) >= ST_PREFIX) jp = j;
        int ji = -1;
#pragma unroll
        for (int j = 0; j < K; ++j)
            if (j > jp && (sw[j] & 3u) == ST_INVALID) ji = j;
        const uint64_t pm = ballot(jp >= 0);
        const uint32_t lp = pm ? 63u - (uint32_t)__builtin_clzll(pm) : 0u;
        // lanes above lp count entirely; lane lp counts from its stopper word
        const bool relevant = pm ? (lane >= lp) : true;
        if (STATS) st.polls++;
        const uint64_t im = ballot(relevant && ji >= 0);
        if (im) {
            if (STATS) st.stalls++;
            if (cfg.fallback_after && ++stalled >= cfg.fallback_after) {
                // reduce the nearest unpublished predecessor ourselves
                const uint32_t li = 63u - (uint32_t)__builtin_clzll(im);
                const int64_t p = nearest - 64 * K + 1 + (int64_t)li * K + __builtin_amdgcn_readlane(ji, (int)li);
                const DescVal<T> dv = fb((uint32_t)p, lane);
                if (lane == 0 && W::install(desc, (uint32_t)p, cfg.tf, dv.state, dv.value)) count_event(hdr + kHdrFallbacks);
                stalled = 0;
                continue;
            }
            if (++spins < kSpinLimit) {
                __builtin_amdgcn_s_sleep(1);
                continue;
            }
            if (lane == 0) __hip_atomic_fetch_or(hdr + kHdrError, kErrSpin, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        spins = 0;
        stalled = 0;
        T v = Op::id();
        if (relevant) {
            const int jfrom = (pm && lane == lp) ? jp : 0;
#pragma unroll
            for (int j = 0; j < K; ++j)
                if (j >= jfrom) v = Op::op(v, val[j]);
        }
        v = wave_inclusive<Op>(v);
        acc = Op::op(read_lane(v, 63), acc);
        if (STATS) st.windows++;
        if (pm) {
            // the stopper's state word, uniform
            uint32_t ss = sw[0];
#pragma unroll
            for (int j = 1; j < K; ++j) ss = (j == jp) ? sw[j] : ss;
            const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)ss, (int)lp);
            if ((hi & 3u) == ST_PREFIX) break;
            const int64_t s = nearest - 64 * K + 1 + (int64_t)lp * K + __builtin_amdgcn_readlane(jp, (int)lp);
            nearest = s - (int64_t)(hi >> kDistShift);
        } else {
            nearest -= 64 * K;
        }
        if (nearest < 0) break;  // a PARTIAL reaching back to tile 0 ends the walk
        if (cfg.partial && ++walked >= cfg.partial && may_publish && lane == 0) {
            W::publish(desc, tile, cfg.tf, ((uint32_t)((int64_t)tile - nearest) << kDistShift) | ST_PARTIAL,
                       Op::op(acc, own));
            // counted by the instrumented build only: an atomic on one shared
            // word would queue ahead of this wave's next poll
            if (STATS) count_event(hdr + kHdrPartials);
        }
    }
    return acc;
}

template <class Op, int K, bool STATS, bool BLOCKED = false, class FB = NoFallback<typename Op::T>,
          class W = WordsFor<Op>>
__device__ __forceinline__ typename Op::T lookback(uint64_t *desc, uint32_t tile, uint32_t lane, LookbackStats &st,
                                                   uint32_t *hdr, LookbackCfg cfg = LookbackCfg{0u, 0u, 0u, 0u},
                                                   typename Op::T own = Op::id(), bool may_publish = false,
                                                   const FB &fb = FB{},
                                                   const Window<K, W::WORDS> *pre = nullptr) {
    if constexpr (BLOCKED)
        return lookback_blocked<Op, K, STATS, FB, W>(desc, tile, lane, st, hdr, cfg, own, may_publish, fb, pre);
    else
        return lookback_interleaved<Op, K, STATS, FB, W>(desc, tile, lane, st, hdr, cfg, own, may_publish, fb, pre);
}

}  // namespace dwps
