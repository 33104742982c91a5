// ws_state.hpp -- the workspace header of the single-pass kernels and the
// rules by which one call hands the workspace to the next.
//
// A workspace is prepared once (ps_workspace_init) and then kept ready by
// the calls themselves, so a call is one kernel launch with no separate
// clear.  Every tile descriptor carries, next to its state ("Single-Pass
// Prefix Scan with Decoupled Look-Back", section "Three states in a
// per-block descriptor": a slot starts out invalid), the 9-bit tag of the
// call that wrote it; a reader takes a word whose tag is not its own call's
// as unpublished.  The tag advances by one per call, so the words a call
// leaves behind are invalid for the next 511 calls without being touched.
// What the header tracks so that no stale word is ever read as valid:
//   * a high-water mark of the descriptor words any call has tagged;
//   * a dirty range [lo, hi) of words that may hold anything: the whole
//     descriptor area after preparation, the tagged words up to the
//     high-water mark whenever the tag wraps (their tags come round again),
//     and whatever a call that uses the workspace as plain scratch has
//     written there;
//   * whether the call in flight has cleaned its part of the dirty range.
// A call that needs dirty words cleans them before any of its descriptors
// is read or written: the workgroup holding the first tile zeroes them and
// raises the ready word, and every other workgroup waits for that word
// before its first descriptor access (the first tile's workgroup is
// running, so the wait ends).  The last workgroup to finish resets the
// ticket and completion counters, advances the tag and shrinks or grows the
// dirty range for the next call.
//
// Plain C++ with no HIP dependency: the kernels use these functions on the
// device and a host test runs them against a model of the descriptor array.
#pragma once

#include <stdint.h>

#include "dwps.h"

#if defined(__HIPCC__)
#define DWPS_HD __host__ __device__
#else
#define DWPS_HD
#endif

namespace dwps {

// 32-bit words of the 256-byte header (their meaning: ps_ws_word in dwps.h).
constexpr int kHdrTicket = PS_WS_TICKET;
constexpr int kHdrError = PS_WS_ERROR;
constexpr int kHdrFallbacks = PS_WS_FALLBACKS;
constexpr int kHdrPartials = PS_WS_PARTIALS;
constexpr int kHdrTag = PS_WS_TAG;
constexpr int kHdrDone = PS_WS_DONE;
constexpr int kHdrMagic = PS_WS_MAGIC;
constexpr int kHdrCapacity = PS_WS_CAPACITY;
constexpr int kHdrHigh = PS_WS_HIGH;
constexpr int kHdrDirtyLo = PS_WS_DIRTY_LO;
constexpr int kHdrDirtyHi = PS_WS_DIRTY_HI;
constexpr int kHdrReady = PS_WS_READY;
constexpr int kHdrCalls = PS_WS_CALLS;
constexpr int kHdrWords = PS_WS_DONE + 1;

constexpr uint32_t kWsMagic = 0x44575053u;  // "DWPS"

constexpr uint32_t kErrSpin = PS_WS_ERR_SPIN;
constexpr uint32_t kErrNotPrepared = PS_WS_ERR_NOT_PREPARED;
constexpr uint32_t kErrCapacity = PS_WS_ERR_CAPACITY;

// Descriptor state word (the high 32 bits of a descriptor word): bits 1..0
// the state, bits 10..2 the tag of the call that wrote it, bits 31..11 the
// distance of a PARTIAL (up to 2^21 - 1 tiles, more than any call has).
constexpr uint32_t ST_INVALID = 0u;    // nothing published
constexpr uint32_t ST_AGGREGATE = 1u;  // payload = the tile's own fold
constexpr uint32_t ST_PREFIX = 2u;     // payload = fold of tiles 0..t (inclusive)
constexpr uint32_t ST_PARTIAL = 3u;    // payload = fold of tiles t-d+1..t, d in the high bits
constexpr uint32_t kTagBits = 9;
constexpr uint32_t kTagCount = 1u << kTagBits;
constexpr uint32_t kTagShift = 2;
constexpr uint32_t kTagField = (kTagCount - 1u) << kTagShift;
constexpr uint32_t kDistShift = kTagShift + kTagBits;
constexpr uint32_t kMaxDistance = (1u << (32 - kDistShift)) - 1u;

DWPS_HD inline uint32_t tag_field(uint32_t tag) { return (tag & (kTagCount - 1u)) << kTagShift; }

// A state word as the call with tag field `tf` sees it: unchanged if that
// call wrote it, else 0 (unpublished).
DWPS_HD inline uint32_t state_seen(uint32_t sw, uint32_t tf) { return (sw & kTagField) == tf ? sw : 0u; }

// What every workgroup reads from the header when a call starts.
struct WsBegin {
    uint32_t magic, capacity, tag, high, dirty_lo, dirty_hi;
};

// What the call does with it, for a call that uses `need` descriptor words.
struct WsPlan {
    bool ok;            // prepared and large enough; otherwise nothing runs
    uint32_t error;     // kErr* bits to raise when !ok
    uint32_t tag;       // this call's tag
    uint32_t clean_lo;  // descriptor words [clean_lo, clean_hi) to zero before use
    uint32_t clean_hi;
};

DWPS_HD inline WsPlan ws_plan(const WsBegin &b, uint32_t need) {
    WsPlan p{true, 0u, b.tag & (kTagCount - 1u), 0u, 0u};
    if (b.magic != kWsMagic) {
        p.ok = false;
        p.error = kErrNotPrepared;
        return p;
    }
    if (need > b.capacity) {
        p.ok = false;
        p.error = kErrCapacity;
        return p;
    }
    const uint32_t hi = b.dirty_hi < need ? b.dirty_hi : need;
    if (b.dirty_lo < hi) {
        p.clean_lo = b.dirty_lo;
        p.clean_hi = hi;
    }
    return p;
}

// The header fields the last workgroup writes for the next call.
struct WsEnd {
    uint32_t tag, high, dirty_lo, dirty_hi;
};

// The union of two ranges as one range (an empty range is lo >= hi).
DWPS_HD inline void range_union(uint32_t &lo, uint32_t &hi, uint32_t a, uint32_t b) {
    if (a >= b) return;
    if (lo >= hi) {
        lo = a;
        hi = b;
        return;
    }
    lo = a < lo ? a : lo;
    hi = b > hi ? b : hi;
}

DWPS_HD inline WsEnd ws_end(const WsBegin &b, const WsPlan &p, uint32_t need) {
    WsEnd e;
    e.high = b.high > need ? b.high : need;
    // the words this call cleaned (a prefix of the dirty range, since the
    // cleaned range starts at dirty_lo) are clean or carry this call's tag
    uint32_t lo = b.dirty_lo, hi = b.dirty_hi;
    if (p.clean_lo < p.clean_hi) lo = p.clean_hi;
    if (lo >= hi) lo = hi = 0u;
    e.tag = (p.tag + 1u) & (kTagCount - 1u);
    // the tags come round again: every tagged word may now read as valid
    if (e.tag == 0u) range_union(lo, hi, 0u, e.high);
    e.dirty_lo = lo;
    e.dirty_hi = hi;
    return e;
}

// A call that writes plain data into descriptor words [a, b) (the staged
// compaction's offsets) marks them dirty.
DWPS_HD inline void ws_mark_dirty(uint32_t &lo, uint32_t &hi, uint32_t a, uint32_t b) { range_union(lo, hi, a, b); }

}  // namespace dwps
