// Host model of a workspace's descriptor words under the hand-over rules of
// ws_state.hpp (the same functions the kernels call).  A random sequence of
// calls -- single-pass calls of random sizes, two-level calls writing their
// totals, staged compactions writing offsets into descriptor words,
// re-preparations -- runs against an array of modelled state words, and
// before every single-pass call the model checks the one property the
// rules exist for: after the call's cleaning, every word it uses reads as
// unpublished under its tag.  Argument "broken" runs a copy of the end rule
// that forgets the wrap; the model must then find a violation.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <random>
#include <vector>

#include "ws_state.hpp"

using namespace dwps;

namespace {

struct Header {
    uint32_t magic = 0, capacity = 0, tag = 0, high = 0, dlo = 0, dhi = 0;
};

void prepare(Header &h, uint32_t capacity) {
    h = Header{};
    h.magic = kWsMagic;
    h.capacity = capacity;
    h.dhi = capacity;
}

// ws_end with the wrap rule left out.
WsEnd end_without_wrap(const WsBegin &b, const WsPlan &p, uint32_t need) {
    WsEnd e;
    e.high = b.high > need ? b.high : need;
    uint32_t lo = b.dirty_lo, hi = b.dirty_hi;
    if (p.clean_lo < p.clean_hi) lo = p.clean_hi;
    if (lo >= hi) lo = hi = 0u;
    e.tag = (p.tag + 1u) & (kTagCount - 1u);
    e.dirty_lo = lo;
    e.dirty_hi = hi;
    return e;
}

}  // namespace

int main(int argc, char **argv) {
    const bool broken = argc > 1 && strcmp(argv[1], "broken") == 0;
    const long calls = argc > 2 ? atol(argv[2]) : 300000;
    const uint32_t cap = 4096;
    std::mt19937_64 g(12345);
    // state words as the hardware would hold them (the payload plays no part)
    std::vector<uint32_t> sw(cap, 0xFFFFFFFFu);  // garbage before preparation
    Header h;
    prepare(h, cap);
    long violations = 0, single = 0, wraps = 0, cleaned = 0;
    // Sizes come in regimes: stretches of small calls (at most 64 words)
    // alternate with stretches of calls of any size.  A stretch of small
    // calls often lasts a multiple of the tag period less one call, so the
    // next large call meets large-index words left by a call with its tag.
    bool small_regime = false;
    long regime_left = 0;
    for (long c = 0; c < calls; ++c) {
        if (regime_left <= 0) {
            small_regime = !small_regime;
            const long periods[4] = {511, 1023, 1535, 2047};
            regime_left = (g() % 2) ? periods[g() % 4] : 1 + (long)(g() % 3000);
            if (!small_regime) regime_left = 1 + (long)(g() % 8);
        }
        const uint32_t kind = (uint32_t)(g() % 100000);
        uint32_t need = small_regime ? 1u + (uint32_t)(g() % 64) : 1u + (uint32_t)(g() % cap);
        if (kind < 2) {
            // re-preparation (after a failed call, say): words keep whatever they hold
            prepare(h, cap);
            continue;
        }
        if (kind < 5000) {
            // two-level call: totals as words with a zero state word
            for (uint32_t i = 0; i < need; ++i) sw[i] = 0u;
            continue;
        }
        if (kind < 5100) {
            // staged compaction: the flag scan is a single-pass call (below),
            // then plain offsets fill [a, b) and the range is marked dirty
            const uint32_t a = need < cap ? need : cap - 1u;
            const uint32_t b = a + (uint32_t)(g() % (cap - a)) + 1u;
            for (uint32_t i = a; i < b; ++i) sw[i] = (uint32_t)g();
            ws_mark_dirty(h.dlo, h.dhi, a, b);
            continue;
        }
        // a single-pass call
        --regime_left;
        const WsBegin b{h.magic, h.capacity, h.tag, h.high, h.dlo, h.dhi};
        const WsPlan p = ws_plan(b, need);
        if (!p.ok) {
            printf("call %ld: plan refused (error %u)\n", c, p.error);
            return 2;
        }
        for (uint32_t i = p.clean_lo; i < p.clean_hi; ++i) sw[i] = 0u;
        cleaned += p.clean_hi - p.clean_lo;
        const uint32_t tf = tag_field(p.tag);
        for (uint32_t i = 0; i < need; ++i)
            if (state_seen(sw[i], tf) != 0u) {
                ++violations;
                break;
            }
        // the call publishes every word it uses, in some state, with its tag
        // and a random PARTIAL distance
        for (uint32_t i = 0; i < need; ++i)
            sw[i] = (1u + (uint32_t)(g() % 3)) | tf | ((uint32_t)(g() % 1000) << kDistShift);
        const WsEnd e = broken ? end_without_wrap(b, p, need) : ws_end(b, p, need);
        if (e.tag == 0u) ++wraps;
        h.tag = e.tag;
        h.high = e.high;
        h.dlo = e.dirty_lo;
        h.dhi = e.dirty_hi;
        ++single;
    }
    printf("%s: %ld single-pass calls, %ld tag wraps, %ld words cleaned, %ld violations\n",
           broken ? "broken" : "rules", single, wraps, cleaned, violations);
    if (broken) return violations > 0 ? 0 : 1;
    return violations == 0 ? 0 : 1;
}
