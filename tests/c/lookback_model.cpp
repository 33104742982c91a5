// Host model of the look-back protocol of the single-pass kernels, run under
// adversarial schedules ("Single-Pass Prefix Scan with Decoupled Look-Back",
// sections "Three states in a per-block descriptor", "Why the work stays
// linear" and "Where the algorithm meets the hardware"; "GPUPrefixSums",
// section "Decoupled Fallback"; "Parallel Prefix Sum (Scan), in depth",
// section "Scanning a whole array: three grid strategies").
//
// Workgroups are coroutines that a scheduler advances one shared-memory
// action at a time -- a descriptor word's load, store or compare-and-swap,
// a ticket -- picking the workgroup at random with weights that starve some
// of them for long stretches.  Descriptor words behave as relaxed atomics:
// every word keeps the history of the values stored to it, and a load
// returns any value no older than the last one the loading workgroup has
// seen of that word (per-location coherence and nothing more), so the words
// of one window come from different moments and a two-word descriptor can
// be read half published.  A compare-and-swap acts on the newest value.
// Only `resident` workgroups run at once; a waiting one keeps its slot.
//
// Each workgroup follows the control wave's phase sequence: it takes a
// ticket when its group of G tiles runs out (or, in the fixed order, owns
// the groups its index names), looks back for the tile two phases behind
// the one it scans (the head of each group only), publishes that tile's
// inclusive prefix (with pairs, the next tile's too), and publishes the
// aggregate of the tile it has just scanned.  The look-back takes windows of
// `win` predecessors: the nearest PREFIX or PARTIAL word ends the window's
// fold, an INVALID word nearer than it makes the wave poll the window again,
// a PARTIAL moves the walk back by its distance; after `partial` windows
// the tile publishes its own PARTIAL; after `fallback` stalled polls in a
// row the wave reduces the stalled predecessor itself and installs its
// descriptor with a compare-and-swap over a word it read as unpublished.
// The segmented form: a tile holding a segment start publishes PREFIX at
// once and looks back only if its first element starts no segment.  With
// close=1 a workgroup that has no tile left to scan resolves the three
// tiles still waiting (prev2, prev and cur) in one step, in order, and
// stops -- the closing phase of the three-phase kernels.
//
// Checked: every descriptor a look-back accepts states a true fact about
// its tile (its payload is the fold its state claims), every exclusive
// prefix equals the fold of the earlier tiles, every workgroup finishes --
// or, for expect=deadlock, the run reaches a state where every resident
// workgroup waits on a tile that no running workgroup owns.  The operators
// are not commutative, so a fold in the wrong order fails.  At the start the
// words hold what earlier calls left: other tags, any state, any payload.
//
// Arguments key=value: words op tiles wgs resident G win partial fallback
// pair persistent tickets withhold close order(asc|desc|random) p_fresh seeds seed
// broken(torn|no_tag|partial_distance|skip_invalid|close_order) expect(ok|deadlock|
// violation).  Exit 0 when the outcome is the expected one.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <coroutine>
#include <exception>
#include <random>
#include <string>
#include <vector>

#include "ws_state.hpp"

using namespace dwps;

namespace {

// ---------------------------------------------------------------------------
// Operators: op(x, y) with x the earlier operand.  None is commutative.
// ---------------------------------------------------------------------------
enum class OpKind { Affine16, Affine32, Segmented };

struct OpDef {
    OpKind k;
    uint64_t id() const { return k == OpKind::Affine16 ? 0x10000u : k == OpKind::Affine32 ? (1ull << 32) : 0u; }
    uint64_t op(uint64_t x, uint64_t y) const {
        switch (k) {
            case OpKind::Affine16: {  // h -> a h + b over Z/2^16, (a << 16) | b
                const uint64_t xa = x >> 16, xb = x & 0xFFFFu, ya = y >> 16, yb = y & 0xFFFFu;
                return (((xa * ya) & 0xFFFFu) << 16) | ((ya * xb + yb) & 0xFFFFu);
            }
            case OpKind::Affine32: {  // the same over Z/2^32, (a << 32) | b
                const uint64_t xa = x >> 32, xb = x & 0xFFFFFFFFu, ya = y >> 32, yb = y & 0xFFFFFFFFu;
                return (((xa * ya) & 0xFFFFFFFFu) << 32) | ((ya * xb + yb) & 0xFFFFFFFFu);
            }
            default: {  // (start flag << 31) | sum mod 2^31: a start in y resets the sum
                const uint64_t yf = y >> 31;
                const uint64_t f = (x >> 31) | yf;
                const uint64_t v = yf ? (y & 0x7FFFFFFFu) : ((x + y) & 0x7FFFFFFFu);
                return (f << 31) | v;
            }
        }
    }
    // a tile whose inclusive prefix is its own fold (it holds a segment start)
    bool self_prefix(uint64_t agg) const { return k == OpKind::Segmented && (agg >> 31) != 0; }
};

struct Config {
    int words = 1;
    OpKind op = OpKind::Affine16;
    uint32_t tiles = 300, wgs = 12, resident = 12, G = 2, win = 4, partial = 1, fallback = 0;
    bool pair = true, persistent = true, tickets = true, withhold = false, close = false;
    std::string order = "random";
    double p_fresh = 0.5;
    uint64_t seed = 1;
    int seeds = 20;
    std::string broken, expect = "ok";
};

struct Counts {
    long steps = 0, loads = 0, stale = 0, stale_tag = 0, torn = 0, mixed = 0, partial_pubs = 0, partial_jumps = 0,
         fallbacks = 0, cas_won = 0, cas_lost = 0, skipped_install = 0, stalls = 0, windows = 0, deadlocks = 0,
         closings = 0, closing_lookbacks = 0;
    void add(const Counts &o) {
        steps += o.steps, loads += o.loads, stale += o.stale, stale_tag += o.stale_tag, torn += o.torn;
        mixed += o.mixed, partial_pubs += o.partial_pubs, partial_jumps += o.partial_jumps;
        fallbacks += o.fallbacks, cas_won += o.cas_won, cas_lost += o.cas_lost;
        skipped_install += o.skipped_install, stalls += o.stalls, windows += o.windows, deadlocks += o.deadlocks;
        closings += o.closings, closing_lookbacks += o.closing_lookbacks;
    }
};

// A coroutine that stops before every shared-memory action.
struct Proc {
    struct promise_type {
        Proc get_return_object() { return Proc{std::coroutine_handle<promise_type>::from_promise(*this)}; }
        std::suspend_always initial_suspend() noexcept { return {}; }
        std::suspend_always final_suspend() noexcept { return {}; }
        std::suspend_always yield_value(int) noexcept { return {}; }
        void return_void() {}
        void unhandled_exception() { std::terminate(); }
    };
    std::coroutine_handle<promise_type> h;
};

struct Model {
    Config c;
    OpDef op;
    std::mt19937_64 rng;
    uint32_t N = 0, tf = 0, ticket = 0;
    std::vector<uint64_t> agg, incl;          // the tiles' folds and inclusive prefixes
    std::vector<uint8_t> first_start;         // segmented: the tile's first element starts a segment
    std::vector<uint64_t> result;             // exclusive prefixes the workgroups found
    std::vector<uint8_t> has_result;
    std::vector<std::vector<uint64_t>> hist;  // descriptor words: every value stored, in order
    std::vector<std::vector<uint32_t>> src;   // the publication each value came from
    std::vector<std::vector<uint32_t>> seen;  // per workgroup, per word: newest index it has read
    std::vector<uint8_t> waiting;             // per workgroup: polling a window that stalled
    uint32_t pubs = 0;
    long violations = 0, last_progress = 0;
    Counts n;

    double uni() { return (double)(rng() >> 11) * 0x1.0p-53; }
    uint32_t word(uint32_t t, int k) const { return (uint32_t)c.words * t + (uint32_t)k; }
    long printed = 0;  // over all schedules
    void violation(const char *what, long a, long b) {
        ++violations;
        if (printed++ < 3) printf("  violation: %s (tile %ld, %ld)\n", what, a, b);
    }
    void progress() { last_progress = n.steps; }

    uint64_t fold(uint32_t lo, uint32_t hi) const {  // tiles lo..hi
        uint64_t f = op.id();
        for (uint32_t i = lo; i <= hi; ++i) f = op.op(f, agg[i]);
        return f;
    }
    // whether (state word, payload) is true of tile t
    bool fact(uint32_t t, uint32_t sw, uint64_t v) const {
        switch (sw & 3u) {
            case ST_AGGREGATE: return v == agg[t];
            case ST_PREFIX: return v == incl[t];
            case ST_PARTIAL: {
                const uint32_t d = sw >> kDistShift;
                return d >= 1 && d <= t + 1 && v == fold(t + 1 - d, t);
            }
            default: return false;
        }
    }

    // relaxed load: any value from the newest one this workgroup has seen on
    uint64_t load(uint32_t w, uint32_t a, uint32_t *source) {
        const uint32_t last = (uint32_t)hist[a].size() - 1u;
        uint32_t &s = seen[w][a];
        uint32_t i = last;
        if (uni() >= c.p_fresh) i = s + (uint32_t)(rng() % (uint64_t)(last - s + 1u));
        n.loads++;
        if (i != last) n.stale++;
        s = i;
        if (source) *source = src[a][i];
        return hist[a][i];
    }
    void store(uint32_t w, uint32_t a, uint64_t v, uint32_t pub) {
        hist[a].push_back(v);
        src[a].push_back(pub);
        seen[w][a] = (uint32_t)hist[a].size() - 1u;
        progress();
    }
    bool cas(uint32_t w, uint32_t a, uint64_t expected, uint64_t v, uint32_t pub) {
        if (hist[a].back() != expected) {
            seen[w][a] = (uint32_t)hist[a].size() - 1u;  // a failed CAS reads the newest value
            return false;
        }
        store(w, a, v, pub);
        return true;
    }
    // one descriptor word of a publication: state word high, 32 payload bits low
    uint64_t encode(uint32_t sw, uint64_t v, int k) const {
        const uint64_t half = (c.words == 1 || k == 0) ? (v & 0xFFFFFFFFu) : (v >> 32);
        return ((uint64_t)(sw | tf) << 32) | half;
    }
    // the state word as the call sees it, the kernels' rule (or a broken one)
    uint32_t seen_state(uint64_t raw) {
        const uint32_t sw = (uint32_t)(raw >> 32);
        if ((sw & 3u) != ST_INVALID && (sw & kTagField) != tf) n.stale_tag++;
        return c.broken == "no_tag" ? sw : state_seen(sw, tf);
    }

    void setup(uint64_t seed) {
        rng.seed(seed);
        N = c.tiles;
        tf = tag_field(5);
        agg.assign(N, 0);
        incl.assign(N, 0);
        first_start.assign(N, 0);
        for (uint32_t t = 0; t < N; ++t) {
            const uint64_t r = rng();
            if (c.op == OpKind::Affine16) agg[t] = ((r | 0x10000u) & 0xFFFFFFFFu);  // odd multiplier
            else if (c.op == OpKind::Affine32) agg[t] = r | (1ull << 32);
            else {
                const bool start = rng() % 10 < 3;
                agg[t] = ((uint64_t)start << 31) | (r & 0x7FFFFFFFu);
                first_start[t] = start && rng() % 2;
            }
            incl[t] = op.op(t ? incl[t - 1] : op.id(), agg[t]);
        }
        result.assign(N, 0);
        has_result.assign(N, 0);
        const uint32_t W = (uint32_t)c.words * N;
        hist.assign(W, {});
        src.assign(W, {});
        for (uint32_t a = 0; a < W; ++a) {
            // left by an earlier call: zero, or any state and payload under another tag
            const uint32_t other = tag_field(1u + (uint32_t)(rng() % (kTagCount - 1u)) + 5u);
            const uint64_t left = (rng() % 3 == 0) ? 0u
                                                    : ((uint64_t)((uint32_t)(rng() % 4) | other |
                                                                  ((uint32_t)(rng() % 8) << kDistShift))
                                                       << 32) | (rng() & 0xFFFFFFFFu);
            hist[a].push_back(left);
            src[a].push_back(0);
        }
        seen.assign(c.wgs, std::vector<uint32_t>(W, 0));
        waiting.assign(c.wgs, 0);
        ticket = 0;
        pubs = 0;
        violations = 0;
        last_progress = 0;
        n = Counts{};
    }
};

#define YIELD co_yield 0

// One workgroup.  Statements between two YIELDs touch no shared word.
Proc workgroup(Model &m, uint32_t w) {
    const Config &c = m.c;
    const OpDef &op = m.op;
    const uint32_t N = m.N, G = c.G;
    const uint32_t groups = (N + G - 1u) / G;
    auto head = [&](uint32_t g) { return g < groups ? g * G : N; };
    uint32_t group;
    if (c.tickets) {
        YIELD;
        group = m.ticket++;
        m.progress();
    } else {
        group = w;
    }
    // the tiles of the pipeline, as the kernels' PipeTiles
    uint32_t prev2 = N, prev = N, cur = N, f1 = N, f2 = head(group);
    uint64_t incl_last = op.id();
    std::vector<uint32_t> sw(c.win);
    std::vector<uint64_t> val(c.win);
    for (;;) {
        // the tile after f2
        uint32_t after = N;
        if (f2 < N) {
            if ((f2 + 1u) % G != 0u) {
                after = f2 + 1u < N ? f2 + 1u : N;
            } else if (c.persistent) {
                if (c.tickets) {
                    YIELD;
                    group = m.ticket++;
                    m.progress();
                } else {
                    group += c.wgs;
                }
                after = head(group);
            }
        }
        // the closing step: nothing left to scan, so prev and cur are
        // resolved now as well, in order, after prev2
        const bool closing = c.close && f1 >= N && f2 >= N && cur < N;
        if (closing) m.n.closings++;
        for (int step = 0; step < (closing ? 3 : 1); ++step) {
            // broken=close_order resolves cur before prev
            const int r = (c.broken == "close_order" && step > 0) ? 3 - step : step;
            const uint32_t t = r == 0 ? prev2 : r == 1 ? prev : cur;
            const uint32_t nxt = r == 0 ? prev : r == 1 ? cur : f1;  // the workgroup's next tile
            // t: its exclusive prefix, by look-back or from the tile before
            const bool have = t < N && t != 0;
            const bool sp2 = have && op.self_prefix(m.agg[t]);
            const bool look = have && t % G == 0u && !(sp2 && m.first_start[t]);
            if (look && r > 0) m.n.closing_lookbacks++;
            uint64_t excl = op.id();
            bool known = t < N;
            if (look) {
                const uint64_t own = m.agg[t];
                const bool may_publish = !sp2;
                uint64_t acc = op.id();
                int64_t nearest = (int64_t)t - 1;
                uint32_t stalled = 0, walked = 0;
                long spins = 0;
                for (;;) {
                    const int64_t base = nearest - (int64_t)c.win + 1;
                    for (uint32_t j = 0; j < c.win; ++j) {
                        const int64_t i = base + (int64_t)j;
                        if (i < 0) {
                            sw[j] = ST_PREFIX;
                            val[j] = op.id();
                            continue;
                        }
                        YIELD;
                        uint32_t s0 = 0, s1 = 0;
                        const uint64_t r0 = m.load(w, m.word((uint32_t)i, 0), &s0);
                        uint64_t r1 = 0;
                        if (c.words == 2) {
                            YIELD;
                            r1 = m.load(w, m.word((uint32_t)i, 1), &s1);
                        }
                        const uint32_t a0 = m.seen_state(r0);
                        uint32_t st = a0;
                        uint64_t v = r0 & 0xFFFFFFFFu;
                        if (c.words == 2) {
                            const uint32_t a1 = m.seen_state(r1);
                            if (a0 != a1) {
                                m.n.torn++;
                                if (c.broken != "torn") st = ST_INVALID;
                            } else if (a0 != ST_INVALID && s0 != s1) {
                                m.n.mixed++;  // halves of two publications of one state word
                            }
                            v |= (r1 & 0xFFFFFFFFu) << 32;
                        }
                        if ((st & 3u) != ST_INVALID && !m.fact((uint32_t)i, st, v)) m.violation("false descriptor read", i, t);
                        sw[j] = st;
                        val[j] = v;
                    }
                    // the nearest PREFIX/PARTIAL word, and an INVALID one nearer than it
                    int js = -1, ji = -1;
                    for (int j = 0; j < (int)c.win; ++j)
                        if ((sw[j] & 3u) >= ST_PREFIX) js = j;
                    for (int j = js + 1; j < (int)c.win; ++j)
                        if ((sw[j] & 3u) == ST_INVALID) ji = j;
                    if (c.broken == "skip_invalid") ji = -1;
                    if (ji >= 0) {
                        m.n.stalls++;
                        m.waiting[w] = 1;
                        if (c.fallback && ++stalled >= c.fallback) {
                            // reduce the predecessor from its input, install over a word read as unpublished
                            m.waiting[w] = 0;
                            const uint32_t p = (uint32_t)(base + ji);
                            const bool pre = p == 0 || op.self_prefix(m.agg[p]);
                            const uint32_t dsw = pre ? ST_PREFIX : ST_AGGREGATE;
                            const uint64_t dv = pre ? m.incl[p] : m.agg[p];
                            const uint32_t pub = ++m.pubs;
                            m.n.fallbacks++;
                            for (int k = 0; k < c.words; ++k) {
                                YIELD;
                                const uint64_t old = m.load(w, m.word(p, k), nullptr);
                                if (state_seen((uint32_t)(old >> 32), m.tf) != ST_INVALID) {
                                    m.n.skipped_install++;
                                    continue;
                                }
                                YIELD;
                                if (m.cas(w, m.word(p, k), old, m.encode(dsw, dv, k), pub))
                                    m.n.cas_won++;
                                else
                                    m.n.cas_lost++;
                            }
                            stalled = 0;
                            continue;
                        }
                        if (++spins > 2000000) {
                            m.violation("spin limit", t, nearest);
                            break;
                        }
                        continue;
                    }
                    m.waiting[w] = 0;
                    stalled = 0;
                    spins = 0;
                    uint64_t f = op.id();
                    for (int j = js >= 0 ? js : 0; j < (int)c.win; ++j) f = op.op(f, val[j]);
                    acc = op.op(f, acc);
                    m.n.windows++;
                    if (js >= 0) {
                        if ((sw[js] & 3u) == ST_PREFIX) break;
                        uint32_t d = sw[js] >> kDistShift;
                        if (c.broken == "partial_distance") d -= 1u;
                        nearest = base + js - (int64_t)d;
                        m.n.partial_jumps++;
                    } else {
                        nearest = base - 1;
                    }
                    if (nearest < 0) break;
                    if (c.partial && ++walked >= c.partial && may_publish) {
                        const uint32_t psw = ((uint32_t)((int64_t)t - nearest) << kDistShift) | ST_PARTIAL;
                        const uint64_t pv = op.op(acc, own);
                        if (!m.fact(t, psw, pv)) m.violation("false PARTIAL published", t, nearest);
                        const uint32_t pub = ++m.pubs;
                        for (int k = 0; k < c.words; ++k) {
                            YIELD;
                            m.store(w, m.word(t, k), m.encode(psw, pv, k), pub);
                        }
                        m.n.partial_pubs++;
                    }
                }
                excl = acc;
            } else if (have && t % G != 0u) {
                excl = incl_last;  // the tile before, resolved a phase (or a moment) ago
            } else if (have) {
                known = false;  // a head whose first element starts a segment needs no carry
            }
            if (t < N) {
                if (known) {
                    m.result[t] = excl;
                    m.has_result[t] = 1;
                }
                if (have && !sp2) {
                    // its inclusive prefix (the second of a pair may have gone out a phase ago)
                    const bool early = c.pair && t % G != 0u && t - 1u != 0u;
                    const uint32_t pub = ++m.pubs;
                    const uint64_t p2 = op.op(excl, m.agg[t]);
                    if (!early)
                        for (int k = 0; k < c.words; ++k) {
                            YIELD;
                            m.store(w, m.word(t, k), m.encode(ST_PREFIX, p2, k), pub);
                        }
                    if (c.pair && look && nxt == t + 1u && nxt < N) {
                        const uint32_t pub2 = ++m.pubs;
                        const uint64_t p1 = op.op(p2, m.agg[nxt]);
                        for (int k = 0; k < c.words; ++k) {
                            YIELD;
                            m.store(w, m.word(nxt, k), m.encode(ST_PREFIX, p1, k), pub2);
                        }
                    }
                }
                incl_last = op.op(excl, m.agg[t]);
            }
        }
        // f1's aggregate (a tile with its own prefix publishes that)
        if (f1 < N) {
            const bool pre = f1 == 0 || op.self_prefix(m.agg[f1]);
            if (!(c.withhold && !pre)) {
                const uint32_t pub = ++m.pubs;
                for (int k = 0; k < c.words; ++k) {
                    YIELD;
                    m.store(w, m.word(f1, k), m.encode(pre ? ST_PREFIX : ST_AGGREGATE, pre ? m.incl[f1] : m.agg[f1], k),
                            pub);
                }
            }
        }
        if (closing || (prev2 >= N && prev >= N && cur >= N && f1 >= N && f2 >= N)) break;
        prev2 = prev;
        prev = cur;
        cur = f1;
        f1 = f2;
        f2 = f2 < N ? after : N;
    }
    m.progress();
}

// One schedule.  Returns "ok", "deadlock" or "violation".
std::string run_one(Model &m, uint64_t seed) {
    m.setup(seed);
    const Config &c = m.c;
    std::vector<uint32_t> pending(c.wgs);
    for (uint32_t i = 0; i < c.wgs; ++i) pending[i] = c.order == "desc" ? c.wgs - 1u - i : i;
    if (c.order == "random") std::shuffle(pending.begin(), pending.end(), m.rng);
    size_t next = 0;
    std::vector<uint32_t> res;   // resident workgroups
    std::vector<Proc> procs(c.wgs);
    std::vector<double> weight(c.wgs, 1.0);
    uint32_t finished = 0;
    std::string outcome = "ok";
    while (finished < c.wgs) {
        while (res.size() < c.resident && next < pending.size()) {
            const uint32_t w = pending[next++];
            procs[w] = workgroup(m, w);
            res.push_back(w);
        }
        if (m.n.steps % 4096 == 0)
            for (auto &x : weight) x = (m.rng() % 5 == 0) ? 0.01 : 1.0;  // starve some for a while
        double tot = 0;
        for (uint32_t w : res) tot += weight[w];
        double r = m.uni() * tot;
        size_t k = 0;
        for (; k + 1 < res.size(); ++k) {
            r -= weight[res[k]];
            if (r < 0) break;
        }
        const uint32_t w = res[k];
        procs[w].h.resume();
        m.n.steps++;
        if (procs[w].h.done()) {
            procs[w].h.destroy();
            procs[w].h = nullptr;
            res.erase(res.begin() + (long)k);
            ++finished;
        }
        if (m.violations) {
            outcome = "violation";
            break;
        }
        // no store, ticket or finish for a long time, and every resident one waits
        if (m.n.steps - m.last_progress > 400000) {
            bool all = true;
            for (uint32_t x : res) all = all && m.waiting[x];
            if (all) {
                m.n.deadlocks++;
                outcome = "deadlock";
                break;
            }
        }
    }
    for (auto &p : procs)
        if (p.h) p.h.destroy();
    if (outcome == "ok")
        for (uint32_t t = 0; t < m.N; ++t) {
            const uint64_t want = t ? m.incl[t - 1] : m.op.id();
            if (m.has_result[t] && m.result[t] != want) {
                m.violation("wrong exclusive prefix", t, 0);
                outcome = "violation";
            }
            const bool skipped = m.op.self_prefix(m.agg[t]) && m.first_start[t] && t % c.G == 0 && t != 0;
            if (!m.has_result[t] && !skipped) {
                m.violation("tile never resolved", t, 0);
                outcome = "violation";
            }
        }
    return outcome;
}

bool parse(Config &c, const char *a) {
    const char *eq = strchr(a, '=');
    if (!eq) return false;
    const std::string k(a, eq), v(eq + 1);
    const long x = atol(v.c_str());
    if (k == "words") c.words = (int)x;
    else if (k == "op") c.op = v == "affine32" ? OpKind::Affine32 : v == "segmented" ? OpKind::Segmented : OpKind::Affine16;
    else if (k == "tiles") c.tiles = (uint32_t)x;
    else if (k == "wgs") c.wgs = (uint32_t)x;
    else if (k == "resident") c.resident = (uint32_t)x;
    else if (k == "G") c.G = (uint32_t)x;
    else if (k == "win") c.win = (uint32_t)x;
    else if (k == "partial") c.partial = (uint32_t)x;
    else if (k == "fallback") c.fallback = (uint32_t)x;
    else if (k == "pair") c.pair = x != 0;
    else if (k == "persistent") c.persistent = x != 0;
    else if (k == "tickets") c.tickets = x != 0;
    else if (k == "withhold") c.withhold = x != 0;
    else if (k == "close") c.close = x != 0;
    else if (k == "order") c.order = v;
    else if (k == "p_fresh") c.p_fresh = atof(v.c_str());
    else if (k == "seed") c.seed = (uint64_t)x;
    else if (k == "seeds") c.seeds = (int)x;
    else if (k == "broken") c.broken = v;
    else if (k == "expect") c.expect = v;
    else return false;
    return true;
}

}  // namespace

int main(int argc, char **argv) {
    Model m;
    for (int i = 1; i < argc; ++i)
        if (!parse(m.c, argv[i])) {
            fprintf(stderr, "bad argument %s\n", argv[i]);
            return 2;
        }
    Config &c = m.c;
    if ((c.op == OpKind::Affine32) != (c.words == 2) || c.win == 0 || c.G == 0 || c.resident == 0 ||
        (c.persistent && !c.tickets && c.resident < c.wgs) ||
        (!c.persistent && c.wgs != (c.tiles + c.G - 1u) / c.G)) {
        fprintf(stderr, "unsupported configuration\n");
        return 2;
    }
    m.op = OpDef{c.op};
    Counts total;
    int ok = 0, dead = 0, bad = 0;
    for (int s = 0; s < c.seeds; ++s) {
        const std::string o = run_one(m, c.seed * 1000003ull + (uint64_t)s);
        total.add(m.n);
        ok += o == "ok";
        dead += o == "deadlock";
        bad += o == "violation";
    }
    printf("schedules %d: ok %d, deadlock %d, violation %d | steps %ld, loads %ld (stale %ld), words of "
           "earlier calls %ld, torn reads %ld, mixed reads %ld, stalls %ld, windows %ld, PARTIAL published %ld, "
           "PARTIAL jumps %ld, fallbacks %ld (installs won %ld, lost %ld, skipped %ld), closing steps %ld, "
           "closing lookbacks %ld\n",
           c.seeds, ok, dead, bad, total.steps, total.loads, total.stale, total.stale_tag, total.torn, total.mixed,
           total.stalls, total.windows, total.partial_pubs, total.partial_jumps, total.fallbacks, total.cas_won,
           total.cas_lost, total.skipped_install, total.closings, total.closing_lookbacks);
    if (c.expect == "ok") return (ok == c.seeds) ? 0 : 1;
    if (c.expect == "deadlock") return (dead == c.seeds) ? 0 : 1;
    return bad > 0 ? 0 : 1;  // expect=violation: a broken rule must be caught
}
