"""The look-back's safety valves, forced from the host: Decoupled Fallback
("GPUPrefixSums", section "Decoupled Fallback") and PARTIAL descriptors (the
bounded-window variant of "Single-Pass Prefix Scan with Decoupled Look-Back",
section "Why the work stays linear").

A fallback only runs when a look-back stalls, and on a healthy chain stalls
are rare.  The fallback tests therefore withhold every AGGREGATE
(PS_DEBUG_WITHHOLD_AGGREGATES: a tile publishes only its inclusive PREFIX),
so that a look-back reaching a tile whose prefix is not yet known stalls
there, and set a fallback after every stalled poll, so that the fallback
supplies the withheld aggregate.  Each test asserts, from the workspace's
fallback counter, that fallbacks were installed, and that the results are
still the oracle's: a fallback installs exactly the word the tile's owner
would have published (for AFFINE16, whose operator does not commute, this
checks that the fallback folds in tile order)."""
import contextlib

import numpy as np
import pytest

import workloads as wl
from gpu_util import (FLAT_TILE, LINREC_TILE, TILE, assert_f32_sum_close, assert_linrec_close, dev, filled_dev,
                      host, require_gpu, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dw():
    return require_gpu()


@pytest.fixture(autouse=True, scope="module")
def _single_pass_only(dw):
    """Every call of this module runs the single-pass chained form, whatever
    its size (the two-level form has no look-back)."""
    old = dw.ps_small_n_config_get()
    dw.ps_small_n_config(0)
    yield
    dw.ps_small_n_config(old)


@contextlib.contextmanager
def lookback_config(dw, fallback_polls, partial, debug=0):
    old = dw.ps_lookback_config_get()
    old_debug = dw.ps_lookback_debug_get()
    dw.ps_lookback_config(fallback_polls, partial)
    dw.ps_lookback_debug(debug)
    try:
        yield
    finally:
        dw.ps_lookback_config(*old)
        dw.ps_lookback_debug(old_debug)


def forced_fallbacks(dw):
    """Aggregates withheld, a fallback after every stalled poll."""
    return lookback_config(dw, 1, 1, dw.PS_DEBUG_WITHHOLD_AGGREGATES)


def header(dw, ws):
    return dw.workspace_header(ws)


def _ws(dw, fn, *args):
    return dw.new_workspace(dw.workspace_bytes(fn, *args))


class FallbackCount:
    """Fallbacks installed in one workspace between two points (the
    counter is cumulative)."""

    def __init__(self, dw, ws):
        self.dw, self.ws = dw, ws
        self.start = header(dw, ws)[dw.PS_WS_FALLBACKS]

    def since(self):
        h = header(self.dw, self.ws)
        assert h[self.dw.PS_WS_ERROR] == 0, "workspace error bits %#x" % h[self.dw.PS_WS_ERROR]
        return h[self.dw.PS_WS_FALLBACKS] - self.start


def test_config_roundtrip(dw):
    with lookback_config(dw, 7, 2, dw.PS_DEBUG_WITHHOLD_AGGREGATES):
        assert dw.ps_lookback_config_get() == (7, 2)
        assert dw.ps_lookback_debug_get() == dw.PS_DEBUG_WITHHOLD_AGGREGATES
    assert dw.ps_lookback_config_get() == (4096, 4)
    assert dw.ps_lookback_debug_get() == 0
    with pytest.raises(dw.DwpsError):
        dw.ps_lookback_debug(2)


@pytest.mark.parametrize("op", ["sum", "max", "min", "and", "or", "xor", "affine16"])
@pytest.mark.parametrize("inclusive", [False, True])
def test_flat_fallback_every_op(dw, orc, op, inclusive):
    """Every u32 operator with its aggregates supplied by fallbacks."""
    import torch
    n = 700 * FLAT_TILE + 321
    x = wl.full_range_u32(n, seed=31)
    if op == "affine16":
        x = x | 0x00010000  # keep the multiplier odd, so products do not vanish
    if op in ("and", "or"):
        # sparse bits, so that the running AND / OR does not saturate at once
        x = x & wl.full_range_u32(n, seed=131) & wl.full_range_u32(n, seed=231)
        if op == "and":
            x = ~x
    d_in = dev(x)
    ws = _ws(dw, "ps_scan", 0, 0, 1, None, None, n, None, None)
    ref, ref_total = orc.scan_u32(x, op, inclusive)
    count = FallbackCount(dw, ws)
    with forced_fallbacks(dw):
        for rep in range(2):
            d_out = torch.empty_like(d_in)
            tot = torch.zeros(1, dtype=torch.int32, device="cuda")
            say("fallback flat", op, inclusive, rep)
            dw.ps_scan(op, inclusive, d_in, d_out, total=tot, workspace=ws)
            assert np.array_equal(host(d_out), ref), rep
            assert int(host(tot)[0]) == int(ref_total)
    installed = count.since()
    say("fallbacks installed", op, inclusive, installed)
    assert installed > 0


def test_flat_fallback_natural_stalls(dw, orc):
    """Without withheld aggregates, at 2^26 elements some look-backs still
    stall; with a fallback after one stalled poll some of those stalls are
    resolved by a fallback, and the results stay exact."""
    import torch
    n = 1 << 26
    x = wl.uniform_u32(n, 256, seed=32)
    d_in = dev(x)
    ref, _ = orc.scan_u32(x, "sum", False)
    ws = _ws(dw, "ps_scan_exclusive_u32", None, None, n, None, None)
    count = FallbackCount(dw, ws)
    with lookback_config(dw, 1, 1):
        for rep in range(5):
            d_out = torch.empty_like(d_in)
            say("natural stalls", rep)
            dw.ps_scan_exclusive_u32(d_in, d_out, workspace=ws)
            assert np.array_equal(host(d_out), ref), rep
    installed = count.since()
    say("fallbacks installed", installed)
    assert installed > 0


@pytest.mark.parametrize("inclusive", [False, True])
def test_f32_fallback(dw, orc, inclusive):
    """fp32 sum (a fallback's aggregate may round differently from the
    owner's; the sum stays within its bound) and max (exact)."""
    import torch
    n = 500 * FLAT_TILE + 5
    x = wl.normal_f32(n, seed=33)
    d_in = torch.from_numpy(x).cuda()
    ref, absprefix, _ = orc.scan_f32_sum(x, inclusive, want_abs=True)
    mx = orc.scan_f32_minmax(x, "max", inclusive)[0]
    ws = _ws(dw, "ps_scan", 0, 1, 1, None, None, n, None, None)
    with forced_fallbacks(dw):
        count = FallbackCount(dw, ws)
        d_out = torch.empty_like(d_in)
        say("fallback f32 sum", inclusive)
        dw.ps_scan("sum", inclusive, d_in, d_out, workspace=ws)
        assert_f32_sum_close(d_out.cpu().numpy(), ref, absprefix, exclusive=not inclusive)
        assert count.since() > 0
        count = FallbackCount(dw, ws)
        d_out = torch.empty_like(d_in)
        say("fallback f32 max", inclusive)
        dw.ps_scan("max", inclusive, d_in, d_out, workspace=ws)
        assert np.array_equal(d_out.cpu().numpy().view(np.uint32), mx.view(np.uint32))
        assert count.since() > 0


@pytest.mark.parametrize("inclusive", [False, True])
def test_u64_fallback(dw, orc, inclusive):
    """The widening scan's two-word descriptors, installed by fallbacks
    (each half by its own compare-and-swap)."""
    import torch
    n = 600 * dw.ps_tile_elements(dw.PS_U64) + 17
    x = wl.full_range_u32(n, seed=39)
    d_in = dev(x)
    ref, ref_total = orc.scan_u32_u64(x, inclusive)
    ws = _ws(dw, "ps_scan_exclusive_u32_u64", None, None, n, None, None)
    count = FallbackCount(dw, ws)
    with forced_fallbacks(dw):
        d_out = torch.empty(n, dtype=torch.int64, device="cuda")
        tot = torch.zeros(1, dtype=torch.int64, device="cuda")
        say("fallback u64", inclusive)
        f = dw.ps_scan_inclusive_u32_u64 if inclusive else dw.ps_scan_exclusive_u32_u64
        f(d_in, d_out, total=tot, workspace=ws)
        assert np.array_equal(host(d_out).view(np.uint64), ref)
        assert int(host(tot).view(np.uint64)[0]) == int(ref_total)
    assert count.since() > 0


def test_linrec_fallback(dw, orc):
    """The recurrence pair (two fp32 planes, two-word descriptors) with its
    aggregates from fallbacks: decays close to one keep A far from zero, so
    the fallback's A carry is checked at every index."""
    import torch
    n = 500 * LINREC_TILE + 3
    a, b = wl.linrec_pairs(n, seed=40, a_lo=1.0 - 2.0 ** -22, a_hi=1.0)
    A, B, SA, SB, _ = orc.scan_linrec_f32(np.stack([a, b], axis=1), True)
    ws = _ws(dw, "ps_scan_linrec_f32", None, None, None, None, n, 1, None, None)
    count = FallbackCount(dw, ws)
    with forced_fallbacks(dw):
        oa = torch.empty(n, dtype=torch.float32, device="cuda")
        ob = torch.empty(n, dtype=torch.float32, device="cuda")
        say("fallback linrec")
        dw.ps_scan_linrec_f32(dev(a), dev(b), ob, out_a=oa, inclusive=True, workspace=ws)
        assert_linrec_close(host(oa), host(ob), A, B, SA, SB, False)
    assert A[-1] > 0.5  # the A plane never approaches the absolute floor
    assert count.since() > 0


def test_no_fallback_chain_completes(dw, orc):
    """Aggregates withheld and no fallback: every look-back waits for its
    predecessor's inclusive prefix, so the prefixes complete one ticket group
    after another -- slower, still exact."""
    import torch
    n = 300 * FLAT_TILE + 11
    x = wl.full_range_u32(n, seed=41)
    ref, _ = orc.scan_u32(x, "sum", True)
    ws = _ws(dw, "ps_scan_inclusive_u32", None, None, n, None, None)
    count = FallbackCount(dw, ws)
    with lookback_config(dw, 0, 4, dw.PS_DEBUG_WITHHOLD_AGGREGATES):
        d_out = torch.empty(n, dtype=torch.int32, device="cuda")
        say("withheld aggregates, no fallback")
        dw.ps_scan_inclusive_u32(dev(x), d_out, workspace=ws)
        assert np.array_equal(host(d_out), ref)
    assert count.since() == 0


@pytest.mark.parametrize("partial", [0, 1, 3])
def test_partial_descriptors_bound_the_walk(dw, orc, partial):
    """With aggregate_only no tile after tile 0 ever publishes its inclusive
    prefix, so without PARTIALs every look-back walks its window back to
    tile 0; with PARTIALs (after 1 or 3 windows walked) later look-backs jump
    the covered stretches, and results stay exact."""
    import torch
    tile = dw.ps_tile_elements(0)
    n = 1100 * tile + 77
    x = wl.full_range_u32(n, seed=34)
    tiles = dw.ps_lookback_tiles(n)
    win = dw.ps_lookback_window()
    d_in = dev(x)
    ref, _ = orc.scan_u32(x, "sum", False)
    ws = _ws(dw, "ps_scan_exclusive_u32", None, None, n, None, None)
    with lookback_config(dw, 0, partial):
        stats = torch.zeros(dw.STATS_WORDS * tiles, dtype=torch.int32, device="cuda")
        d_out = torch.empty_like(d_in)
        say("partial walk", partial)
        dw.ps_lookback_stats_u32(d_in, d_out, stats, aggregate_only=True, workspace=ws)
        assert np.array_equal(host(d_out), ref)
        h = header(dw, ws)
    st = host(stats).reshape(tiles, dw.STATS_WORDS).astype(np.int64)
    t = np.arange(1, tiles)
    full_walk = (t + win - 1) // win
    say("windows per tile", partial, float(st[1:, 1].mean()), float(full_walk.mean()), h[dw.PS_WS_PARTIALS])
    assert h[dw.PS_WS_ERROR] == 0
    if not partial:
        assert np.array_equal(st[1:, 1], full_walk) and h[dw.PS_WS_PARTIALS] == 0
    else:
        assert h[dw.PS_WS_PARTIALS] > 0
        assert st[1:, 1].sum() < 0.75 * full_walk.sum()


@pytest.mark.parametrize("inclusive", [False, True])
def test_segmented_fallback(dw, orc, inclusive):
    """Segmented scan with its start-free tiles' aggregates from fallbacks:
    the fallback rebuilds the tile's start bitmap from the offsets, reduces
    (start flag, value) pairs and installs AGGREGATE (PREFIX for a tile that
    holds a start)."""
    values, off = wl.zipf_segments(n=1 << 24, num_segments=1 << 14, seed=35)
    long_n = 600 * TILE + 9
    lx = wl.full_range_u32(long_n, seed=36)
    loff = np.array([0, 5, 200 * TILE + 3, 450 * TILE, long_n], np.uint32)
    for x, o in ((values, off), (lx, loff)):
        ws = _ws(dw, "ps_segmented_scan_u32", None, x.size, None, o.size - 1, None, 0, None)
        ref = orc.segmented_scan_u32(x, o, inclusive, sentinel=0xDEADBEEF)
        count = FallbackCount(dw, ws)
        with forced_fallbacks(dw):
            d_out = filled_dev(x, 0xDEADBEEF)
            say("fallback segmented", x.size, inclusive)
            dw.ps_segmented_scan_u32(dev(x), dev(o), d_out, inclusive=inclusive, workspace=ws)
            assert np.array_equal(host(d_out), ref)
        installed = count.since()
        say("fallbacks installed", installed)
        assert installed > 0


@pytest.mark.parametrize("width", [1, 2, 4])
def test_compact_fallback(dw, orc, width):
    """Compaction of 4-, 8- and 16-byte records with the tile counts from
    fallbacks (the fallback counts the tile's keep flags itself)."""
    import torch
    n = (1 << 22) + 17
    rec = wl.full_range_u32(n * width, seed=37).reshape(n, width)
    if width == 1:
        rec = rec.reshape(n)
    flags = wl.flag_pattern(n, "random", seed=38)
    ref, ref_count = orc.compact(rec, flags, out=np.full_like(rec, 0xA5A5A5A5))
    ws = _ws(dw, "ps_compact", None, 4 * width, None, n, None, None, None)
    count = FallbackCount(dw, ws)
    with forced_fallbacks(dw):
        d_out = dev(np.full_like(rec, 0xA5A5A5A5))
        cnt = torch.zeros(1, dtype=torch.int64, device="cuda")
        say("fallback compact", width)
        dw.ps_compact(dev(rec), dev(flags), d_out, cnt, workspace=ws)
        assert int(host(cnt)[0]) == ref_count
        assert np.array_equal(host(d_out), ref)
    installed = count.since()
    say("fallbacks installed", installed)
    assert installed > 0
