"""The instrumented builds of the three single-pass kernels ("Single-Pass
Prefix Scan with Decoupled Look-Back", sections "Three states in a
per-block descriptor" and "Why the work stays linear": how many polls and
windows a look-back takes): their results are the ordinary entry points'
(checked against the oracle), and every statistics row is consistent --
tiles that do not look back show no polls, a looking tile polls at least
once per window, stalls never exceed polls, and every tile's scan phase was
timed."""
import numpy as np
import pytest

import workloads as wl
from gpu_util import FLAT_TILE, SEG_DATA_WAVES, TILE, assert_f32_sum_close, dev, filled_dev, host, require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dw():
    return require_gpu()


def _check_rows(st, looks, data_clock=False, arrivals=0):
    """st: (tiles, 16) rows (polls, windows, ticks, stalls, the phase timing
    of the tile's scan phase, the timeline, and word 15: for the flat kernels
    data wave 0's view of that phase, for the segmented kernel the data
    waves' arrivals at its first barrier); looks: which tiles look back;
    arrivals: the segmented kernel's data wave count."""
    polls, windows, stalls = st[:, 0], st[:, 1], st[:, 3]
    w15 = st[:, 15]
    if data_clock:
        # every tile was scanned in a phase that data wave 0 timed: to the
        # end of the scan (never 0 ticks), to the last store issued, to
        # barrier A (not before the stores)
        scanned, stored, at_a = w15 & 1023, (w15 >> 10) & 1023, (w15 >> 20) & 1023
        assert np.all(scanned > 0) and np.all(at_a >= stored) and np.all(w15 >> 30 == 0)
    elif arrivals:
        # the first data wave came no later than the last, which scanned its
        # span after the phase began (never 0 ticks; the first may read 0:
        # the control wave stamps its start of the phase after its own
        # bookkeeping at the barrier before), their indices name data waves
        first, last = w15 & 1023, (w15 >> 10) & 1023
        who_last, who_first = (w15 >> 20) & 15, (w15 >> 24) & 15
        assert np.all(last > 0) and np.all(first <= last) and np.all(w15 >> 28 == 0)
        assert np.all(who_last < arrivals) and np.all(who_first < arrivals)
        # the control wave saw every data wave arrive by the time it left
        # the barrier (a few ticks of slack for the counter's reads)
        assert np.all(last <= np.minimum(st[:, 4] + st[:, 5], 1023) + 5)
    else:
        assert np.all(w15 == 0)
    # every tile is scanned in exactly one phase, which both waves timed
    assert np.all(st[:, 4] + st[:, 5] > 0) and np.all(st[:, 6] + st[:, 7] > 0)
    # and no phase part takes longer than a millisecond
    assert np.all(st[:, 4:8] < 100_000)
    # every tile was stored in some phase, its workgroup started before it
    assert np.all(st[:, 9] != 0) and np.all(((st[:, 8] - st[:, 11]) & 0xFFFFFFFF) < 10_000_000)
    assert np.all(polls[~looks] == 0) and np.all(windows[~looks] == 0)
    assert np.all(polls[looks] >= 1) and np.all(windows[looks] >= 1)
    assert np.all(polls >= windows) and np.all(stalls <= polls)
    # polls that did not stall each closed a window
    assert np.all(polls - stalls == windows)


@pytest.mark.parametrize("op,dtype", [("sum", 0), ("sum", 1), ("max", 1)])
def test_flat_stats(dw, orc, op, dtype):
    import torch
    n = 900 * FLAT_TILE + 17
    tiles = dw.ps_lookback_tiles(n)
    stats = torch.zeros(dw.STATS_WORDS * tiles, dtype=torch.int32, device="cuda")
    if dtype == 0:
        x = wl.uniform_u32(n, 256, seed=701)
        d_out = torch.empty(n, dtype=torch.int32, device="cuda")
        say("flat stats u32", op)
        dw.ps_scan_lookback_stats(op, False, dev(x), d_out, stats)
        assert np.array_equal(host(d_out), orc.scan_u32(x, op, False)[0])
    else:
        x = wl.normal_f32(n, seed=702)
        d_out = torch.empty(n, dtype=torch.float32, device="cuda")
        say("flat stats f32", op)
        dw.ps_scan_lookback_stats(op, True, torch.from_numpy(x).cuda(), d_out, stats)
        got = host(d_out)
        if op == "sum":
            ref, absprefix, _ = orc.scan_f32_sum(x, True, want_abs=True)
            assert_f32_sum_close(got, ref, absprefix, exclusive=False)
        else:
            assert np.array_equal(got.view(np.uint32), orc.scan_f32_minmax(x, "max", True)[0].view(np.uint32))
    st = host(stats).reshape(tiles, dw.STATS_WORDS).astype(np.int64)
    t = np.arange(tiles)
    _check_rows(st, (t % dw.ps_lookback_group() == 0) & (t > 0), data_clock=True)


def test_segmented_stats(dw, orc):
    import torch
    values, off = wl.zipf_segments(n=1 << 24, num_segments=1 << 12, seed=703)
    n = values.size
    tiles = -(-n // TILE)
    stats = torch.zeros(dw.STATS_WORDS * tiles, dtype=torch.int32, device="cuda")
    d_out = filled_dev(values, 0xDEADBEEF)
    say("segmented stats")
    dw.ps_segmented_lookback_stats_u32(dev(values), dev(off), d_out, stats)
    assert np.array_equal(host(d_out), orc.segmented_scan_u32(values, off, False, sentinel=0xDEADBEEF))
    st = host(stats).reshape(tiles, dw.STATS_WORDS).astype(np.int64)
    # a tile looks back iff it heads a ticket group, is not tile 0, and its
    # first element does not start a segment
    first_is_start = np.zeros(tiles, bool)
    starts = off[:-1][off[:-1] < off[1:]]  # non-empty segments' first rows
    first_is_start[(starts[starts % TILE == 0] // TILE).astype(np.int64)] = True
    t = np.arange(tiles)
    looks = (t % 2 == 0) & (t > 0) & ~first_is_start
    assert looks.sum() > 100  # the giant segment spans many tiles
    _check_rows(st, looks, arrivals=SEG_DATA_WAVES)


def test_compact_stats(dw, orc):
    import torch
    rec, flags = wl.compaction_records(n=(1 << 22) + 5, seed=704)
    n = flags.size
    tiles = -(-n // dw.ps_compact_tile_records(16))
    stats = torch.zeros(dw.STATS_WORDS * tiles, dtype=torch.int32, device="cuda")
    d_out = torch.zeros_like(dev(rec))
    cnt = torch.zeros(1, dtype=torch.int64, device="cuda")
    say("compact stats")
    dw.ps_compact_lookback_stats(dev(rec), dev(flags), d_out, cnt, stats)
    ref, count = orc.compact(rec, flags)
    assert int(host(cnt)[0]) == count
    assert np.array_equal(host(d_out)[:count], ref[:count])
    st = host(stats).reshape(tiles, dw.STATS_WORDS).astype(np.int64)
    t = np.arange(tiles)
    _check_rows(st, (t % 2 == 0) & (t > 0))


@pytest.mark.parametrize("with_a", [False, True])
def test_linrec_stats(dw, with_a):
    """The instrumented recurrence gives the ordinary single-pass call's
    results bit for bit (the same arithmetic in the same order)."""
    import torch
    n = 700 * dw.ps_linrec_tile_elements() + 5
    a, b = wl.linrec_pairs(n=n, seed=705)
    da, db = dev(a), dev(b)
    tiles = -(-n // dw.ps_linrec_tile_elements())
    stats = torch.zeros(dw.STATS_WORDS * tiles, dtype=torch.int32, device="cuda")
    got_b = torch.empty(n, dtype=torch.float32, device="cuda")
    got_a = torch.empty(n, dtype=torch.float32, device="cuda") if with_a else None
    ref_b = torch.empty(n, dtype=torch.float32, device="cuda")
    ref_a = torch.empty(n, dtype=torch.float32, device="cuda") if with_a else None
    old = dw.ps_small_n_config_get()
    dw.ps_small_n_config(0)
    try:
        say("linrec stats", with_a)
        dw.ps_linrec_lookback_stats(da, db, got_b, stats, out_a=got_a)
        dw.ps_scan_linrec_f32(da, db, ref_b, out_a=ref_a)
    finally:
        dw.ps_small_n_config(old)
    assert np.array_equal(host(got_b).view(np.uint32), host(ref_b).view(np.uint32))
    if with_a:
        assert np.array_equal(host(got_a).view(np.uint32), host(ref_a).view(np.uint32))
    st = host(stats).reshape(tiles, dw.STATS_WORDS).astype(np.int64)
    t = np.arange(tiles)
    _check_rows(st, (t % dw.ps_lookback_group() == 0) & (t > 0), data_clock=True)


def test_stats_argument_errors(dw):
    import ctypes
    L = dw.lib()
    wsb = ctypes.c_size_t(1 << 20)
    fake = ctypes.c_void_p(0x10000000)
    # unsupported pairs and record widths are refused before anything runs
    assert L.ps_scan_lookback_stats(fake, ctypes.byref(wsb), 3, 0, 0, fake, fake, 1000, fake, None) == 5
    assert L.ps_compact_lookback_stats(fake, ctypes.byref(wsb), fake, 8, fake, 1000, fake, fake, fake, None) == 5
    # null stats
    assert L.ps_scan_lookback_stats(fake, ctypes.byref(wsb), 0, 0, 0, fake, fake, 1000, None, None) == 1
    assert L.ps_linrec_lookback_stats(fake, ctypes.byref(wsb), fake, fake, None, fake, 1000, 1, None, None) == 1
