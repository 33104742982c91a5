"""The look-back's safety valves, forced from the host: Decoupled Fallback
("GPUPrefixSums", section "Decoupled Fallback") after a single stalled poll,
and PARTIAL descriptors (the bounded-window variant of "Single-Pass Prefix
Scan with Decoupled Look-Back", section "Why the work stays linear").  Every
result must stay identical to the oracle's: a fallback installs exactly the
word the tile's owner would publish, and a PARTIAL covers exactly the tiles
it names."""
import contextlib

import numpy as np
import pytest

import workloads as wl
from gpu_util import (FLAT_TILE, TILE, assert_f32_sum_close, dev, filled_dev, host, require_gpu, say,
                      ws_error_word)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dw():
    return require_gpu()


@pytest.fixture(autouse=True, scope="module")
def _single_pass_only(dw):
    """Every call of this module runs the single-pass chained form, whatever
    its size (the two-level form has its own tests)."""
    old = dw.ps_small_n_config_get()
    dw.ps_small_n_config(0)
    yield
    dw.ps_small_n_config(old)


@contextlib.contextmanager
def lookback_config(dw, fallback_polls, partial):
    old = dw.ps_lookback_config_get()
    dw.ps_lookback_config(fallback_polls, partial)
    try:
        yield
    finally:
        dw.ps_lookback_config(*old)


def header(ws):
    """Workspace header words: ticket counter, error word, fallbacks, PARTIALs."""
    return host(ws[:16].clone()).view(np.uint32).astype(np.int64)


def _ws(dw, fn, *args):
    import torch
    return torch.empty(dw.workspace_bytes(fn, *args), dtype=torch.uint8, device="cuda")


def test_config_roundtrip(dw):
    with lookback_config(dw, 7, 2):
        assert dw.ps_lookback_config_get() == (7, 2)
    assert dw.ps_lookback_config_get() == (4096, 4)


@pytest.mark.parametrize("op", ["sum", "max", "min", "xor", "affine16"])
@pytest.mark.parametrize("inclusive", [False, True])
def test_flat_fallback_every_stall(dw, orc, op, inclusive):
    """A fallback after every stalled poll: the installed aggregates must be
    exact (AFFINE16 checks that the fallback folds in tile order)."""
    import torch
    n = 1400 * FLAT_TILE + 321
    x = wl.full_range_u32(n, seed=31)
    if op == "affine16":
        x = x | 0x00010000  # keep the multiplier odd, so products do not vanish
    d_in = dev(x)
    ws = _ws(dw, "ps_scan", 0, 0, 1, None, None, n, None, None)
    ref, ref_total = orc.scan_u32(x, op, inclusive)
    fallbacks = 0
    with lookback_config(dw, 1, 1):
        for rep in range(3):
            d_out = torch.empty_like(d_in)
            tot = torch.zeros(1, dtype=torch.int32, device="cuda")
            say("fallback flat", op, inclusive, rep)
            dw.ps_scan(op, inclusive, d_in, d_out, total=tot, workspace=ws)
            assert np.array_equal(host(d_out), ref), rep
            assert int(host(tot)[0]) == int(ref_total)
            h = header(ws)
            assert h[1] == 0
            fallbacks += int(h[2])
    say("fallbacks performed", fallbacks)


def test_flat_fallback_counts(dw, orc):
    """At 2^26 elements some look-backs stall; with a fallback after one stalled
    poll some of those stalls are resolved by a fallback, and the results stay
    exact."""
    import torch
    n = 1 << 26
    x = wl.uniform_u32(n, 256, seed=32)
    d_in = dev(x)
    ref, _ = orc.scan_u32(x, "sum", False)
    ws = _ws(dw, "ps_scan_exclusive_u32", None, None, n, None, None)
    total_fallbacks = 0
    with lookback_config(dw, 1, 1):
        for rep in range(5):
            d_out = torch.empty_like(d_in)
            say("fallback counts", rep)
            dw.ps_scan_exclusive_u32(d_in, d_out, workspace=ws)
            assert np.array_equal(host(d_out), ref), rep
            h = header(ws)
            assert h[1] == 0
            total_fallbacks += int(h[2])
    say("fallbacks performed", total_fallbacks)
    assert total_fallbacks > 0


def test_f32_fallback(dw, orc):
    import torch
    n = 700 * FLAT_TILE + 5
    x = wl.normal_f32(n, seed=33)
    d_in = torch.from_numpy(x).cuda()
    ref, absprefix, _ = orc.scan_f32_sum(x, True, want_abs=True)
    with lookback_config(dw, 1, 1):
        for rep in range(3):
            d_out = torch.empty_like(d_in)
            say("fallback f32", rep)
            dw.ps_scan_inclusive_f32(d_in, d_out)
            assert_f32_sum_close(d_out.cpu().numpy(), ref, absprefix, exclusive=False)
        mx = orc.scan_f32_minmax(x, "max", True)[0]
        d_out = torch.empty_like(d_in)
        dw.ps_scan("max", True, d_in, d_out)
        assert np.array_equal(d_out.cpu().numpy().view(np.uint32), mx.view(np.uint32))


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
        stats = torch.zeros(4 * tiles, dtype=torch.int32, device="cuda")
        d_out = torch.empty_like(d_in)
        say("partial walk", partial)
        dw.ps_lookback_stats_u32(d_in, d_out, stats, aggregate_only=True, workspace=ws)
        assert np.array_equal(host(d_out), ref)
        h = header(ws)
    st = host(stats).reshape(tiles, 4).astype(np.int64)
    t = np.arange(1, tiles)
    full_walk = (t + win - 1) // win
    say("windows per tile", partial, float(st[1:, 1].mean()), float(full_walk.mean()), int(h[3]))
    assert h[1] == 0
    if not partial:
        assert np.array_equal(st[1:, 1], full_walk) and h[3] == 0
    else:
        assert h[3] > 0
        assert st[1:, 1].sum() < 0.75 * full_walk.sum()


@pytest.mark.parametrize("inclusive", [False, True])
def test_segmented_fallback(dw, orc, inclusive):
    """Segmented scan with a fallback after every stalled poll: the fallback
    reduces (start flag, value) pairs and publishes PREFIX for tiles holding a
    start, AGGREGATE otherwise."""
    import torch
    values, off = wl.zipf_segments(n=1 << 24, num_segments=1 << 14, seed=35)
    long_n = 600 * TILE + 9
    lx = wl.full_range_u32(long_n, seed=36)
    loff = np.array([0, 5, 200 * TILE + 3, 450 * TILE, long_n], np.uint32)
    with lookback_config(dw, 1, 1):
        for x, o in ((values, off), (lx, loff)):
            ws = _ws(dw, "ps_segmented_scan_u32", None, x.size, None, o.size - 1, None, 0, None)
            ref = orc.segmented_scan_u32(x, o, inclusive, sentinel=0xDEADBEEF)
            for rep in range(2):
                d_out = filled_dev(x, 0xDEADBEEF)
                say("fallback segmented", x.size, inclusive, rep)
                dw.ps_segmented_scan_u32(dev(x), dev(o), d_out, inclusive=inclusive, workspace=ws)
                assert np.array_equal(host(d_out), ref), rep
                assert ws_error_word(ws) == 0


@pytest.mark.parametrize("width", [1, 4])
def test_compact_fallback(dw, orc, width):
    import torch
    n = (1 << 22) + 17
    rec = wl.full_range_u32(n * width, seed=37).reshape(n, width)
    if width == 1:
        rec = rec.reshape(n)
    flags = wl.flag_pattern(n, "random", seed=38)
    ref, ref_count = orc.compact(rec, flags, out=np.full_like(rec, 0xA5A5A5A5))
    with lookback_config(dw, 1, 1):
        for rep in range(2):
            d_out = dev(np.full_like(rec, 0xA5A5A5A5))
            cnt = torch.zeros(1, dtype=torch.int64, device="cuda")
            say("fallback compact", width, rep)
            dw.ps_compact(dev(rec), dev(flags), d_out, cnt)
            assert int(host(cnt)[0]) == ref_count
            assert np.array_equal(host(d_out), ref)
