"""The prepared workspace that keeps itself ready between calls: one launch
per call, with descriptors tagged by their call ("Single-Pass Prefix Scan
with Decoupled Look-Back", section "Three states in a per-block
descriptor": a slot starts out invalid, and a word left by another call is
read as invalid).  Every result is compared with the oracle."""
import ctypes

import numpy as np
import pytest

import workloads as wl
from gpu_util import FLAT_TILE, assert_linrec_close, dev, filled_dev, host, require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dw():
    return require_gpu()


def _flat_ws(dw, n):
    return dw.new_workspace(dw.workspace_bytes("ps_scan_single_pass", 0, 0, 0, None, None, n, None, None))


def _single(dw, x, ws, inclusive=False):
    import torch
    d_out = torch.empty(x.size, dtype=torch.int32, device="cuda")
    dw.ps_scan_single_pass("sum", inclusive, dev(x), d_out, workspace=ws)
    return host(d_out)


def test_prepared_header(dw):
    import torch
    ws = dw.new_workspace(4096)
    torch.cuda.synchronize()
    h = dw.workspace_header(ws)
    cap = (4096 - dw.PS_WS_HEADER_BYTES) // 8
    assert h[dw.PS_WS_MAGIC] == 0x44575053
    assert h[dw.PS_WS_CAPACITY] == cap
    assert (h[dw.PS_WS_DIRTY_LO], h[dw.PS_WS_DIRTY_HI]) == (0, cap)
    for w in (dw.PS_WS_TICKET, dw.PS_WS_ERROR, dw.PS_WS_TAG, dw.PS_WS_DONE, dw.PS_WS_HIGH, dw.PS_WS_READY,
              dw.PS_WS_CALLS):
        assert h[w] == 0, w


def test_header_after_calls(dw, orc):
    """After each single-pass call: no ticket or completion count left over,
    the tag advanced by one, the words the call used no longer dirty."""
    n = 37 * FLAT_TILE + 5
    ws = _flat_ws(dw, n)
    x = wl.full_range_u32(n, seed=501)
    ref, _ = orc.scan_u32(x, "sum", False)
    tiles = dw.ps_lookback_tiles(n)
    for call in range(3):
        assert np.array_equal(_single(dw, x, ws), ref), call
        h = dw.workspace_header(ws)
        assert h[dw.PS_WS_TICKET] == 0 and h[dw.PS_WS_DONE] == 0 and h[dw.PS_WS_READY] == 0
        assert h[dw.PS_WS_TAG] == call + 1 and h[dw.PS_WS_CALLS] == call + 1
        assert h[dw.PS_WS_HIGH] == tiles
        assert h[dw.PS_WS_DIRTY_LO] >= tiles or h[dw.PS_WS_DIRTY_LO] == h[dw.PS_WS_DIRTY_HI]
        assert h[dw.PS_WS_ERROR] == 0


def test_tag_wrap(dw, orc):
    """A large call, 511 small ones, then another large call with the same
    tag as the first: the first call's words past the small calls' reach
    carry that tag again, and must have been zeroed (the wrap marks every
    tagged word dirty) -- else the second call would read the first call's
    prefixes of a different input."""
    big = 40 * FLAT_TILE + 3
    small = FLAT_TILE // 2
    ws = _flat_ws(dw, big)
    xa = wl.full_range_u32(big, seed=502)
    xb = wl.full_range_u32(big, seed=503)
    xs = wl.full_range_u32(small, seed=504)
    ref_a, _ = orc.scan_u32(xa, "sum", True)
    ref_b, _ = orc.scan_u32(xb, "sum", True)
    ref_s, _ = orc.scan_u32(xs, "sum", True)
    say("tag wrap: first large call")
    assert np.array_equal(_single(dw, xa, ws, True), ref_a)
    import torch
    d_s = dev(xs)
    d_out = torch.empty(small, dtype=torch.int32, device="cuda")
    say("tag wrap: 511 small calls")
    for _ in range(511):
        dw.ps_scan_single_pass("sum", True, d_s, d_out, workspace=ws)
    assert np.array_equal(host(d_out), ref_s)
    h = dw.workspace_header(ws)
    assert h[dw.PS_WS_TAG] == 0 and h[dw.PS_WS_CALLS] == 512
    say("tag wrap: second large call, same tag as the first")
    assert np.array_equal(_single(dw, xb, ws, True), ref_b)
    h = dw.workspace_header(ws)
    assert h[dw.PS_WS_TAG] == 1 and h[dw.PS_WS_ERROR] == 0


def test_one_workspace_every_entry_point(dw, orc):
    """One workspace, sized for the largest call, serves flat scans of both
    widths, the recurrence, the segmented scan, both compactions and the
    two-level form in turn, sizes going up and down."""
    import torch
    n = 60 * FLAT_TILE + 9
    need = max(dw.workspace_bytes("ps_scan_single_pass", 0, 0, 0, None, None, n, None, None),
               dw.workspace_bytes("ps_scan_exclusive_u32_u64", None, None, n, None, None),
               dw.workspace_bytes("ps_scan_linrec_f32", None, None, None, None, n, 1, None, None),
               dw.workspace_bytes("ps_segmented_scan_u32", None, n, None, 1000, None, 0, None),
               dw.workspace_bytes("ps_compact", None, 16, None, n, None, None, None),
               dw.workspace_bytes("ps_compact_staged", None, 16, None, n, None, None, None))
    ws = dw.new_workspace(need)
    old = dw.ps_small_n_config_get()
    dw.ps_small_n_config(0)
    try:
        for rnd, m in enumerate((n, n // 3, n, 5 * FLAT_TILE)):
            x = wl.full_range_u32(m, seed=510 + rnd)
            ref, _ = orc.scan_u32(x, "max", False)
            d_out = torch.empty(m, dtype=torch.int32, device="cuda")
            say("every entry point: flat", rnd, m)
            dw.ps_scan("max", False, dev(x), d_out, workspace=ws)
            assert np.array_equal(host(d_out), ref)

            ref64, _ = orc.scan_u32_u64(x, True)
            d64 = torch.empty(m, dtype=torch.int64, device="cuda")
            say("every entry point: widening", rnd)
            dw.ps_scan_inclusive_u32_u64(dev(x), d64, workspace=ws)
            assert np.array_equal(host(d64).view(np.uint64), ref64)

            vals = wl.full_range_u32(m, seed=520 + rnd)
            off = wl.random_segments(m, 1000, seed=520 + rnd)
            ref_s = orc.segmented_scan_u32(vals, off, False, sentinel=7)
            d_s = filled_dev(vals, 7)
            say("every entry point: segmented", rnd)
            dw.ps_segmented_scan_u32(dev(vals), dev(off), d_s, workspace=ws)
            assert np.array_equal(host(d_s), ref_s)

            rec = wl.full_range_u32(4 * m, seed=530 + rnd).reshape(m, 4)
            flags = wl.flag_pattern(m, "random", seed=540 + rnd)
            ref_c, ref_count = orc.compact(rec, flags)
            for fn in ("ps_compact_staged", "ps_compact"):
                d_c = torch.zeros(m, 4, dtype=torch.int32, device="cuda")
                cnt = torch.zeros(1, dtype=torch.int64, device="cuda")
                say("every entry point:", fn, rnd)
                getattr(dw, fn)(dev(rec), dev(flags), d_c, cnt, workspace=ws)
                assert int(host(cnt)[0]) == ref_count
                assert np.array_equal(host(d_c)[:ref_count], ref_c[:ref_count])

            a, b = wl.linrec_pairs(m, seed=545 + rnd)
            A, B, SA, SB, _ = orc.scan_linrec_f32(np.stack([a, b], axis=1), True)
            oa = torch.empty(m, dtype=torch.float32, device="cuda")
            ob = torch.empty(m, dtype=torch.float32, device="cuda")
            say("every entry point: recurrence", rnd)
            dw.ps_scan_linrec_f32(dev(a), dev(b), ob, out_a=oa, inclusive=True, workspace=ws)
            assert_linrec_close(host(oa), host(ob), A, B, SA, SB, False)

            d_t = torch.empty(m, dtype=torch.int32, device="cuda")
            say("every entry point: two-level", rnd)
            dw.ps_scan_two_level("max", False, dev(x), d_t, workspace=ws)
            assert np.array_equal(host(d_t), ref)
        assert dw.workspace_header(ws)[dw.PS_WS_ERROR] == 0
    finally:
        dw.ps_small_n_config(old)


def test_staged_offsets_are_cleaned(dw, orc):
    """The staged compaction leaves its offsets in descriptor words and marks
    them dirty; a later single-pass call whose descriptors reach into them
    (the widening scan: two words per tile of half the size) zeroes them
    first.  With every flag set, offset i is i, so the words hold every
    state and tag bit pattern in turn."""
    import torch
    m = 500 * FLAT_TILE
    ws = dw.new_workspace(max(dw.workspace_bytes("ps_compact_staged", None, 4, None, m, None, None, None),
                              dw.workspace_bytes("ps_scan_exclusive_u32_u64", None, None, m, None, None)))
    old = dw.ps_small_n_config_get()
    dw.ps_small_n_config(0)
    try:
        x = wl.full_range_u32(m, seed=551)
        ref, _ = orc.scan_u32_u64(x, False)
        d64 = torch.empty(m, dtype=torch.int64, device="cuda")
        words = 2 * (m // dw.ps_tile_elements(dw.PS_U64))
        # first the widening scan alone: its words are clean afterwards
        dw.ps_scan_exclusive_u32_u64(dev(x), d64, workspace=ws)
        assert np.array_equal(host(d64).view(np.uint64), ref)
        assert dw.workspace_header(ws)[dw.PS_WS_DIRTY_LO] >= words
        rec = wl.full_range_u32(m, seed=550)
        flags = np.ones(m, np.uint8)
        d_c = torch.zeros(m, dtype=torch.int32, device="cuda")
        cnt = torch.zeros(1, dtype=torch.int64, device="cuda")
        say("staged compaction, then the widening scan")
        dw.ps_compact_staged(dev(rec), dev(flags), d_c, cnt, workspace=ws)
        assert int(host(cnt)[0]) == m
        assert np.array_equal(host(d_c), rec)
        # the offsets made part of the widening scan's words dirty again
        h = dw.workspace_header(ws)
        assert h[dw.PS_WS_DIRTY_LO] < words < h[dw.PS_WS_DIRTY_HI]
        d64.fill_(0)
        dw.ps_scan_exclusive_u32_u64(dev(x), d64, workspace=ws)
        assert np.array_equal(host(d64).view(np.uint64), ref)
        assert dw.workspace_header(ws)[dw.PS_WS_ERROR] == 0
    finally:
        dw.ps_small_n_config(old)


def test_unprepared_workspace_computes_nothing(dw):
    """A zero-filled (never prepared) workspace: the kernel raises
    PS_WS_ERR_NOT_PREPARED and writes no output."""
    import torch
    n = 10 * FLAT_TILE
    ws = torch.zeros(dw.workspace_bytes("ps_scan_single_pass", 0, 0, 0, None, None, n, None, None),
                     dtype=torch.uint8, device="cuda")
    x = wl.full_range_u32(n, seed=560)
    d_out = filled_dev(x, 0x5A5A5A5A)
    say("unprepared workspace")
    dw.ps_scan_single_pass("sum", False, dev(x), d_out, workspace=ws)
    assert np.all(host(d_out) == 0x5A5A5A5A)
    assert dw.workspace_header(ws)[dw.PS_WS_ERROR] == dw.PS_WS_ERR_NOT_PREPARED


def test_capacity_checked_on_the_device(dw):
    """A workspace prepared smaller than a later call claims it is: the
    kernel raises PS_WS_ERR_CAPACITY and writes nothing."""
    import torch
    n = 10 * FLAT_TILE
    need = dw.workspace_bytes("ps_scan_single_pass", 0, 0, 0, None, None, n, None, None)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    L = dw.lib()
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert L.ps_workspace_init(ctypes.c_void_p(ws.data_ptr()), dw.PS_WS_HEADER_BYTES + 8, s) == 0
    x = wl.full_range_u32(n, seed=561)
    d_out = filled_dev(x, 0x5A5A5A5A)
    say("capacity too small")
    dw.ps_scan_single_pass("sum", False, dev(x), d_out, workspace=ws)
    assert np.all(host(d_out) == 0x5A5A5A5A)
    assert dw.workspace_header(ws)[dw.PS_WS_ERROR] == dw.PS_WS_ERR_CAPACITY


def test_init_argument_errors(dw):
    import torch
    L = dw.lib()
    ws = torch.empty(1024, dtype=torch.uint8, device="cuda")
    assert L.ps_workspace_init(None, 1024, None) == 1                            # PS_ERR_NULL
    assert L.ps_workspace_init(ctypes.c_void_p(ws.data_ptr() + 4), 512, None) == 7  # PS_ERR_ALIGNMENT
    assert L.ps_workspace_init(ctypes.c_void_p(ws.data_ptr()), 255, None) == 4   # PS_ERR_WORKSPACE


def test_cached_workspace_on_another_stream(dw, orc):
    """A call on a non-current stream without a workspace uses the one kept
    for that stream, allocated on it: a same-size allocation on the default
    stream right after the call, filled at once, must not land on the
    workspace while the scan still uses it."""
    import torch
    n = (1 << 24) + 11
    x = wl.full_range_u32(n, seed=562)
    ref, _ = orc.scan_u32(x, "sum", True)
    d_in = dev(x)
    s = torch.cuda.Stream()
    d_out = torch.empty_like(d_in)
    torch.cuda.synchronize()
    old = dw.ps_small_n_config_get()
    dw.ps_small_n_config(0)
    try:
        for rep in range(3):
            say("cached workspace on a side stream", rep)
            dw.ps_scan_inclusive_u32(d_in, d_out, stream=s)
            need = dw.workspace_bytes("ps_scan_inclusive_u32", None, None, n, None, None)
            junk = torch.empty(need, dtype=torch.uint8, device="cuda")
            junk.fill_(0xFF)
            s.synchronize()
            assert np.array_equal(host(d_out), ref), rep
            del junk
    finally:
        dw.ps_small_n_config(old)
