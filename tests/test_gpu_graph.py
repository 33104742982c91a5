"""Every entry point captured in a HIP graph (torch.cuda.CUDAGraph) and
replayed: the workspace reset is a fill kernel, not a memset node, and a call
launches nothing that a capture refuses.  Each replay runs with the program's
own eager calls (same entry point, same workspace, other data) and a
synchronization in between, and must give the eager result again: bit-exact
for integer work, within the oracle's tolerance for fp32 sums and the
recurrence (their grouping follows the look-back's timing)."""
import numpy as np
import pytest

import workloads as wl
from gpu_util import assert_f32_sum_close, assert_linrec_close, dev, host, require_gpu, say

pytestmark = pytest.mark.gpu

SENTINEL = -0x21524111  # 0xDEADBEEF as int32
REPLAYS = 3


@pytest.fixture(scope="module")
def dw():
    return require_gpu()


def _ws(dw, fn, *args):
    import torch
    return dw.new_workspace(dw.workspace_bytes(fn, *args))


def _capture(fn):
    """fn() captured once after a warm-up on a side stream (torch's recipe)."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def _replay_loop(g, outs, check, eager_other):
    import torch
    for r in range(REPLAYS):
        for o in outs:
            o.fill_(SENTINEL if o.dtype != torch.float32 else float("nan"))
        eager_other()          # eager work on the same workspace before the replay
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        check(r)


def _flat_u32_case(dw, fn_name, n, seed, call_kw=None):
    import torch
    fn = getattr(dw, fn_name)
    x = wl.full_range_u32(n, seed=seed)
    y = wl.full_range_u32(n, seed=seed + 1)
    dx, dy = dev(x), dev(y)
    out = torch.empty(n, dtype=torch.int32, device="cuda")
    other = torch.empty_like(out)
    tot = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = _ws(dw, fn_name, None, None, n, None, None)
    fn(dx, out, tot, workspace=ws)
    torch.cuda.synchronize()
    ref, ref_tot = host(out).copy(), int(host(tot)[0])
    fn(dy, other, workspace=ws)
    torch.cuda.synchronize()
    ref_other = host(other).copy()
    g = _capture(lambda: fn(dx, out, tot, workspace=ws))

    def eager():
        other.fill_(0)
        fn(dy, other, workspace=ws)

    def check(r):
        assert np.array_equal(host(out), ref), r
        assert int(host(tot)[0]) == ref_tot, r
        assert np.array_equal(host(other), ref_other), r
    _replay_loop(g, [out, tot], check, eager)
    return x, ref


@pytest.mark.parametrize("n", [70_001, (1 << 23) + 3])
def test_u32_exclusive(dw, orc, n):
    """Both forms behind the default entry point: two-level at 70 001
    elements, single-pass chained above 2^23."""
    say("graph u32 exclusive", n)
    x, ref = _flat_u32_case(dw, "ps_scan_exclusive_u32", n, seed=n + 300)
    assert np.array_equal(ref, orc.scan_u32(x, "sum", False)[0])


def test_generic_affine_single_pass(dw, orc):
    import torch
    n = 3_000_017
    x = wl.full_range_u32(n, seed=301) | np.uint32(0x00010000)
    y = wl.full_range_u32(n, seed=302) | np.uint32(0x00010000)
    dx, dy = dev(x), dev(y)
    out = torch.empty(n, dtype=torch.int32, device="cuda")
    other = torch.empty_like(out)
    ws = _ws(dw, "ps_scan_single_pass", dw.PS_OP_AFFINE16, dw.PS_U32, 1, None, None, n, None, None)
    say("graph affine16 single-pass")
    call = lambda: dw.ps_scan_single_pass("affine16", True, dx, out, workspace=ws)  # noqa: E731
    call()
    torch.cuda.synchronize()
    ref = orc.scan_u32(x, "affine16", True)[0]
    ref_other = orc.scan_u32(y, "affine16", True)[0]
    assert np.array_equal(host(out), ref)
    g = _capture(call)

    def eager():
        dw.ps_scan_single_pass("affine16", True, dy, other, workspace=ws)

    def check(r):
        assert np.array_equal(host(out), ref), r
        assert np.array_equal(host(other), ref_other), r
    _replay_loop(g, [out], check, eager)


def test_widening(dw, orc):
    import torch
    n = (1 << 23) + 3
    x = wl.full_range_u32(n, seed=303)
    dx = dev(x)
    out = torch.empty(n, dtype=torch.int64, device="cuda")
    other = torch.empty_like(out)
    ws = _ws(dw, "ps_scan_exclusive_u32_u64", None, None, n, None, None)
    say("graph widening")
    call = lambda: dw.ps_scan_exclusive_u32_u64(dx, out, workspace=ws)  # noqa: E731
    ref = orc.scan_u32_u64(x, False)[0]
    g = _capture(call)

    def eager():
        dw.ps_scan_inclusive_u32_u64(dx, other, workspace=ws)

    def check(r):
        assert np.array_equal(host(out).view(np.uint64), ref), r
        assert np.array_equal(host(other).view(np.uint64), orc.scan_u32_u64(x, True)[0]), r
    _replay_loop(g, [out], check, eager)


def test_f32_sum(dw, orc):
    import torch
    n = (1 << 23) + 3
    x = wl.normal_f32(n, seed=304)
    dx = dev(x)
    out = torch.empty(n, dtype=torch.float32, device="cuda")
    other = torch.empty_like(out)
    ws = _ws(dw, "ps_scan_inclusive_f32", None, None, n, None, None)
    ref, absprefix, _ = orc.scan_f32_sum(x, True)
    say("graph f32 sum")
    g = _capture(lambda: dw.ps_scan_inclusive_f32(dx, out, workspace=ws))

    def eager():
        dw.ps_scan_exclusive_f32(dx, other, workspace=ws)

    def check(r):
        assert_f32_sum_close(host(out), ref, absprefix, exclusive=False)
    _replay_loop(g, [out], check, eager)


def test_recurrence(dw, orc):
    import torch
    n = (1 << 23) + 3
    a, b = wl.linrec_pairs(n, seed=305, a_lo=-1.1, a_hi=1.1)
    da, db = dev(a), dev(b)
    oa = torch.empty(n, dtype=torch.float32, device="cuda")
    ob = torch.empty_like(oa)
    other = torch.empty_like(oa)
    ws = _ws(dw, "ps_scan_linrec_f32", None, None, None, None, n, 1, None, None)
    A, B, SA, SB, _ = orc.scan_linrec_f32(np.stack([a, b], 1), True)
    say("graph recurrence")
    g = _capture(lambda: dw.ps_scan_linrec_f32(da, db, ob, out_a=oa, inclusive=True, workspace=ws))

    def eager():
        dw.ps_scan_linrec_f32(da, db, other, inclusive=False, workspace=ws)

    def check(r):
        assert_linrec_close(host(oa), host(ob), A, B, SA, SB, False)
    _replay_loop(g, [oa, ob], check, eager)


def test_segmented(dw, orc):
    import torch
    n = (1 << 22) + 11
    x = wl.full_range_u32(n, seed=306)
    off = wl.random_segments(n, 40_000, seed=307, cover=False)
    off2 = wl.random_segments(n, 777, seed=308, cover=True)
    dx, doff, doff2 = dev(x), dev(off), dev(off2)
    out = torch.empty(n, dtype=torch.int32, device="cuda")
    other = torch.empty_like(out)
    ws = _ws(dw, "ps_segmented_scan_u32", None, n, None, off.size - 1, None, 0, None)
    ref = orc.segmented_scan_u32(x, off, False, sentinel=0xDEADBEEF)
    ref_other = orc.segmented_scan_u32(x, off2, True, sentinel=0xDEADBEEF)
    say("graph segmented")
    g = _capture(lambda: dw.ps_segmented_scan_u32(dx, doff, out, inclusive=False, workspace=ws))

    def eager():
        other.fill_(SENTINEL)
        dw.ps_segmented_scan_u32(dx, doff2, other, inclusive=True, workspace=ws)

    def check(r):
        assert np.array_equal(host(out).view(np.uint32), ref), r
        assert np.array_equal(host(other).view(np.uint32), ref_other), r
    _replay_loop(g, [out], check, eager)


@pytest.mark.parametrize("fn", ["ps_compact", "ps_compact_staged"])
def test_compaction(dw, orc, fn):
    import torch
    n = (1 << 20) + 3
    rec = wl.full_range_u32(4 * n, seed=309).reshape(n, 4)
    flags = wl.flag_pattern(n, "random", seed=310)
    flags2 = wl.flag_pattern(n, "clustered", seed=311, run=37)
    drec, dfl, dfl2 = dev(rec), dev(flags), dev(flags2)
    out = torch.empty_like(drec)
    other = torch.empty_like(drec)
    cnt = torch.zeros(1, dtype=torch.int64, device="cuda")
    cnt2 = torch.zeros(1, dtype=torch.int64, device="cuda")
    ws = _ws(dw, fn, None, 16, None, n, None, None, None)
    ref, ref_count = orc.compact(rec, flags)
    ref2, ref_count2 = orc.compact(rec, flags2)
    say("graph", fn)
    g = _capture(lambda: getattr(dw, fn)(drec, dfl, out, cnt, workspace=ws))

    def eager():
        getattr(dw, fn)(drec, dfl2, other, cnt2, workspace=ws)

    def check(r):
        c = int(host(cnt)[0])
        assert c == ref_count, r
        assert np.array_equal(host(out)[:c].view(np.uint32), ref[:c]), r
        c2 = int(host(cnt2)[0])
        assert c2 == ref_count2 and np.array_equal(host(other)[:c2].view(np.uint32), ref2[:c2]), r
    _replay_loop(g, [out, cnt], check, eager)
