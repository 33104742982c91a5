"""Parity of the widening uint32 -> uint64 sum scan (HIP, through the C ABI)
with the oracle: bit-exact 64-bit sums, no wrap below 2^64."""
import numpy as np
import pytest

import workloads as wl
from gpu_util import dev, host, require_gpu, say, ws_error_word
from pins import golden

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


def _run(dw, x, inclusive, workspace=None):
    import torch
    d_in = dev(x)
    d_out = torch.full((x.size,), -1, dtype=torch.int64, device="cuda")
    tot = torch.full((1,), -1, dtype=torch.int64, device="cuda")
    f = dw.ps_scan_inclusive_u32_u64 if inclusive else dw.ps_scan_exclusive_u32_u64
    f(d_in, d_out, total=tot, workspace=workspace)
    return d_out.cpu().numpy().view(np.uint64), int(tot.cpu().numpy().view(np.uint64)[0])


def _check(dw, orc, x, inclusive):
    got, total = _run(dw, x, inclusive)
    ref, ref_total = orc.scan_u32_u64(x, inclusive)
    if not np.array_equal(got, ref):
        bad = np.nonzero(got != ref)[0]
        raise AssertionError("%d elements differ, first %d: gpu %d oracle %d"
                             % (bad.size, bad[0], got[bad[0]], ref[bad[0]]))
    assert total == ref_total


def test_tile_shape(dw):
    assert dw.ps_tile_elements(dw.PS_U64) == 6144


def test_worked_examples(dw):
    for name in ("p1_lead_scan.json", "p3_inclusive_exclusive.json", "p5_flat_example.json"):
        g = golden(name)
        x = np.array(g["input"], np.uint32)
        say("u64 worked example", name)
        assert _run(dw, x, False)[0].tolist() == g["exclusive"]
        assert _run(dw, x, True)[0].tolist() == g["inclusive"]


WT = 6144
EDGE = [1, 2, 3, 4, 5, 63, 64, 65, 255, 256, 257, 1023, 1024, 1025, WT - 1, WT, WT + 1, 2 * WT - 1, 2 * WT,
        2 * WT + 1, 3 * WT + 7, 257 * WT, 513 * WT + 1, 1_000_003]


@pytest.mark.parametrize("n", EDGE)
@pytest.mark.parametrize("inclusive", [False, True])
def test_edge_sizes_full_range(dw, orc, n, inclusive):
    """Full-range inputs: the running sum passes 2^32 after a few elements, so
    every carry into the high word is checked."""
    x = wl.full_range_u32(n, seed=n + 11)
    say("u64 edge", n, inclusive)
    _check(dw, orc, x, inclusive)


def test_empty_writes_total(dw):
    import torch
    tot = torch.full((1,), -1, dtype=torch.int64, device="cuda")
    d = torch.empty(0, dtype=torch.int32, device="cuda")
    o = torch.empty(0, dtype=torch.int64, device="cuda")
    dw.ps_scan_exclusive_u32_u64(d, o, total=tot)
    assert int(tot.cpu()[0]) == 0


@pytest.mark.parametrize("inclusive", [False, True])
def test_unaligned_buffers(dw, orc, inclusive):
    """Input one element past a 16-byte boundary, output 8 bytes past one: the
    per-element path."""
    import torch
    n = 7 * WT + 13
    x = wl.full_range_u32(n, seed=77)
    vx = dev(np.concatenate(([0], x)).astype(np.uint32))[1:]
    vo = torch.full((n + 1,), -1, dtype=torch.int64, device="cuda")[1:]
    assert vx.data_ptr() % 16 != 0 and vo.data_ptr() % 16 != 0
    say("u64 unaligned", inclusive)
    f = dw.ps_scan_inclusive_u32_u64 if inclusive else dw.ps_scan_exclusive_u32_u64
    f(vx, vo)
    ref, _ = orc.scan_u32_u64(x, inclusive)
    assert np.array_equal(vo.cpu().numpy().view(np.uint64), ref)


def test_generic_entry_point(dw, orc):
    import torch
    n = 50 * WT + 3
    x = wl.full_range_u32(n, seed=78)
    out = torch.empty(n, dtype=torch.int64, device="cuda")
    dw.ps_scan("sum", True, dev(x), out, dtype=dw.PS_U64)
    ref, _ = orc.scan_u32_u64(x, True)
    assert np.array_equal(out.cpu().numpy().view(np.uint64), ref)


def test_repeated_runs_reuse_workspace(dw, orc):
    import torch
    n = 1 << 24
    x = wl.full_range_u32(n, seed=79)
    ws = dw.new_workspace(dw.workspace_bytes("ps_scan_exclusive_u32_u64", None, None, n, None, None))
    ref, ref_total = orc.scan_u32_u64(x, False)
    for it in range(10):
        say("u64 repeat", it)
        got, total = _run(dw, x, False, workspace=ws)
        assert np.array_equal(got, ref) and total == ref_total, it
        assert ws_error_word(ws) == 0


def test_fallback_every_stall(dw, orc):
    """A fallback after every stalled poll installs both descriptor words."""
    import torch
    n = (1 << 25) + 5
    x = wl.full_range_u32(n, seed=80)
    ws = dw.new_workspace(dw.workspace_bytes("ps_scan_exclusive_u32_u64", None, None, n, None, None))
    ref, _ = orc.scan_u32_u64(x, False)
    old = dw.ps_lookback_config_get()
    dw.ps_lookback_config(1, 1)
    try:
        for rep in range(3):
            say("u64 fallback", rep)
            got, _ = _run(dw, x, False, workspace=ws)
            assert np.array_equal(got, ref), rep
            assert ws_error_word(ws) == 0
    finally:
        dw.ps_lookback_config(*old)


@pytest.mark.parametrize("inclusive", [False, True])
def test_large_config(dw, orc, inclusive):
    """2^28 values in [0, 255]: the 32-bit scan wraps about 8 times, the
    widening scan must not (total ~ 3.4e10)."""
    x = wl.large_u32()
    say("u64 config 2^28", inclusive)
    got, total = _run(dw, x, inclusive)
    ref, ref_total = orc.scan_u32_u64(x, inclusive)
    assert total == ref_total and ref_total > (1 << 32)
    assert np.array_equal(got, ref)
