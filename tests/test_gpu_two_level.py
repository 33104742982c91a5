"""Parity of the two-level (reduce-then-scan) scan with the oracle, in its
three forms: one tile (one launch), up to 1024 tiles (tile totals, then a
scan pass that folds the earlier totals itself), more (tile totals, a
one-workgroup scan of them, the scan pass).  Integer results bit-exact, fp32
sums within 1e-5 * sum |x|, fp32 max/min bit-exact."""
import numpy as np
import pytest

import workloads as wl
from gpu_util import assert_f32_sum_close, dev, host, require_gpu, say

pytestmark = pytest.mark.gpu

TT = 4096          # elements per tile of the two-level passes
FOLD_MAX = 1024    # tiles up to which the scan pass folds the totals itself
SIZES = [1, 2, 5, 255, 1023, TT - 1, TT, TT + 1, 2 * TT + 3, 63 * TT + 1, FOLD_MAX * TT - 7, FOLD_MAX * TT,
         FOLD_MAX * TT + 1, 3000 * TT + 77]
U32_OPS = ["sum", "max", "min", "and", "or", "xor", "affine16"]


@pytest.fixture(scope="module")
def dw():
    return require_gpu()


def _run(dw, x, op, inclusive, dtype=None, out_dtype=None):
    import torch
    d_in = dev(x)
    out_dtype = out_dtype or d_in.dtype
    d_out = torch.full((x.size,), -1, dtype=out_dtype, device="cuda")
    tot = torch.full((1,), -1, dtype=out_dtype, device="cuda")
    dw.ps_scan_two_level(op, inclusive, d_in, d_out, tot, dtype=dtype)
    return host(d_out), host(tot)[0]


def test_tile_shape(dw):
    assert dw.ps_two_level_tile_elements() == TT


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("inclusive", [False, True])
def test_u32_sum_sizes(dw, orc, n, inclusive):
    x = wl.full_range_u32(n, seed=n + 5)
    say("two-level u32 sum", n, inclusive)
    got, total = _run(dw, x, "sum", inclusive)
    ref, ref_total = orc.scan_u32(x, "sum", inclusive)
    assert np.array_equal(got, ref)
    assert int(total) == ref_total


@pytest.mark.parametrize("op", U32_OPS)
@pytest.mark.parametrize("n", [3 * TT + 11, 700 * TT + 5, 1500 * TT + 3])
@pytest.mark.parametrize("inclusive", [False, True])
def test_u32_all_operators(dw, orc, op, n, inclusive):
    """AFFINE16 is not commutative: every fold, the totals' included, must
    keep index order."""
    x = wl.full_range_u32(n, seed=n + 6)
    if op == "affine16":
        x = x | 0x00010000
    say("two-level", op, n, inclusive)
    got, total = _run(dw, x, op, inclusive)
    ref, ref_total = orc.scan_u32(x, op, inclusive)
    assert np.array_equal(got, ref), op
    assert int(total) == ref_total


@pytest.mark.parametrize("n", [33, TT + 1, 500 * TT + 9, 2000 * TT + 1])
@pytest.mark.parametrize("inclusive", [False, True])
def test_f32_sum_tolerance(dw, orc, n, inclusive):
    x = wl.normal_f32(n, seed=n + 7)
    say("two-level f32 sum", n, inclusive)
    got, total = _run(dw, x, "sum", inclusive)
    ref, absprefix, ref_total = orc.scan_f32_sum(x, inclusive)
    assert_f32_sum_close(got, ref, absprefix, exclusive=not inclusive)
    assert abs(float(total) - ref_total) <= 1e-5 * float(np.abs(x.astype(np.float64)).sum())


@pytest.mark.parametrize("op", ["max", "min"])
@pytest.mark.parametrize("n", [5, 900 * TT + 3, 1100 * TT + 3])
def test_f32_minmax_bit_exact(dw, orc, op, n):
    x = wl.normal_f32(n, seed=n + 8)
    say("two-level f32", op, n)
    got, total = _run(dw, x, op, True)
    ref, ref_total = orc.scan_f32_minmax(x, op, True)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    assert float(total) == ref_total


@pytest.mark.parametrize("n", [7, 2 * TT + 1, 1030 * TT + 1])
@pytest.mark.parametrize("inclusive", [False, True])
def test_widening_sum(dw, orc, n, inclusive):
    import torch
    x = wl.full_range_u32(n, seed=n + 9)
    say("two-level u32 -> u64", n, inclusive)
    got, total = _run(dw, x, "sum", inclusive, dtype=dw.PS_U64, out_dtype=torch.int64)
    ref, ref_total = orc.scan_u32_u64(x, inclusive)
    assert np.array_equal(got.view(np.uint64), ref)
    assert int(np.int64(total).view(np.uint64)) == ref_total


def test_empty_input_writes_identity_total(dw):
    import torch
    d = torch.empty(0, dtype=torch.int32, device="cuda")
    tot = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    dw.ps_scan_two_level("min", False, d, d.clone(), tot)
    assert int(host(tot)[0]) == 0xFFFFFFFF


@pytest.mark.parametrize("n", [TT - 3, 40 * TT + 1, 1200 * TT])
def test_in_place(dw, orc, n):
    x = wl.full_range_u32(n, seed=n + 10)
    d = dev(x)
    say("two-level in place", n)
    dw.ps_scan_two_level("sum", True, d, d)
    assert np.array_equal(host(d), orc.scan_u32(x, "sum", True)[0])


@pytest.mark.parametrize("n", [TT + 5, 1100 * TT + 5])
def test_unaligned_pointers(dw, orc, n):
    import torch
    x = wl.full_range_u32(n, seed=n + 11)
    vx = dev(np.concatenate(([0], x)).astype(np.uint32))[1:]
    vo = torch.zeros(n + 1, dtype=torch.int32, device="cuda")[1:]
    assert vx.data_ptr() % 16 and vo.data_ptr() % 16
    say("two-level unaligned", n)
    dw.ps_scan_two_level("xor", False, vx, vo)
    assert np.array_equal(host(vo), orc.scan_u32(x, "xor", False)[0])


def test_large_config(dw, orc):
    """2^28 elements: 65 536 tiles, the three-launch form."""
    x = wl.large_u32()
    say("two-level 2^28")
    got, total = _run(dw, x, "sum", False)
    ref, ref_total = orc.scan_u32(x, "sum", False)
    assert np.array_equal(got, ref) and int(total) == ref_total
