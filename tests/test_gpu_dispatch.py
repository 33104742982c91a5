"""The flat entry points at their default setting: inputs up to 2^23
elements run the two-level form, larger ones the single-pass chained form.
Both sides of the switch, every entry point, checked against the oracle."""
import numpy as np
import pytest

import workloads as wl
from gpu_util import assert_f32_sum_close, assert_linrec_close, dev, host, require_gpu, say

pytestmark = pytest.mark.gpu

SWITCH = 1 << 23


@pytest.fixture(scope="module")
def dw():
    d = require_gpu()
    assert d.ps_small_n_config_get() == SWITCH
    return d


@pytest.mark.parametrize("n", [1, 4097, 1 << 20, SWITCH, SWITCH + 1])
@pytest.mark.parametrize("inclusive", [False, True])
def test_u32_sum_across_the_switch(dw, orc, n, inclusive):
    import torch
    x = wl.full_range_u32(n, seed=n + 41)
    d_in, d_out = dev(x), torch.empty(n, dtype=torch.int32, device="cuda")
    tot = torch.zeros(1, dtype=torch.int32, device="cuda")
    say("default u32", n, inclusive)
    (dw.ps_scan_inclusive_u32 if inclusive else dw.ps_scan_exclusive_u32)(d_in, d_out, tot)
    ref, ref_total = orc.scan_u32(x, "sum", inclusive)
    assert np.array_equal(host(d_out), ref) and int(host(tot)[0]) == ref_total


@pytest.mark.parametrize("n", [77, 300_001])
def test_f32_and_widening_small(dw, orc, n):
    import torch
    x = wl.normal_f32(n, seed=n + 42)
    d_out = torch.empty(n, dtype=torch.float32, device="cuda")
    dw.ps_scan_inclusive_f32(dev(x), d_out)
    ref, absprefix, _ = orc.scan_f32_sum(x, True)
    assert_f32_sum_close(host(d_out), ref, absprefix, exclusive=False)
    u = wl.full_range_u32(n, seed=n + 43)
    o64 = torch.empty(n, dtype=torch.int64, device="cuda")
    dw.ps_scan_exclusive_u32_u64(dev(u), o64)
    assert np.array_equal(host(o64).view(np.uint64), orc.scan_u32_u64(u, False)[0])


@pytest.mark.parametrize("op", ["max", "affine16"])
def test_generic_small(dw, orc, op):
    import torch
    n = 123_457
    x = wl.full_range_u32(n, seed=44) | np.uint32(0x00010000)
    d_out = torch.empty(n, dtype=torch.int32, device="cuda")
    dw.ps_scan(op, False, dev(x), d_out)
    assert np.array_equal(host(d_out), orc.scan_u32(x, op, False)[0])


@pytest.mark.parametrize("n", [3, 5000, 2_000_003])
def test_recurrence_small(dw, orc, n):
    import torch
    a, b = wl.linrec_pairs(n, seed=n + 45, a_lo=-1.2, a_hi=1.2)
    oa = torch.empty(n, dtype=torch.float32, device="cuda")
    ob = torch.empty_like(oa)
    say("default linrec", n)
    dw.ps_scan_linrec_f32(dev(a), dev(b), ob, out_a=oa, inclusive=True)
    A, B, SA, SB, _ = orc.scan_linrec_f32(np.stack([a, b], 1), True)
    assert_linrec_close(host(oa), host(ob), A, B, SA, SB, False)


@pytest.mark.parametrize("n", [5, 40_000, 3_000_001])
def test_single_pass_entry_at_small_sizes(dw, orc, n):
    import torch
    x = wl.full_range_u32(n, seed=n + 46)
    d_out = torch.empty(n, dtype=torch.int32, device="cuda")
    dw.ps_scan_single_pass("xor", True, dev(x), d_out)
    assert np.array_equal(host(d_out), orc.scan_u32(x, "xor", True)[0])


def test_workspace_fits_either_form(dw, orc):
    """A workspace sized by the query at the default setting serves a call
    after the setting changed."""
    import torch
    n = 5_000_000
    ws = dw.new_workspace(dw.workspace_bytes("ps_scan_exclusive_u32", None, None, n, None, None))
    x = wl.full_range_u32(n, seed=47)
    ref, _ = orc.scan_u32(x, "sum", False)
    old = dw.ps_small_n_config_get()
    try:
        for setting in (0, SWITCH, 1 << 24):
            dw.ps_small_n_config(setting)
            d_out = torch.empty(n, dtype=torch.int32, device="cuda")
            dw.ps_scan_exclusive_u32(dev(x), d_out, workspace=ws)
            assert np.array_equal(host(d_out), ref), setting
    finally:
        dw.ps_small_n_config(old)
