"""ps_scan_noalloc, the entry point that allocates nothing (its workspace is
an array inside the library), against ps_scan on the same inputs: two calls
in a row, the second smaller, at sizes that take the single-pass kernel and
the two-level form, for an integer sum (bit-exact), an fp32 max (bit-exact)
and an fp32 sum (within the fp32 bound of the oracle)."""
import numpy as np
import pytest

import workloads as wl
from gpu_util import FLAT_TILE, assert_f32_sum_close, dev, host, require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dw():
    return require_gpu()


def _both(dw, op, inclusive, x, dtype=None):
    import torch
    d_in = dev(x)
    a = torch.empty_like(d_in)
    b = torch.empty_like(d_in)
    ta = torch.zeros(1, dtype=d_in.dtype, device="cuda")
    tb = torch.zeros(1, dtype=d_in.dtype, device="cuda")
    dw.ps_scan_noalloc(op, inclusive, d_in, a, total=ta, dtype=dtype)
    dw.ps_scan(op, inclusive, d_in, b, total=tb, dtype=dtype)
    return host(a), host(b), host(ta), host(tb)


@pytest.mark.parametrize("sizes", [((1 << 26) + 77, 300 * FLAT_TILE + 5), ((1 << 24) + 3, 1000)])
def test_noalloc_matches_ps_scan(dw, orc, sizes):
    for rep, n in enumerate(sizes):
        say("noalloc u32 sum", n, rep)
        x = wl.full_range_u32(n, seed=600 + rep)
        got, want, tg, tw = _both(dw, "sum", False, x)
        ref, ref_total = orc.scan_u32(x, "sum", False)
        assert np.array_equal(got, want) and np.array_equal(got, ref)
        assert int(tg[0]) == int(tw[0]) == int(ref_total)

        say("noalloc f32 max / sum", n, rep)
        f = wl.normal_f32(n, seed=610 + rep)
        got, want, _, _ = _both(dw, "max", True, f)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
        got, want, _, _ = _both(dw, "sum", True, f)
        ref, absprefix, _ = orc.scan_f32_sum(f, True, want_abs=True)
        assert_f32_sum_close(got, ref, absprefix, exclusive=False)
        assert_f32_sum_close(want, ref, absprefix, exclusive=False)


def test_noalloc_size_limit(dw):
    import torch
    assert dw.ps_scan_noalloc_bytes() == 4 << 20
    # the widening sum's workspace outgrows the array past about 1.6e9 elements;
    # the size check happens before any pointer is used
    big = torch.empty(0, dtype=torch.int32, device="cuda")
    L = dw.lib()
    st = L.ps_scan_noalloc(0, 2, 0, big.data_ptr() or 16, big.data_ptr() or 16, 1_700_000_000, None, None)
    assert st == 3  # PS_ERR_SIZE
