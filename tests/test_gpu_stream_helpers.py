"""The measurement helpers: copy, read-only and write-only streams, and the
recurrence's two-plane stream (the practical bandwidth ceilings the scans
are compared with)."""
import numpy as np
import pytest

import workloads as wl
from gpu_util import dev, host, require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dw():
    return require_gpu()


@pytest.mark.parametrize("n", [1, 3, 4, 5, 1023, 4096, 16384, 16385, 1_000_003])
def test_copy_and_fill(dw, n):
    import torch
    x = wl.full_range_u32(n, seed=n + 60)
    d_out = torch.zeros(n, dtype=torch.int32, device="cuda")
    say("copy", n)
    dw.ps_copy_u32(dev(x), d_out)
    assert np.array_equal(host(d_out), x)
    dw.ps_fill_u32(d_out, 0xDEADBEEF)
    assert np.all(host(d_out) == 0xDEADBEEF)


def test_fill_unaligned(dw):
    import torch
    n = 10_001
    buf = torch.zeros(n + 1, dtype=torch.int32, device="cuda")
    dw.ps_fill_u32(buf[1:], 5)
    h = host(buf)
    assert h[0] == 0 and np.all(h[1:] == 5)


@pytest.mark.parametrize("n", [4, 16384, 1 << 20])
def test_read_leaves_sink(dw, n):
    import torch
    x = wl.full_range_u32(n, seed=n + 61)
    sink = torch.full((1,), 12345, dtype=torch.int32, device="cuda")
    dw.ps_read_u32(dev(x), sink)
    assert int(host(sink)[0]) == 12345


@pytest.mark.parametrize("both", [False, True])
@pytest.mark.parametrize("n", [4, 16384, 1_000_004])
def test_planes_stream(dw, n, both):
    """b' = a * b and a' = a + b element by element: one IEEE fp32 operation
    each, so the results equal numpy's bit for bit (values in [0.5, 2):
    no subnormals)."""
    import torch
    g = np.random.default_rng(n + 62)
    a = g.uniform(0.5, 2.0, n).astype(np.float32)
    b = g.uniform(0.5, 2.0, n).astype(np.float32)
    ob = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
    oa = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda") if both else None
    say("planes stream", n, both)
    dw.ps_stream_planes_f32(torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda(), ob, out_a=oa)
    assert np.array_equal(host(ob).view(np.uint32), (a * b).view(np.uint32))
    if both:
        assert np.array_equal(host(oa).view(np.uint32), (a + b).view(np.uint32))


def test_kernel_timing_samples_every_nth_call(dw):
    """ps_kernel_timing(every=N) times the 1st, (N+1)th, ... main-kernel
    launch: 7 calls at N = 3 give 3 timed launches, each a plausible kernel
    time; N = 1 times all of them; timing off records none."""
    import torch
    x = torch.zeros(1 << 20, dtype=torch.int32, device="cuda")
    y = torch.empty_like(x)
    for every, calls, want in ((3, 7, 3), (1, 4, 4), (5, 5, 1)):
        dw.ps_kernel_timing(True, every=every)
        for _ in range(calls):
            dw.ps_copy_u32(x, y)
        ms, launches = dw.ps_kernel_timing_read()
        assert launches == want, (every, calls, launches)
        assert 0.0 < ms / launches < 10.0
    dw.ps_kernel_timing(False)
    dw.ps_copy_u32(x, y)
    assert dw.ps_kernel_timing_read() == (0.0, 0)
