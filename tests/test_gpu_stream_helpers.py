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


def _mix_expected(x, n_out):
    """The mix stream's output from its definition: the words both sides
    have copied, zeros after them up to n_out."""
    both = min(x.size, n_out)
    out = np.zeros(n_out, np.uint32)
    out[:both] = x[:both]
    return out


@pytest.mark.parametrize("n_in,n_out", [(4, 4), (4096, 8192), (8192 * 3 + 4, 4 * 1000), (1 << 20, 3 << 19),
                                        (12, 1 << 16), (1 << 16, 0), (0, 4096), (4 * 1_000_003, 8 * 1_000_003)])
def test_mix_stream(dw, n_in, n_out):
    import torch
    x = wl.full_range_u32(n_in, seed=n_in + 63)
    d_in = dev(x) if n_in else torch.empty(0, dtype=torch.int32, device="cuda")
    buf = torch.full((n_out + 4,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
    say("mix stream", n_in, n_out)
    dw.ps_stream_mix_u32(d_in, buf[:n_out])
    h = host(buf)
    assert np.array_equal(h[:n_out], _mix_expected(x, n_out)) and np.all(h[n_out:] == 0x5A5A5A5A)


def _mix_even_expected(x, n_out):
    """The even mix stream's output from its definition: workgroup b writes
    its share of oc output vectors, each the input vector at the same offset
    of its block of 1024 (the last input vector past the end)."""
    vin = x.reshape(-1, 4)
    ni, no = len(vin), n_out // 4
    oc = -(-(no * 1024) // ni)
    out = np.zeros((no, 4), np.uint32)
    for b in range(-(-ni // 1024)):
        for j in range(oc):
            if b * oc + j < no:
                out[b * oc + j] = vin[min(b * 1024 + j, ni - 1)]
    return out.reshape(-1)


@pytest.mark.parametrize("n_in,n_out", [(4, 4), (4096, 4096), (8192 * 3 + 4, 4 * 1000), (1 << 20, 3 << 18),
                                        (4 * 1_000_003, 4 * 285_715), (1 << 16, 0)])
def test_mix_even_stream(dw, n_in, n_out):
    import torch
    x = wl.full_range_u32(n_in, seed=n_in + 65)
    buf = torch.full((n_out + 4,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
    say("mix even stream", n_in, n_out)
    dw.ps_stream_mix_even_u32(dev(x), buf[:n_out])
    h = host(buf)
    assert np.array_equal(h[:n_out], _mix_even_expected(x, n_out)) and np.all(h[n_out:] == 0x5A5A5A5A)


@pytest.mark.parametrize("threads", [64, 128, 256])
@pytest.mark.parametrize("vecs", [4, 8, 16])
def test_stream_shapes(dw, threads, vecs):
    """Every shape of the stream sweep copies and fills exactly n words and
    nothing past them, and its read leaves the sink alone: sizes below one
    block, between whole blocks and above the resident grid's first pass."""
    import torch
    for n in (4, 4 * (threads * vecs * 3 + 5), 1_000_004, 4 * 256 * 16 * 2048 + 12):
        x = wl.full_range_u32(n, seed=n + threads + vecs)
        d_in = dev(x)
        sink = torch.full((1,), 12345, dtype=torch.int32, device="cuda")
        for nt in (False, True):
            for persistent in (False, True):
                say("stream shape", threads, vecs, nt, persistent, n)
                buf = torch.full((n + 4,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
                dw.ps_stream_shape("copy", buf[:n], d_in, threads=threads, vecs=vecs, nontemporal=nt,
                                   persistent=persistent)
                h = host(buf)
                assert np.array_equal(h[:n], x) and np.all(h[n:] == 0x5A5A5A5A)
                dw.ps_stream_shape("write", buf[:n], threads=threads, vecs=vecs, nontemporal=nt,
                                   persistent=persistent, value=0xC0FFEE00 + n % 251)
                h = host(buf)
                assert np.all(h[:n] == 0xC0FFEE00 + n % 251) and np.all(h[n:] == 0x5A5A5A5A)
                dw.ps_stream_shape("read", sink, d_in, threads=threads, vecs=vecs, nontemporal=nt,
                                   persistent=persistent)
                assert int(host(sink)[0]) == 12345
