"""The largest input the C ABI takes: n = 2^32 - 1 elements (records, pairs).

At this size the oracle would need tens of GiB of host memory and a minute
of CPU time per call, so these tests build their inputs on the device from
closed forms and check EVERY output against the closed form of its prefix,
computed independently with plain integer arithmetic (chunks of 2^27 on the
device, never through this library):
  * x[i] = i mod 7:  sum of x[0 .. i-1] = 21 * (i // 7) + r (r - 1) / 2,
    r = i mod 7 (mod 2^32 for uint32 results);
  * x[i] = 2^32 - 1: sum of x[0 .. i-1] = (i - 1) * 2^32 + (2^32 - i) for
    i >= 1 (the widening scan's high and low words);
  * records rec[i] = i kept where i mod 3 == 0: out[k] = 3 k, count =
    ceil(n / 3);
  * the recurrence with a = 0: every state forgets, h[t] = b[t] exactly.
A period of 7 does not divide the tile sizes, so a tile stored at the wrong
place, a prefix taken from the wrong tile or a 32-bit index that wraps
changes the result.  Up to about 80 GiB of device memory (the recurrence's
four planes and a temporary)."""
import numpy as np
import pytest

from gpu_util import require_gpu, say

pytestmark = pytest.mark.gpu

N = (1 << 32) - 1
CH = 1 << 27
MASK32 = (1 << 32) - 1


@pytest.fixture(scope="module")
def dw():
    d = require_gpu()
    import torch
    free, _ = torch.cuda.mem_get_info()
    if free < 96 * (1 << 30):
        pytest.skip("needs about 96 GiB of free device memory")
    return d


def _as_i32(t):
    """int64 values in [0, 2^32) -> the int32 tensor holding their uint32 bits."""
    import torch
    return (t - (t >> 31) * (1 << 32)).to(torch.int32)


def _chunks(n):
    for c0 in range(0, n, CH):
        yield c0, min(n, c0 + CH)


def _mod7_u32(n):
    import torch
    x = torch.empty(n, dtype=torch.int32, device="cuda")
    for c0, c1 in _chunks(n):
        x[c0:c1] = (torch.arange(c0, c1, dtype=torch.int64, device="cuda") % 7).to(torch.int32)
    return x


def _s7(i):
    """sum_{j < i} (j mod 7) for an int64 tensor i (exact in int64)."""
    r = i % 7
    return 21 * (i // 7) + r * (r - 1) // 2


def _check_u32(out, expect_fn, n, what):
    """out (int32 bits of uint32) against expect_fn(i) mod 2^32, chunk by chunk."""
    import torch
    for c0, c1 in _chunks(n):
        i = torch.arange(c0, c1, dtype=torch.int64, device="cuda")
        got = out[c0:c1].to(torch.int64) & MASK32
        want = expect_fn(i) & MASK32
        bad = torch.nonzero(got != want)
        if bad.numel():
            k = int(bad[0, 0])
            raise AssertionError("%s: %d rows differ in [%d, %d), first %d: %d vs %d"
                                 % (what, bad.numel(), c0, c1, c0 + k, int(got[k]), int(want[k])))


@pytest.mark.parametrize("form", ["default", "two_level"])
def test_flat_u32(dw, form):
    import torch
    x = _mod7_u32(N)
    out = torch.empty(N, dtype=torch.int32, device="cuda")
    tot = torch.zeros(1, dtype=torch.int32, device="cuda")
    for inclusive in (False, True):
        say("max size u32", form, inclusive)
        if form == "default":
            (dw.ps_scan_inclusive_u32 if inclusive else dw.ps_scan_exclusive_u32)(x, out, tot)
        else:
            dw.ps_scan_two_level("sum", inclusive, x, out, tot)
        torch.cuda.synchronize()
        if inclusive:
            _check_u32(out, lambda i: _s7(i + 1), N, "inclusive")
        else:
            _check_u32(out, _s7, N, "exclusive")
        assert (int(tot[0]) & MASK32) == (_s7(torch.tensor([N])).item() & MASK32)
    del x, out


def test_widening(dw):
    import torch
    x = torch.full((N,), -1, dtype=torch.int32, device="cuda")  # 2^32 - 1 everywhere
    out = torch.empty(N, dtype=torch.int64, device="cuda")
    say("max size u32 -> u64")
    dw.ps_scan_exclusive_u32_u64(x, out)
    torch.cuda.synchronize()
    del x
    words = out.view(torch.int32)
    for c0, c1 in _chunks(N):
        i = torch.arange(c0, c1, dtype=torch.int64, device="cuda")
        lo = words[2 * c0:2 * c1:2].to(torch.int64) & MASK32
        hi = words[2 * c0 + 1:2 * c1:2].to(torch.int64) & MASK32
        want_lo = torch.where(i == 0, 0, (1 << 32) - i)
        want_hi = torch.where(i == 0, 0, i - 1)
        assert torch.equal(lo, want_lo) and torch.equal(hi, want_hi), (c0, c1)


def test_segmented(dw):
    """Segment k starts at 1000 k + (k^2 mod 997) (lengths 5 .. 1995), about
    4.3 M segments, so the offsets' sample is capped and probe rounds
    narrow every tile's bracket; the last 12 345 rows belong to no segment
    and must keep their sentinel."""
    import torch
    hi_row = N - 12345
    k = torch.arange(0, hi_row // 1000 + 2, dtype=torch.int64, device="cuda")
    starts = 1000 * k + (k * k) % 997
    starts = starts[starts < hi_row]
    offsets = torch.cat([starts, torch.tensor([hi_row], dtype=torch.int64, device="cuda")])
    assert bool(torch.all(offsets[1:] > offsets[:-1]))
    d_off = _as_i32(offsets)
    x = _mod7_u32(N)
    out = torch.full((N,), 0x5EED, dtype=torch.int32, device="cuda")
    say("max size segmented", offsets.numel() - 1)
    dw.ps_segmented_scan_u32(x, d_off, out, inclusive=False)
    torch.cuda.synchronize()
    del x

    def expect(i):
        s = torch.searchsorted(offsets, i, right=True) - 1
        seg_start = offsets[s.clamp(min=0)]
        return _s7(i) - _s7(seg_start)
    _check_u32(out[:hi_row], expect, hi_row, "segmented exclusive")
    assert bool(torch.all(out[hi_row:] == 0x5EED))


def test_compaction_4_byte_records(dw):
    import torch
    rec = torch.empty(N, dtype=torch.int32, device="cuda")
    flags = torch.empty(N, dtype=torch.uint8, device="cuda")
    for c0, c1 in _chunks(N):
        i = torch.arange(c0, c1, dtype=torch.int64, device="cuda")
        rec[c0:c1] = _as_i32(i)
        flags[c0:c1] = (i % 3 == 0).to(torch.uint8)
    out = torch.empty(N, dtype=torch.int32, device="cuda")
    cnt = torch.zeros(1, dtype=torch.int64, device="cuda")
    say("max size compaction")
    dw.ps_compact(rec, flags, out, cnt)
    torch.cuda.synchronize()
    del rec, flags
    count = (N + 2) // 3
    assert int(cnt[0]) == count
    _check_u32(out[:count], lambda k: 3 * k, count, "compaction")


def test_recurrence_forgets(dw):
    import torch
    a = torch.zeros(N, dtype=torch.float32, device="cuda")
    b = _mod7_u32(N).to(torch.float32)
    ob = torch.empty(N, dtype=torch.float32, device="cuda")
    oa = torch.empty(N, dtype=torch.float32, device="cuda")
    say("max size recurrence")
    dw.ps_scan_linrec_f32(a, b, ob, out_a=oa, inclusive=True)
    torch.cuda.synchronize()
    assert torch.equal(ob, b)
    assert bool(torch.all(oa == 0.0))
