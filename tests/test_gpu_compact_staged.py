"""Parity of the staged compaction (flag scan, then scatter: the ablation of
the fused kernel) with the oracle and with the fused kernel: bit-exact
records, exact count, untouched slots past the count."""
import numpy as np
import pytest

import workloads as wl
from gpu_util import dev, host, require_gpu, say

pytestmark = pytest.mark.gpu

FILL = 0xA5A5A5A5


@pytest.fixture(scope="module")
def dw():
    return require_gpu()


def _run(dw, fn, records, flags):
    import torch
    d_out = dev(np.full_like(records, FILL))
    cnt = torch.full((1,), -7, dtype=torch.int64, device="cuda")
    getattr(dw, fn)(dev(records), dev(flags), d_out, cnt)
    return host(d_out), int(host(cnt)[0])


@pytest.mark.parametrize("n", [1, 2, 3, 5, 63, 64, 65, 4097, 300_007, (1 << 23) + 3])
@pytest.mark.parametrize("width", [1, 2, 4])
@pytest.mark.parametrize("kind", ["none", "all", "random", "clustered"])
def test_staged_matches_oracle_and_fused(dw, orc, n, width, kind):
    rec = wl.full_range_u32(n * width, seed=n + width + 50).reshape(n, width)
    if width == 1:
        rec = rec.reshape(n)
    flags = wl.flag_pattern(n, kind, seed=n + 51, run=37)
    if kind == "random":
        flags = flags * wl.uniform_u32(n, 255, seed=n + 52).astype(np.uint8) + flags  # any nonzero keeps
    say("staged compact", n, width, kind)
    got, count = _run(dw, "ps_compact_staged", rec, flags)
    ref, ref_count = orc.compact(rec, flags, out=np.full_like(rec, FILL))
    assert count == ref_count
    assert np.array_equal(got, ref)
    fused, fcount = _run(dw, "ps_compact", rec, flags)
    assert fcount == count and np.array_equal(fused, got)


def test_empty(dw):
    import torch
    cnt = torch.full((1,), -7, dtype=torch.int64, device="cuda")
    e = torch.empty(0, dtype=torch.int32, device="cuda")
    dw.ps_compact_staged(e, torch.empty(0, dtype=torch.uint8, device="cuda"), e.clone(), cnt)
    assert int(host(cnt)[0]) == 0


def test_records_config(dw, orc):
    """The 2^26 x 16-byte record workload, Bernoulli(0.3) flags."""
    rec, flags = wl.compaction_records()
    say("staged compact config")
    got, count = _run(dw, "ps_compact_staged", rec, flags)
    ref, ref_count = orc.compact(rec, flags)
    assert count == ref_count and np.array_equal(got[:count], ref[:count])
