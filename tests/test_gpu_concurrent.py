"""Calls in flight together on different streams, each with its own
workspace: the persistent kernels of one call only ever wait on tiles handed
out to their own running workgroups, so two of them sharing the GPU both
finish, and neither disturbs the other's descriptors or counter.  Every
result is checked against the oracle after all streams drained."""
import numpy as np
import pytest

import workloads as wl
from gpu_util import dev, host, require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dw():
    return require_gpu()


def test_three_streams_interleaved(dw, orc):
    import torch
    n = (1 << 24) + 77
    x = wl.full_range_u32(n, seed=401)
    vals, offs = wl.zipf_segments(n=1 << 23, num_segments=1 << 12, seed=402)
    rec = wl.full_range_u32(4 * (1 << 21), seed=403).reshape(-1, 4)
    flags = wl.flag_pattern(rec.shape[0], "random", seed=404)
    dx, dv, do, dr, df = dev(x), dev(vals), dev(offs), dev(rec), dev(flags)
    streams = [torch.cuda.Stream() for _ in range(3)]
    ws = [dw.new_workspace(dw.workspace_bytes("ps_scan_exclusive_u32", None, None, n, None, None)),
          dw.new_workspace(dw.workspace_bytes("ps_segmented_scan_u32", None, vals.size, None, offs.size - 1, None, 0,
                                         None)),
          dw.new_workspace(dw.workspace_bytes("ps_compact", None, 16, None, flags.size, None, None, None))]
    rounds = 4
    outs = [[torch.empty_like(dx), torch.empty_like(dv), torch.empty_like(dr),
             torch.zeros(1, dtype=torch.int64, device="cuda")] for _ in range(rounds)]
    torch.cuda.synchronize()
    say("three streams interleaved", rounds)
    for r in range(rounds):
        o = outs[r]
        # a round's three calls, each on its own stream and workspace, are in
        # flight together; each kind moves to another stream every round
        dw.ps_scan_exclusive_u32(dx, o[0], workspace=ws[0], stream=streams[r % 3])
        dw.ps_segmented_scan_u32(dv, do, o[1], inclusive=True, workspace=ws[1], stream=streams[(r + 1) % 3])
        dw.ps_compact(dr, df, o[2], o[3], workspace=ws[2], stream=streams[(r + 2) % 3])
        # the next round's call of each kind reuses that kind's workspace on
        # another stream: every stream waits for this round (device-side
        # events, no host synchronization)
        ev = [torch.cuda.Event() for _ in streams]
        for e, s in zip(ev, streams):
            e.record(s)
        for s in streams:
            for e in ev:
                s.wait_event(e)
    torch.cuda.synchronize()
    ref_x, _ = orc.scan_u32(x, "sum", False)
    ref_v = orc.segmented_scan_u32(vals, offs, True, sentinel=0)
    ref_c, ref_count = orc.compact(rec, flags)
    for r in range(rounds):
        o = outs[r]
        assert np.array_equal(host(o[0]), ref_x), r
        assert np.array_equal(host(o[1]), ref_v), r
        c = int(host(o[3])[0])
        assert c == ref_count and np.array_equal(host(o[2])[:c], ref_c[:c]), r
