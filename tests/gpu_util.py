"""Helpers of the GPU parity tests: device transfer, workspace error word,
and the fp32 tolerance of the flat sum scan."""
from __future__ import annotations

import sys

import numpy as np
import pytest

TILE = 12288         # elements per tile of the segmented kernel (12 data waves x 4 x 256)
SEG_DATA_WAVES = 12  # data waves per workgroup of the segmented kernel
FLAT_TILE = 12288    # elements per tile of the flat scan (8 data waves x 6 x 256)
FLAT_GROUP = 2       # consecutive flat tiles claimed per ticket
LINREC_TILE = 6144   # pairs per tile of the recurrence scan (8 data waves x 3 x 256)
# Absolute floor of the recurrence tolerance: products of decays below
# 2^-100 are past any use, and an fp32 result there may be subnormal or
# flushed (error below 2^-126).
LINREC_FLOOR = 2.0 ** -100


def require_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import device_wide_prefix_chained_amd as dw
    dw.lib()  # raises when the HIP library is missing: no silent fallback
    return dw


def say(*args):
    """Name the case on stdout before a GPU step (flushed, so that it survives
    a crash of the process)."""
    print("[gpu-case]", *args, flush=True)
    sys.stdout.flush()


def dev(a):
    """Host array -> device tensor.  uint32 data travels as bit-identical int32
    tensors (PyTorch's uint32 support is minimal; the library reads bits)."""
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint32:
        a = a.view(np.int32)
    return torch.from_numpy(a).to("cuda")


def host(t):
    """Device tensor -> host array; int32 tensors come back as uint32."""
    import torch
    torch.cuda.synchronize()
    a = t.cpu().numpy()
    return a.view(np.uint32) if a.dtype == np.int32 else a


def filled_dev(like, fill):
    """A device array shaped like the host array ``like``, every element = fill."""
    return dev(np.full_like(like, fill))


def ws_error_word(ws) -> int:
    """Word 1 of a workspace header: nonzero when a look-back hit its spin limit."""
    return int(host(ws[4:8].clone()).view(np.uint32)[0])


def assert_f32_sum_close(gpu, ref64, absprefix, exclusive):
    """|gpu_i - ref_i| <= 1e-5 * sum_{j<=i} |x_j| at every index; exclusive
    output 0 must be exactly +0.0."""
    gpu64 = gpu.astype(np.float64)
    err = np.abs(gpu64 - ref64)
    tol = 1e-5 * absprefix
    bad = np.nonzero(err > tol)[0]
    assert bad.size == 0, ("fp32 tolerance broken at %d indices, first %d: gpu %r ref %r tol %r"
                           % (bad.size, bad[0], gpu[bad[0]], ref64[bad[0]], tol[bad[0]]))
    if exclusive and gpu.size:
        assert gpu[0] == 0.0 and not np.signbit(gpu[0])
    return float((err / np.maximum(tol, 1e-300)).max()) if gpu.size else 0.0


def product_bound(n, first=0):
    """Relative rounding bound of the A component at indices first ..
    first + n - 1: a product of t + 1 fp32 factors, formed in any grouping,
    is rounded t times, so it lies within gamma_t = t u / (1 - t u) of the
    exact product (u = 2^-24; the identity pad multiplies exactly).
    gamma_(t+1) is used for both forms (the exclusive form has one factor
    less); past t u = 1/2 the bound says nothing and is capped at 1."""
    u = 2.0 ** -24
    tu = np.arange(first + 1, first + n + 1, dtype=np.float64) * u
    return np.where(tu < 0.5, tu / (1.0 - np.minimum(tu, 0.5)), 1.0)


def assert_linrec_close(gpu_a, gpu_b, ref_a, ref_b, mag_a, mag_b, exclusive, first=0):
    """Recurrence-pair tolerance at every index: B within 1e-5 * (the same
    scan over (|a|, |b|)) + 2^-100, which reduces to the fp32 sum scan's bound
    when a = 1; A within max(1e-5, gamma_(t+1)) * prod |a| + 2^-100 (the B
    bound, widened where the product's own rounding bound is larger).  An
    exclusive output 0 must be exactly (1, 0).  gpu_a may be None (B only).
    `first` is the index of the first element given (the total of n pairs is
    index n - 1)."""
    worst = 0.0
    comps = [("B", gpu_b, ref_b, 1e-5 * mag_b)]
    if gpu_a is not None:
        comps.append(("A", gpu_a, ref_a, np.maximum(1e-5, product_bound(gpu_a.size, first)) * mag_a))
    for name, g, r, rel in comps:
        err = np.abs(g.astype(np.float64) - r)
        tol = rel + LINREC_FLOOR
        bad = np.nonzero(~(err <= tol))[0]  # NaN counts as bad
        assert bad.size == 0, ("%s: tolerance broken at %d indices, first %d: gpu %r ref %r tol %r"
                               % (name, bad.size, bad[0], g[bad[0]], r[bad[0]], tol[bad[0]]))
        if g.size:
            worst = max(worst, float((err / tol).max()))
    if exclusive and gpu_b.size:
        assert gpu_b[0] == 0.0
        if gpu_a is not None:
            assert gpu_a[0] == 1.0
    return worst
