"""Parity of the flat chained scan (HIP, through the C ABI) with the oracle.

Integer results must be bit-exact; fp32 sums must satisfy
|gpu_i - oracle_fp64_i| <= 1e-5 * sum_{j<=i}|x_j| at every index; fp32
max/min are exact and compared bit for bit."""
import numpy as np
import pytest

import workloads as wl
from gpu_util import FLAT_GROUP, FLAT_TILE, TILE, assert_f32_sum_close, dev, host, require_gpu, say, ws_error_word
from pins import golden

pytestmark = pytest.mark.gpu

FT = FLAT_TILE
EDGE_SIZES = [1, 2, 3, 4, 5, 31, 32, 33, 63, 64, 65, 255, 256, 257, 1023, 1024, 1025, 1536, 1537,
              TILE - 1, TILE, TILE + 1, FT - 1, FT, FT + 1, 2 * FT - 1, 2 * FT, 2 * FT + 1,
              3 * FT - 1, 3 * FT + 17, 64 * FT + 5, 65 * FT - 3, 257 * FT, 513 * FT + 1, 1_000_003]
U32_OPS = ["sum", "max", "min", "and", "or", "xor", "affine16"]


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


def test_tile_shape_matches_the_library(dw):
    assert dw.ps_tile_elements(0) == FLAT_TILE
    assert dw.ps_lookback_group() == FLAT_GROUP


def _run_u32(dw, x, op="sum", inclusive=False, with_total=True):
    import torch
    d_in = dev(x)
    d_out = torch.empty_like(d_in)
    d_tot = torch.zeros(1, dtype=torch.int32, device="cuda") if with_total else None
    dw.ps_scan(op, inclusive, d_in, d_out, d_tot)
    return host(d_out), (int(host(d_tot)[0]) if with_total else None)


def test_worked_examples(dw, orc):
    import torch
    for name in ("p1_lead_scan.json", "p3_inclusive_exclusive.json", "p5_flat_example.json"):
        g = golden(name)
        x = np.array(g["input"], np.uint32)
        say("worked example", name)
        d_in, d_out = dev(x), torch.empty(len(x), dtype=torch.int32, device="cuda")
        tot = torch.zeros(1, dtype=torch.int32, device="cuda")
        dw.ps_scan_exclusive_u32(d_in, d_out, tot)
        assert host(d_out).tolist() == g["exclusive"] and int(host(tot)[0]) == sum(g["input"])
        dw.ps_scan_inclusive_u32(d_in, d_out, tot)
        assert host(d_out).tolist() == g["inclusive"]


@pytest.mark.parametrize("n", EDGE_SIZES)
@pytest.mark.parametrize("inclusive", [False, True])
def test_u32_sum_edge_sizes(dw, orc, n, inclusive):
    x = wl.full_range_u32(n, seed=n)
    say("u32 sum", n, inclusive)
    got, total = _run_u32(dw, x, "sum", inclusive)
    ref, ref_total = orc.scan_u32(x, "sum", inclusive)
    assert np.array_equal(got, ref)
    assert total == ref_total


@pytest.mark.parametrize("op", U32_OPS)
@pytest.mark.parametrize("n", [1000, 3 * FT + 17, 300 * FT + 1])
@pytest.mark.parametrize("inclusive", [False, True])
def test_u32_all_operators(dw, orc, op, n, inclusive):
    r = np.random.default_rng(n + 17)
    if op in ("and", "or"):
        # mostly-set / mostly-clear bits, so the running result keeps changing
        x = r.integers(0, 1 << 32, size=(n, 3), dtype=np.uint64).astype(np.uint32)
        x = (x[:, 0] | x[:, 1] | x[:, 2]) if op == "and" else (x[:, 0] & x[:, 1] & x[:, 2])
    else:
        x = r.integers(0, 1 << 32, size=n, dtype=np.uint64).astype(np.uint32)
    say("u32", op, n, inclusive)
    got, total = _run_u32(dw, x, op, inclusive)
    ref, ref_total = orc.scan_u32(x, op, inclusive)
    assert np.array_equal(got, ref), op
    assert total == ref_total


@pytest.mark.parametrize("n", [1, 33, FT + 1, 100_003, 3_000_001])
@pytest.mark.parametrize("inclusive", [False, True])
def test_f32_sum_tolerance(dw, orc, n, inclusive):
    import torch
    x = wl.normal_f32(n, seed=n)
    say("f32 sum", n, inclusive)
    d_in = dev(x)
    d_out = torch.empty_like(d_in)
    tot = torch.zeros(1, dtype=torch.float32, device="cuda")
    (dw.ps_scan_inclusive_f32 if inclusive else dw.ps_scan_exclusive_f32)(d_in, d_out, tot)
    ref, ab, ref_total = orc.scan_f32_sum(x, inclusive)
    assert_f32_sum_close(host(d_out), ref, ab, exclusive=not inclusive)
    assert abs(float(host(tot)[0]) - ref_total) <= 1e-5 * ab[-1]


@pytest.mark.parametrize("n", [7, FT * 5 + 3, 1_000_003])
def test_f32_small_integers_are_exact(dw, orc, n):
    """fp32 inputs that are small integers stay exact under any grouping while
    every partial sum is below 2^24, so the result equals the integer scan."""
    import torch
    x = wl.small_int_f32(n, seed=n)
    say("f32 small-int", n)
    d_in = dev(x)
    d_out = torch.empty_like(d_in)
    dw.ps_scan_inclusive_f32(d_in, d_out)
    ref, _, _ = orc.scan_f32_sum(x, inclusive=True)
    assert np.array_equal(host(d_out).astype(np.float64), ref)


@pytest.mark.parametrize("op", ["max", "min"])
@pytest.mark.parametrize("n", [5, FT + 3, 1_000_003])
@pytest.mark.parametrize("inclusive", [False, True])
def test_f32_minmax_bit_exact(dw, orc, op, n, inclusive):
    import torch
    x = wl.normal_f32(n, seed=n + 1)
    say("f32", op, n, inclusive)
    d_in = dev(x)
    d_out = torch.empty_like(d_in)
    tot = torch.zeros(1, dtype=torch.float32, device="cuda")
    dw.ps_scan(op, inclusive, d_in, d_out, tot)
    ref, ref_total = orc.scan_f32_minmax(x, op, inclusive)
    assert np.array_equal(host(d_out).view(np.uint32), ref.view(np.uint32))
    assert np.float32(host(tot)[0]).view(np.uint32) == np.float32(ref_total).view(np.uint32)


def test_f32_signed_zero_ties(dw, orc):
    import torch
    z = np.tile(np.array([0.0, -0.0, 0.0, -0.0], np.float32), 3 * FT)
    for op in ("max", "min"):
        for src in (z, -z):
            d_in = dev(src)
            d_out = torch.empty_like(d_in)
            dw.ps_scan(op, True, d_in, d_out)
            ref, _ = orc.scan_f32_minmax(src, op, True)
            assert np.array_equal(host(d_out).view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("shift", [1, 2, 3])
def test_unaligned_pointers(dw, orc, shift):
    """4-byte but not 16-byte aligned input/output take the scalar path."""
    import torch
    n = 7 * FT + 11
    x = wl.full_range_u32(n + shift, seed=shift)
    d_all = dev(x)
    d_in = d_all[shift:]
    out_all = torch.empty(n + 4, dtype=torch.int32, device="cuda")
    d_out = out_all[4 - shift: 4 - shift + n]
    say("unaligned", shift)
    for inclusive in (False, True):
        dw.ps_scan("sum", inclusive, d_in, d_out)
        ref, _ = orc.scan_u32(x[shift:], "sum", inclusive)
        assert np.array_equal(host(d_out), ref)


def test_in_place(dw, orc):
    n = 5 * FT + 123
    x = wl.full_range_u32(n, seed=99)
    for inclusive in (False, True):
        d = dev(x)
        say("in-place", inclusive)
        dw.ps_scan("sum", inclusive, d, d)
        ref, _ = orc.scan_u32(x, "sum", inclusive)
        assert np.array_equal(host(d), ref)


def test_empty_input_writes_identity_total(dw):
    import torch
    d_in = torch.empty(0, dtype=torch.int32, device="cuda")
    for op, ident in (("sum", 0), ("min", 0xFFFFFFFF), ("affine16", 0x10000)):
        tot = torch.full((1,), 12345, dtype=torch.int32, device="cuda")
        dw.ps_scan(op, False, d_in, d_in, tot)
        assert int(host(tot)[0]) == ident
    ftot = torch.zeros(1, dtype=torch.float32, device="cuda")
    dw.ps_scan("max", True, torch.empty(0, dtype=torch.float32, device="cuda"),
               torch.empty(0, dtype=torch.float32, device="cuda"), ftot)
    assert host(ftot)[0] == -np.inf


def test_workspace_reuse_and_error_word(dw, orc):
    """One workspace serves calls of different sizes; the spin-limit error
    word stays clear."""
    import torch
    ws = dw.new_workspace(dw.workspace_bytes("ps_scan_exclusive_u32", None, None, 1 << 22, None, None))
    for n in (1 << 22, 5, FT * 7 + 1, 1 << 22):
        x = wl.full_range_u32(n, seed=n + 3)
        d_in = dev(x)
        d_out = torch.empty_like(d_in)
        dw.ps_scan_exclusive_u32(d_in, d_out, workspace=ws)
        ref, _ = orc.scan_u32(x, "sum", False)
        assert np.array_equal(host(d_out), ref)
        assert ws_error_word(ws) == 0


def test_torch_uint32_tensors(dw, orc):
    """The binding also takes torch.uint32 tensors (created and copied only)."""
    import torch
    x = wl.full_range_u32(FT * 3 + 5, seed=8)
    d_in = torch.from_numpy(x).to("cuda")
    assert d_in.dtype == torch.uint32
    d_out = torch.empty_like(d_in)
    dw.ps_scan_exclusive_u32(d_in, d_out)
    torch.cuda.synchronize()
    ref, _ = orc.scan_u32(x, "sum", False)
    assert np.array_equal(d_out.cpu().numpy(), ref)


def test_non_default_stream(dw, orc):
    import torch
    n = 2_000_003
    x = wl.full_range_u32(n, seed=5)
    s = torch.cuda.Stream()
    d_in = dev(x)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        d_out = torch.empty_like(d_in)
        dw.ps_scan_inclusive_u32(d_in, d_out, stream=s)
    s.synchronize()
    ref, _ = orc.scan_u32(x, "sum", True)
    assert np.array_equal(host(d_out), ref)


def test_calls_without_a_stream_use_the_current_one(dw, orc):
    """A call given no stream runs on the current stream of its tensors'
    device: the handle the binding passes is the one torch.cuda.current_stream
    names, also inside a stream context, and the call's result is exact
    there."""
    import torch
    from device_wide_prefix_chained_amd import _binding as B
    x = wl.full_range_u32(100_003, seed=6)
    d_in = dev(x)
    assert B._raw_stream(d_in, None) == torch.cuda.current_stream().cuda_stream
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        assert B._raw_stream(d_in, None) == s.cuda_stream == torch.cuda.current_stream().cuda_stream
        d_out = torch.empty_like(d_in)
        dw.ps_scan_exclusive_u32(d_in, d_out)
    s.synchronize()
    assert np.array_equal(host(d_out), orc.scan_u32(x, "sum", False)[0])
    assert B._raw_stream(d_in, s) == s.cuda_stream


def test_repeated_runs_stay_exact(dw, orc):
    """Ordering races show up rarely ("Parallel Prefix Sum (Scan), in depth",
    "Failure modes"): 50 back-to-back runs at 2^24 must all be bit-exact."""
    import torch
    n = 1 << 24
    x = wl.uniform_u32(n, 256, seed=11)
    ref, _ = orc.scan_u32(x, "sum", False)
    d_in = dev(x)
    d_out = torch.empty_like(d_in)
    ws = dw.new_workspace(dw.workspace_bytes("ps_scan_exclusive_u32", None, None, n, None, None))
    say("repeat x50", n)
    for it in range(50):
        d_out.fill_(-1)
        dw.ps_scan_exclusive_u32(d_in, d_out, workspace=ws)
        got = host(d_out)
        assert np.array_equal(got, ref), "run %d differs" % it
        assert ws_error_word(ws) == 0


@pytest.mark.parametrize("aggregate_only", [False, True])
def test_lookback_instrumented(dw, orc, aggregate_only):
    """The instrumented kernel gives the same result; with aggregate_only every
    look-back has to slide its 64-wide window back to tile 0."""
    import torch
    tile = dw.ps_tile_elements(0)
    n = 1100 * tile + 77
    x = wl.full_range_u32(n, seed=21)
    tiles = dw.ps_lookback_tiles(n)
    stats = torch.zeros(dw.STATS_WORDS * tiles, dtype=torch.int32, device="cuda")
    d_in = dev(x)
    d_out = torch.empty_like(d_in)
    say("lookback stats", aggregate_only)
    old = dw.ps_lookback_config_get()
    dw.ps_lookback_config(old[0], 0)  # no PARTIAL shortcuts: the plain sliding window
    try:
        dw.ps_lookback_stats_u32(d_in, d_out, stats, aggregate_only=aggregate_only)
    finally:
        dw.ps_lookback_config(*old)
    ref, _ = orc.scan_u32(x, "sum", False)
    assert np.array_equal(host(d_out), ref)
    st = host(stats).reshape(tiles, dw.STATS_WORDS).astype(np.int64)
    assert st[0, 0] == 0 and st[0, 1] == 0  # tile 0 never looks back
    assert np.all(st[1:, 0] >= st[1:, 1])
    t = np.arange(tiles)
    first = (t % dw.ps_lookback_group() == 0) & (t > 0)
    if not aggregate_only:
        # the first tile of each group looks back, the others follow it
        assert np.all(st[first, 1] >= 1) and np.all(st[~first, 0] == 0)
    if aggregate_only:
        t = np.arange(1, tiles)
        win = dw.ps_lookback_window()
        assert np.array_equal(st[1:, 1], (t + win - 1) // win)


def test_small_config_u32(dw, orc):
    """u32 exclusive and inclusive sum scan, n = 2^20, values in [0, 15]."""
    x = wl.small_u32()
    for inclusive in (False, True):
        say("small config", inclusive)
        got, total = _run_u32(dw, x, "sum", inclusive)
        ref, ref_total = orc.scan_u32(x, "sum", inclusive)
        assert np.array_equal(got, ref) and total == ref_total


@pytest.mark.parametrize("n", [wl.N_LARGE_U32, wl.N_RAGGED_U32], ids=["2^28", "2^28-12345"])
def test_large_config_u32(dw, orc, n):
    """u32 exclusive + inclusive sum scan at 2^28 (1 GiB) and the ragged size,
    values in [0, 255]; the totals wrap modulo 2^32 about 8 times."""
    import torch
    x = wl.large_u32()[:n]
    d_in = dev(x)
    d_out = torch.empty_like(d_in)
    tot = torch.zeros(1, dtype=torch.int32, device="cuda")
    for inclusive in (False, True):
        say("large config", n, inclusive)
        (dw.ps_scan_inclusive_u32 if inclusive else dw.ps_scan_exclusive_u32)(d_in, d_out, tot)
        got = host(d_out)
        ref, ref_total = orc.scan_u32(x, "sum", inclusive)
        assert np.array_equal(got, ref)
        assert int(host(tot)[0]) == ref_total
        del got, ref


def test_f32_config(dw, orc):
    """fp32 inclusive sum scan at 2^27 (N(0,1)) within 1e-5 * prefix sum of
    |x| of the fp64 oracle, the exclusive form likewise, and the max scan on
    the same input bit-exact."""
    import torch
    x = wl.f32_normal()
    d_in = dev(x)
    d_out = torch.empty_like(d_in)
    for inclusive in (True, False):
        say("f32 config sum", inclusive)
        (dw.ps_scan_inclusive_f32 if inclusive else dw.ps_scan_exclusive_f32)(d_in, d_out)
        got = host(d_out)
        ref, ab, _ = orc.scan_f32_sum(x, inclusive)
        worst = assert_f32_sum_close(got, ref, ab, exclusive=not inclusive)
        print("worst err/tol", worst)
        del got, ref, ab
    say("f32 config max")
    dw.ps_scan("max", True, d_in, d_out)
    ref, _ = orc.scan_f32_minmax(x, "max", True)
    assert np.array_equal(host(d_out).view(np.uint32), ref.view(np.uint32))
