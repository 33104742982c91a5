"""Parity of the segmented scan (HIP, through the C ABI) with the oracle:
bit-exact, including the rows that belong to no segment (left untouched)."""
import numpy as np
import pytest

import workloads as wl
from gpu_util import TILE, dev, host, require_gpu, say, ws_error_word
from pins import golden

pytestmark = pytest.mark.gpu

SENTINEL = 0xDEADBEEF


@pytest.fixture(scope="module")
def dw():
    return require_gpu()


def _run(dw, x, offsets, inclusive, workspace=None):
    d_out = dev(np.full(x.size, SENTINEL, np.uint32))
    dw.ps_segmented_scan_u32(dev(x), dev(offsets), d_out, inclusive=inclusive, workspace=workspace)
    return host(d_out)


def _check(dw, orc, x, offsets, inclusive):
    got = _run(dw, x, offsets, inclusive)
    ref = orc.segmented_scan_u32(x, offsets, inclusive, sentinel=SENTINEL)
    if not np.array_equal(got, ref):
        bad = np.nonzero(got != ref)[0]
        raise AssertionError("%d rows differ, first %d: gpu %d oracle %d"
                             % (bad.size, bad[0], got[bad[0]], ref[bad[0]]))


def test_worked_example(dw, orc):
    g = golden("p5_segmented_example.json")
    x = np.array(g["values"], np.uint32)
    off = np.array(g["offsets"], np.uint32)
    for inclusive, key in ((False, "exclusive"), (True, "inclusive")):
        say("segmented worked example", key)
        assert _run(dw, x, off, inclusive).tolist() == g[key]


@pytest.mark.parametrize("n", [1, 5, 100, TILE - 1, TILE, TILE + 1, 3 * TILE + 7, 100_003, 1_000_003])
@pytest.mark.parametrize("nseg", [1, 2, 17, 1000])
@pytest.mark.parametrize("cover", [True, False])
@pytest.mark.parametrize("inclusive", [False, True])
def test_random_segmentations(dw, orc, n, nseg, cover, inclusive):
    x = wl.full_range_u32(n, seed=n + nseg)
    off = wl.random_segments(n, nseg, seed=n * 7 + nseg, cover=cover)
    say("segmented", n, nseg, cover, inclusive)
    _check(dw, orc, x, off, inclusive)


@pytest.mark.parametrize("inclusive", [False, True])
def test_special_segmentations(dw, orc, inclusive):
    n = 50_000
    x = wl.full_range_u32(n, seed=3)
    cases = {
        "unit segments": np.arange(n + 1, dtype=np.uint32),
        "one segment": np.array([0, n], np.uint32),
        "all empty at 0": np.zeros(9, np.uint32),
        "all empty inside": np.full(5, 777, np.uint32),
        "zero segments": np.array([0], np.uint32),
        "heads on tile edges": np.arange(0, n + 1, TILE, dtype=np.uint32),
        "heads one past tile edges": np.concatenate(([0], np.arange(1, n, TILE), [n])).astype(np.uint32),
        "empties between": np.array([0, 10, 10, 10, TILE, TILE, 3 * TILE, n, n], np.uint32),
        "gap at both ends": np.array([TILE + 5, 2 * TILE, 3 * TILE + 1, n - 100], np.uint32),
        # runs of repeated offsets longer than one 512-entry batch of the
        # start search, inside a tile and on a tile edge
        "long runs of empty segments": np.concatenate(
            ([0], np.full(2000, 777), np.full(1500, TILE), [TILE + 3], np.full(600, n - 1), [n])).astype(np.uint32),
    }
    for name, off in cases.items():
        say("segmented special", name, inclusive)
        _check(dw, orc, x, off, inclusive)


@pytest.mark.parametrize("inclusive", [False, True])
def test_long_segments_chain(dw, orc, inclusive):
    """Segments much longer than a tile: head-free tiles must chain through
    the look-back, and the chain must stop at every head."""
    n = 400 * TILE + 33
    x = wl.full_range_u32(n, seed=4)
    off = np.array([0, 3, 150 * TILE + 1, 150 * TILE + 2, 399 * TILE, n], np.uint32)
    say("long segments", inclusive)
    _check(dw, orc, x, off, inclusive)


def test_tile_shape(dw):
    assert dw.ps_segmented_tile_elements() == TILE


@pytest.mark.parametrize("inclusive", [False, True])
@pytest.mark.parametrize("seed", [1, 2, 3])
def test_tile_level_patterns(dw, orc, inclusive, seed):
    """Every tile gets one of: no start, a start on its first element, one in
    its middle, one on its last element, several, a run of empty segments --
    so that every pairing of neighbours (and of the two tiles of a ticket
    group) occurs, including head-free runs that chain across groups."""
    rng = np.random.default_rng(seed)
    tiles = 97
    n = tiles * TILE - 1234
    starts = []
    for t in range(tiles):
        b = t * TILE
        kind = int(rng.integers(0, 6))
        if kind == 1:
            starts.append(b)
        elif kind == 2:
            starts.append(b + int(rng.integers(1, TILE - 1)))
        elif kind == 3:
            starts.append(b + TILE - 1)
        elif kind == 4:
            starts.extend(sorted(b + rng.choice(TILE, 5, replace=False)))
        elif kind == 5:
            starts.extend([b + 100] * 3)
    # repeated offsets (kind 5, or a start at 0) are empty segments
    off = np.array(sorted([0] + [s for s in starts if s < n] + [n]), np.uint32)
    x = wl.full_range_u32(n, seed=seed + 50)
    say("segmented tile patterns", seed, inclusive, off.size - 1)
    _check(dw, orc, x, off, inclusive)


@pytest.mark.parametrize("inclusive", [False, True])
def test_unaligned_buffers(dw, orc, inclusive):
    """values and out one element past a 16-byte boundary: the 4-byte path."""
    import torch
    n = 7 * TILE + 11
    x = wl.full_range_u32(n, seed=8)
    off = wl.random_segments(n, 40, seed=9, cover=False)
    vx = dev(np.concatenate(([0], x)).astype(np.uint32))[1:]
    vo = dev(np.full(n + 1, SENTINEL, np.uint32))[1:]
    assert vx.data_ptr() % 16 != 0 and vo.data_ptr() % 16 != 0
    say("segmented unaligned", inclusive)
    dw.ps_segmented_scan_u32(vx, dev(off), vo, inclusive=inclusive)
    torch.cuda.synchronize()
    assert np.array_equal(host(vo), orc.segmented_scan_u32(x, off, inclusive, sentinel=SENTINEL))


@pytest.mark.parametrize("inclusive", [False, True])
@pytest.mark.parametrize("nseg", [131071, 131072])
def test_many_segments(dw, orc, inclusive, nseg):
    """2^17 segments over 2^22 + 5 values, about 32 elements per segment: a
    257-entry sample of the offsets, 300-400 starts per tile."""
    n = 32 * 131072 + 5
    x = wl.full_range_u32(n, seed=nseg)
    off = wl.random_segments(n, nseg, seed=nseg + 1, cover=True)
    say("segmented many segments", nseg, inclusive)
    _check(dw, orc, x, off, inclusive)


@pytest.mark.parametrize("inclusive", [False, True])
def test_more_offsets_than_the_sample_brackets(dw, orc, inclusive):
    """2^20 + 7 segments (a fifth of them empty) over 2^22 + 9 values: the
    offsets' sample is capped at 1 024 entries, so its stride exceeds 512 and
    rounds of evenly spaced probes narrow each tile's bracket before the
    contiguous loads; a tile holds about 2 400 starts (several batches)."""
    n = (1 << 22) + 9
    x = wl.full_range_u32(n, seed=91)
    off = wl.random_segments(n, (1 << 20) + 7, seed=92, cover=True)
    say("segmented 2^20 + 7 segments", inclusive)
    _check(dw, orc, x, off, inclusive)


@pytest.mark.parametrize("inclusive", [False, True])
def test_dense_cluster_in_sparse_offsets(dw, orc, inclusive):
    """Mostly long segments with a run of 5000 unit segments and a run of 3000
    two-element segments: tiles holding thousands of starts next to tiles
    holding none."""
    n = 1 << 22
    starts = list(range(0, 700_000, 997))
    starts += list(range(700_000, 705_000))                 # unit segments
    starts += list(range(705_000, 711_000, 2))              # two-element segments
    starts += list(range(711_000, n - 20_000, 1531))
    off = np.array(starts + [n - 20_000], np.uint32)
    x = wl.full_range_u32(n, seed=77)
    say("segmented dense cluster", inclusive)
    _check(dw, orc, x, off, inclusive)


def test_repeated_runs_stay_exact(dw, orc):
    import torch
    values, off = wl.zipf_segments(n=1 << 22, num_segments=1 << 12, seed=12)
    ref = orc.segmented_scan_u32(values, off, False, sentinel=SENTINEL)
    ws = dw.new_workspace(dw.workspace_bytes("ps_segmented_scan_u32", None, values.size, None, off.size - 1,
                                        None, 0, None))
    for it in range(20):
        say("segmented repeat", it)
        got = _run(dw, values, off, False, workspace=ws)
        assert np.array_equal(got, ref), it
        assert ws_error_word(ws) == 0


@pytest.mark.parametrize("inclusive", [False, True])
def test_skewed_config(dw, orc, inclusive):
    """2^26 values in [0, 1023] over 2^16 CSR segments: 10% empty, one holding
    25% of the elements, the rest with rank-size Zipf(1.2) lengths."""
    values, off = wl.zipf_segments()
    say("segmented config", inclusive)
    _check(dw, orc, values, off, inclusive)


def test_validate_offsets(dw, orc):
    import torch
    r = torch.zeros(1, dtype=torch.int64, device="cuda")
    cases = [
        (np.array([0, 2, 5, 6], np.uint32), 6),
        (np.array([0, 0, 0], np.uint32), 0),
        (np.array([0, 3, 2, 6], np.uint32), 6),
        (np.array([0, 2, 5, 7], np.uint32), 6),
        (np.array([5], np.uint32), 4),
        (wl.zipf_segments(n=1 << 20, num_segments=1 << 10, seed=2)[1], 1 << 20),
    ]
    bad = wl.zipf_segments(n=1 << 20, num_segments=1 << 10, seed=2)[1].copy()
    bad[700], bad[701] = bad[701] + 1, bad[700]
    cases.append((bad, 1 << 20))
    for off, n in cases:
        dw.ps_validate_offsets(dev(off), n, r)
        assert int(host(r)[0]) == orc.validate_offsets(off, n)
