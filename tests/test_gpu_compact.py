"""Parity of the fused stable compaction (HIP, through the C ABI) with the
oracle: bit-exact records, exact count, untouched slots past the count."""
import numpy as np
import pytest

import workloads as wl
from gpu_util import dev, host, require_gpu, say
from pins import golden

pytestmark = pytest.mark.gpu

FILL = 0xA5A5A5A5


@pytest.fixture(scope="module")
def dw():
    return require_gpu()


def _run(dw, records, flags):
    import torch
    d_out = dev(np.full_like(records, FILL))
    cnt = torch.full((1,), -7, dtype=torch.int64, device="cuda")
    dw.ps_compact(dev(records), dev(flags), d_out, cnt)
    return host(d_out), int(host(cnt)[0])


def _check(dw, orc, records, flags):
    got, count = _run(dw, records, flags)
    ref, ref_count = orc.compact(records, flags, out=np.full_like(records, FILL))
    assert count == ref_count
    assert np.array_equal(got, ref)


def test_worked_examples(dw, orc):
    g = golden("p2_compaction_example.json")
    x = np.array(g["input"], np.int32).view(np.uint32)
    flags = (np.array(g["input"]) > 0).astype(np.uint8)
    say("compaction worked example")
    got, count = _run(dw, x, flags)
    assert count == len(g["output"]) and got[:count].view(np.int32).tolist() == g["output"]
    g = golden("p3_flags_offsets.json")
    flags = np.array(g["flags"], np.uint8)
    got, count = _run(dw, np.arange(len(flags), dtype=np.uint32), flags)
    assert got[:count].tolist() == g["kept_positions"]
    g = golden("p3_exercise_input.json")
    x = np.array(g["input"], np.uint32)
    got, count = _run(dw, x, (x >= 5).astype(np.uint8))
    assert got[:count].tolist() == [v for v in g["input"] if v >= 5]


# the page's edge lengths other than 0 (test_empty covers n = 0), then tile edges
@pytest.mark.parametrize("n", [m for m in golden("p3_exercise_input.json")["edge_lengths"] if m] +
                         [63, 64, 65, 2047, 2048, 2049, 4095, 4096, 4097, 300_007])
@pytest.mark.parametrize("width", [1, 2, 4])
@pytest.mark.parametrize("kind", ["none", "all", "random", "clustered"])
def test_edge_lengths(dw, orc, n, width, kind):
    rec = wl.full_range_u32(n * width, seed=n + width).reshape(n, width)
    if width == 1:
        rec = rec.reshape(n)
    flags = wl.flag_pattern(n, kind, seed=n, run=37)
    if kind == "random":
        flags = flags * wl.uniform_u32(n, 255, seed=n + 1).astype(np.uint8) + flags  # any nonzero keeps
    say("compact", n, width, kind)
    _check(dw, orc, rec, flags)


def test_tile_shape(dw):
    for rb in (4, 8, 16):
        assert dw.ps_compact_tile_records(rb) == 8 * 6 * 64 * (16 // rb)
    assert dw.ps_compact_tile_records(12) == 0


@pytest.mark.parametrize("width", [1, 2, 4])
@pytest.mark.parametrize("rel", [(1, -1), (1, 0), (1, 1), (2, -1), (2, 0), (2, 1), (3, 5), (64, 7), (301, 0)])
@pytest.mark.parametrize("kind", ["none", "all", "random", "clustered"])
def test_tile_relative_lengths(dw, orc, width, rel, kind):
    """Lengths around whole tiles and ticket groups of the compaction kernel
    for each record width (its tile holds 48 KiB of records)."""
    tile = dw.ps_compact_tile_records(4 * width)
    n = rel[0] * tile + rel[1]
    rec = wl.full_range_u32(n * width, seed=n + 3 * width).reshape(n, width)
    if width == 1:
        rec = rec.reshape(n)
    flags = wl.flag_pattern(n, kind, seed=n + 5, run=tile // 3 + 1)
    say("compact tile-relative", width, rel, kind)
    _check(dw, orc, rec, flags)


@pytest.mark.parametrize("width", [1, 2, 4])
def test_unaligned_buffers(dw, orc, width):
    """Flags one byte past an aligned address, and for 4- and 8-byte records
    records that are not 16-byte aligned: the per-record load path."""
    import torch
    n = 3 * dw.ps_compact_tile_records(4 * width) + 77
    rec = wl.full_range_u32(n * width, seed=21 + width).reshape(n, width)
    flags = wl.flag_pattern(n, "random", seed=22 + width)
    d_flags = dev(np.concatenate(([7], flags)).astype(np.uint8))[1:]
    shift = 0 if width == 4 else 1
    full = np.concatenate((np.zeros((shift, width), np.uint32), rec))
    d_rec = dev(full)[shift:]
    d_out = dev(np.full((n + shift, width), FILL, np.uint32))[shift:]
    if width == 1:
        d_rec, d_out = d_rec.reshape(n), d_out.reshape(n)
    assert d_flags.data_ptr() % 2 == 1
    if width < 4:
        assert d_rec.data_ptr() % 16 != 0
    cnt = torch.full((1,), -7, dtype=torch.int64, device="cuda")
    say("compact unaligned", width)
    dw.ps_compact(d_rec, d_flags, d_out, cnt)
    ref, ref_count = orc.compact(rec.reshape(n) if width == 1 else rec, flags,
                                 out=np.full((n,) if width == 1 else (n, width), FILL, np.uint32))
    assert int(host(cnt)[0]) == ref_count
    assert np.array_equal(host(d_out), ref)


def test_empty(dw):
    import torch
    cnt = torch.full((1,), 99, dtype=torch.int64, device="cuda")
    d = torch.empty((0, 4), dtype=torch.int32, device="cuda")
    dw.ps_compact(d, torch.empty(0, dtype=torch.uint8, device="cuda"), d, cnt)
    assert int(host(cnt)[0]) == 0


def test_repeated_runs_stay_exact(dw, orc):
    rec, flags = wl.compaction_records(n=1 << 22, seed=40)
    ref, ref_count = orc.compact(rec, flags, out=np.full_like(rec, FILL))
    for it in range(20):
        say("compact repeat", it)
        got, count = _run(dw, rec, flags)
        assert count == ref_count and np.array_equal(got, ref), it


def test_records_config(dw, orc):
    """2^26 records of 16 bytes {u32 id, u32 key, f32 a, f32 b}, keep flag
    Bernoulli(0.3): dense, stable output and the exact count."""
    rec, flags = wl.compaction_records()
    say("compaction config")
    got, count = _run(dw, rec, flags)
    ref, ref_count = orc.compact(rec, flags, out=np.full_like(rec, FILL))
    assert count == ref_count
    assert np.array_equal(got, ref)
    ids = got[:count, 0]
    assert np.all(ids[1:] > ids[:-1])  # stable: kept ids strictly increasing
