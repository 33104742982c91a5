"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds input recipes only: random draws from
``numpy.random.default_rng(seed)`` (PCG64) shaped like the workloads the pages
talk about.  It computes no scan, segmented scan or compaction result; the
oracle and the GPU library each receive the same arrays from here and nothing
else.  (The one running sum below is numpy's ``cumsum`` turning segment
lengths into CSR offsets: that builds an *input* -- any non-decreasing offsets
array is a valid one -- and is not the operation under test.)

Workloads (sizes as named):
  * u32 sum scan, n = 2^20, values uniform in [0, 15]            (seed 1)
  * u32 sum scan, n = 2^28, values uniform in [0, 255]           (seed 2);
    the ragged size 2^28 - 12345 is the prefix of the same array
  * fp32 sum / max scan, n = 2^27, values ~ N(0, 1)               (seed 3)
  * compaction, 2^26 records of 16 bytes {u32 id, u32 key, f32 a, f32 b},
    keep flag ~ Bernoulli(0.3)                                    (seed 4)
  * linear recurrence h[t] = a[t] h[t-1] + b[t], n = 2^27 pairs as two fp32
    planes: decays a uniform in [0.9, 1), inputs b ~ N(0, 1)      (seed 6)
  * segmented u32 scan, 2^26 values uniform in [0, 1023], 2^16 CSR segments:
    10% empty, one holding 25% of the elements, the rest with rank-size
    Zipf(s = 1.2) lengths                                         (seed 5)
"""
from __future__ import annotations

import numpy as np

SEED_SMALL_U32 = 1
SEED_LARGE_U32 = 2
SEED_F32 = 3
SEED_COMPACT = 4
SEED_SEGMENTED = 5
SEED_LINREC = 6

N_SMALL_U32 = 1 << 20
N_LARGE_U32 = 1 << 28
N_RAGGED_U32 = (1 << 28) - 12345
N_F32 = 1 << 27
N_COMPACT = 1 << 26
N_SEGMENTED = 1 << 26
NUM_SEGMENTS = 1 << 16
N_LINREC = 1 << 27


def rng(seed: int) -> np.random.Generator:
    return np.random.default_rng(seed)


def uniform_u32(n: int, high: int, seed: int) -> np.ndarray:
    """n uint32 values uniform in [0, high)."""
    return rng(seed).integers(0, high, size=n, dtype=np.uint32)


def full_range_u32(n: int, seed: int) -> np.ndarray:
    """n uint32 values uniform over all 2^32 bit patterns."""
    return rng(seed).integers(0, 1 << 32, size=n, dtype=np.uint64).astype(np.uint32)


def normal_f32(n: int, seed: int) -> np.ndarray:
    return rng(seed).standard_normal(n, dtype=np.float32)


def small_int_f32(n: int, seed: int, lo: int = -8, hi: int = 8) -> np.ndarray:
    """fp32 values that are small integers in [lo, hi] (exact under any grouping
    while every partial sum stays below 2^24 in magnitude)."""
    return rng(seed).integers(lo, hi + 1, size=n).astype(np.float32)


def small_u32(n: int = N_SMALL_U32, seed: int = SEED_SMALL_U32) -> np.ndarray:
    """u32 scan input, n = 2^20, values uniform in [0, 15]."""
    return uniform_u32(n, 16, seed)


def large_u32(n: int = N_LARGE_U32, seed: int = SEED_LARGE_U32) -> np.ndarray:
    """u32 scan input, n = 2^28 (1 GiB), values uniform in [0, 255].  The ragged
    case uses the first 2^28 - 12345 elements of the same array."""
    return uniform_u32(n, 256, seed)


def f32_normal(n: int = N_F32, seed: int = SEED_F32) -> np.ndarray:
    """fp32 scan input, n = 2^27, values ~ N(0, 1)."""
    return normal_f32(n, seed)


def linrec_pairs(n: int = N_LINREC, seed: int = SEED_LINREC, a_lo: float = 0.9, a_hi: float = 1.0):
    """Return (a, b), two fp32 planes of n recurrence coefficients: a uniform
    in [a_lo, a_hi) (the per-step decay of a recurrent state; a_lo < 0 gives
    signed multipliers), b ~ N(0, 1) (the per-step input)."""
    g = rng(seed)
    a = g.uniform(a_lo, a_hi, size=n).astype(np.float32)
    b = g.standard_normal(n, dtype=np.float32)
    return a, b


RECORD_DTYPE = np.dtype([("id", "<u4"), ("key", "<u4"), ("a", "<f4"), ("b", "<f4")])


def compaction_records(n: int = N_COMPACT, seed: int = SEED_COMPACT, p: float = 0.3):
    """Return (records, flags): records is an (n, 4) uint32 array whose rows are
    16-byte {u32 id = i, u32 key, f32 a, f32 b} records (a, b ~ N(0,1) stored
    bit-for-bit), flags is uint8 with P(flag = 1) = p."""
    g = rng(seed)
    rec = np.empty((n, 4), dtype=np.uint32)
    rec[:, 0] = np.arange(n, dtype=np.uint32)
    rec[:, 1] = g.integers(0, 1 << 32, size=n, dtype=np.uint64).astype(np.uint32)
    rec[:, 2] = g.standard_normal(n, dtype=np.float32).view(np.uint32)
    rec[:, 3] = g.standard_normal(n, dtype=np.float32).view(np.uint32)
    flags = (g.random(n) < p).astype(np.uint8)
    return rec, flags


def flag_pattern(n: int, kind: str, seed: int = 0, p: float = 0.3, run: int = 4096):
    """Keep-flag distributions: 'none', 'all', 'random' (Bernoulli p) and
    'clustered' (alternating runs of length ``run``, starting with a random phase)."""
    if kind == "none":
        return np.zeros(n, dtype=np.uint8)
    if kind == "all":
        return np.ones(n, dtype=np.uint8)
    g = rng(seed)
    if kind == "random":
        return (g.random(n) < p).astype(np.uint8)
    if kind == "clustered":
        phase = int(g.integers(0, 2))
        idx = np.arange(n, dtype=np.int64) // run
        return ((idx + phase) % 2 == 0).astype(np.uint8)
    raise ValueError(kind)


def zipf_segments(n: int = N_SEGMENTED, num_segments: int = NUM_SEGMENTS,
                  seed: int = SEED_SEGMENTED, s: float = 1.2,
                  empty_frac: float = 0.10, giant_frac: float = 0.25):
    """Return (values, offsets) for the skewed segmented workload.

    values: n uint32 uniform in [0, 1023].  Segments: a random permutation picks
    floor(empty_frac * N + 0.5) empty segments and one giant segment holding
    giant_frac * n elements; the other M segments get rank-size Zipf lengths
    proportional to k^-s (k = 1..M) scaled to the remaining elements (floor,
    at least 1, leftover elements to the largest fractional parts), assigned in
    a random order.  offsets has N + 1 entries, offsets[0] = 0, offsets[N] = n.
    """
    g = rng(seed)
    values = g.integers(0, 1024, size=n, dtype=np.uint32)
    perm = g.permutation(num_segments)
    n_empty = int(empty_frac * num_segments + 0.5)
    giant = int(giant_frac * n)
    rest_ids = perm[n_empty + 1:]
    m = rest_ids.size
    remaining = n - giant
    lengths = np.zeros(num_segments, dtype=np.int64)
    lengths[perm[n_empty]] = giant
    if m:
        w = np.arange(1, m + 1, dtype=np.float64) ** (-s)
        real = w / w.sum() * remaining
        base = np.maximum(np.floor(real).astype(np.int64), 1)
        deficit = remaining - int(base.sum())
        if deficit > 0:
            order = np.argsort(-(real - np.floor(real)), kind="stable")
            base[order[:deficit]] += 1
        elif deficit < 0:
            order = np.argsort(-base, kind="stable")
            base[order[:-deficit]] -= 1
        lengths[rest_ids] = base[g.permutation(m)]
    offsets = np.zeros(num_segments + 1, dtype=np.int64)
    np.cumsum(lengths, out=offsets[1:])
    assert offsets[-1] == n
    return values, offsets.astype(np.uint32)


def random_segments(n: int, num_segments: int, seed: int, empty_frac: float = 0.2,
                    cover: bool = True):
    """Small random CSR segmentations for parity tests: ``num_segments``
    segments with random lengths (a fraction of them empty).  With cover=False
    the segments start after a random gap and end before n."""
    g = rng(seed)
    if num_segments == 0:
        return np.zeros(1, dtype=np.uint32)
    lo, hi = 0, n
    if not cover and n > 2:
        lo = int(g.integers(0, n // 4 + 1))
        hi = int(n - g.integers(0, n // 4 + 1))
        hi = max(hi, lo)
    span = hi - lo
    cuts = np.sort(g.integers(0, span + 1, size=num_segments - 1)) if num_segments > 1 else np.zeros(0, np.int64)
    empty = g.random(num_segments - 1) < empty_frac if num_segments > 1 else np.zeros(0, bool)
    # an "empty" segment repeats the previous boundary
    bounds = np.concatenate(([0], cuts, [span])).astype(np.int64)
    for k in range(1, num_segments):
        if empty[k - 1]:
            bounds[k] = bounds[k - 1]   # still non-decreasing: the cuts are sorted
    return (bounds + lo).astype(np.uint32)
