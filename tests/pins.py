"""Pins for the CPU oracle: facts fixed by the pages and by mathematics.

Each pin is a function ``pin(orc)`` that raises AssertionError when the oracle
``orc`` (an ``oracle.Oracle``) disagrees with something that does not come
from the oracle itself:

* worked examples printed on the pages (``tests/golden/*.json``, each with
  its page title and section);
* closed forms (constant and iota inputs, modular wrap-around);
* library routines that compute the same thing another way
  (``numpy.cumsum``, ``numpy.*.accumulate``, ``math.fsum``, numpy boolean
  indexing as the stable CPU filter);
* an O(n^2) brute force that folds every prefix from scratch with Python
  built-ins (``sum``, ``max``, ``min``, ``functools.reduce``) and, for the
  affine-pair operator, by applying the maps to numbers;
* a Blelloch up-sweep/down-sweep written here from its description (a
  reduction tree, then prefixes pushed from the root to the leaves);
* a Hillis-Steele scan written here from its description;
* for the recurrence pair, exact rational arithmetic: the maps h -> a h + b
  composed on numbers, the closed-form sums of products, a tree grouping;
* invariants (last inclusive value = total, differences of the exclusive
  scan = input, reset at every segment start, untouched rows outside).

The same pins are run against deliberately broken builds of the oracle in
``test_oracle_mutants.py``; every planted mistake must trip at least one.
"""
from __future__ import annotations

import functools
import json
import math
import operator
from fractions import Fraction
from pathlib import Path

import numpy as np

GOLDEN = Path(__file__).resolve().parent / "golden"
M32 = 0xFFFFFFFF

PINS = []


def pin(fn):
    PINS.append(fn)
    return fn


def golden(name: str) -> dict:
    return json.loads((GOLDEN / name).read_text())


# --------------------------------------------------------------------------
# Independent references written from the pages' descriptions
# --------------------------------------------------------------------------
def _affine_apply(elems, h):
    """Apply the maps h -> a*h + b (mod 2^16) of the packed elems in order."""
    for e in elems:
        a, b = int(e) >> 16, int(e) & 0xFFFF
        h = (a * h + b) & 0xFFFF
    return h


def _affine_fold(elems):
    """The packed (a, b) of the composition of elems, recovered by evaluating
    it at h = 0 (gives b) and h = 1 (gives a + b)."""
    f0 = _affine_apply(elems, 0)
    f1 = _affine_apply(elems, 1)
    return (((f1 - f0) & 0xFFFF) << 16) | f0


BRUTE_FOLD = {
    "sum": lambda xs: sum(int(v) for v in xs) & M32,
    "max": lambda xs: max((int(v) for v in xs), default=0),
    "min": lambda xs: min((int(v) for v in xs), default=M32),
    "and": lambda xs: functools.reduce(operator.and_, (int(v) for v in xs), M32),
    "or": lambda xs: functools.reduce(operator.or_, (int(v) for v in xs), 0),
    "xor": lambda xs: functools.reduce(operator.xor, (int(v) for v in xs), 0),
    "affine16": _affine_fold,
}
IDENTITY = {"sum": 0, "max": 0, "min": M32, "and": M32, "or": 0, "xor": 0,
            "affine16": 1 << 16}
U32_OPS = list(BRUTE_FOLD)


def _pair_combine(op):
    """Two-operand form of each operator, built from the brute-force folds so
    that it does not restate the oracle's switch."""
    fold = BRUTE_FOLD[op]
    return lambda a, b: fold([a, b])


def brute_force_scan(x, op, inclusive):
    """O(n^2): output i folds x[0..i] (inclusive) or x[0..i-1] (exclusive) anew."""
    fold = BRUTE_FOLD[op]
    n = len(x)
    return [fold(x[: i + 1] if inclusive else x[:i]) for i in range(n)]


def brute_force_wide(x, inclusive):
    """O(n^2) with Python integers (no wrap at all): output i sums x[0..i] or
    x[0..i-1] anew."""
    return [sum(int(v) for v in (x[: i + 1] if inclusive else x[:i])) for i in range(len(x))]


def blelloch_exclusive(x, op):
    """Work-efficient scan from its description ("Blelloch: work-efficient
    up-sweep and down-sweep"; "Work-efficient tree scan"): pad to a power of
    two with the identity, build the reduction tree level by level (each
    parent is left (+) right), give the root the identity, then push prefixes
    down: a left child receives its parent's prefix, a right child the
    parent's prefix combined with the left sibling's subtree total.  Returns
    (exclusive scan of x, total)."""
    comb = _pair_combine(op)
    ident = IDENTITY[op]
    n = len(x)
    size = 1
    while size < n:
        size *= 2
    leaves = [int(v) for v in x] + [ident] * (size - n)
    levels = [leaves]
    while len(levels[-1]) > 1:
        below = levels[-1]
        levels.append([comb(below[2 * j], below[2 * j + 1]) for j in range(len(below) // 2)])
    total = levels[-1][0]
    prefix = [ident]
    for depth in range(len(levels) - 2, -1, -1):
        below = levels[depth]
        nxt = []
        for j, p in enumerate(prefix):
            nxt.append(p)
            nxt.append(comb(p, below[2 * j]))
        prefix = nxt
    return prefix[:n], total


def hillis_steele_steps(x):
    """Inclusive sum scan by distance doubling ("Hillis-Steele: short span,
    too much work"): at distance d every element at i >= d adds the OLD value
    d places to its left.  Returns the array after each step."""
    cur = [int(v) for v in x]
    steps = []
    d = 1
    while d < len(cur):
        cur = [cur[i] + (cur[i - d] if i >= d else 0) for i in range(len(cur))]
        steps.append(cur)
        d *= 2
    return steps


def _u32(v):
    return np.asarray(v, dtype=np.uint32)


# --------------------------------------------------------------------------
# Flat uint32 scans
# --------------------------------------------------------------------------
@pin
def pin_worked_examples_flat(orc):
    for name in ("p1_lead_scan.json", "p3_inclusive_exclusive.json", "p5_flat_example.json"):
        g = golden(name)
        x = _u32(g["input"])
        ex, tex = orc.scan_u32(x, "sum", inclusive=False)
        inc, tin = orc.scan_u32(x, "sum", inclusive=True)
        assert ex.tolist() == g["exclusive"], name
        assert inc.tolist() == g["inclusive"], name
        assert tex == tin == g["inclusive"][-1], name


@pin
def pin_hillis_steele_trace(orc):
    g = golden("p2_hillis_steele_trace.json")
    steps = hillis_steele_steps(g["input"])
    assert steps == g["steps"]
    inc, _ = orc.scan_u32(_u32(g["input"]), "sum", inclusive=True)
    assert inc.tolist() == g["steps"][-1]


@pin
def pin_blelloch_printed_result(orc):
    g = golden("p2_blelloch_result.json")
    ref, total = blelloch_exclusive(g["input"], "sum")
    assert ref == g["exclusive"] and total == g["total"]
    ex, tex = orc.scan_u32(_u32(g["input"]), "sum", inclusive=False)
    assert ex.tolist() == g["exclusive"] and tex == g["total"]


@pin
def pin_lengths_to_offsets(orc):
    g = golden("p3_lengths_offsets.json")
    ex, total = orc.scan_u32(_u32(g["lengths"]), "sum", inclusive=False)
    assert ex.tolist() == g["offsets"] and total == g["total"]


@pin
def pin_brute_force_all_ops(orc):
    r = np.random.default_rng(101)
    for op in U32_OPS:
        for n in (0, 1, 2, 3, 7, 17, 64):
            for hi in (16, 1 << 32):
                x = r.integers(0, hi, size=n, dtype=np.uint64).astype(np.uint32)
                for inclusive in (False, True):
                    y, total = orc.scan_u32(x, op, inclusive)
                    assert y.tolist() == brute_force_scan(x.tolist(), op, inclusive), (op, n, inclusive)
                    assert total == BRUTE_FOLD[op](x.tolist()), (op, n, inclusive)


@pin
def pin_blelloch_random_all_ops(orc):
    r = np.random.default_rng(202)
    for op in U32_OPS:
        for n in (1, 8, 64, 100, 256, 1000):
            x = r.integers(0, 1 << 32, size=n, dtype=np.uint64).astype(np.uint32)
            ref, total = blelloch_exclusive(x.tolist(), op)
            y, t = orc.scan_u32(x, op, inclusive=False)
            assert y.tolist() == ref and t == total, (op, n)


@pin
def pin_numpy_accumulate(orc):
    r = np.random.default_rng(303)
    n = 100_003
    x = r.integers(0, 1 << 32, size=n, dtype=np.uint64).astype(np.uint32)
    lib = {
        "sum": lambda v: np.cumsum(v, dtype=np.uint32),
        "max": np.maximum.accumulate,
        "min": np.minimum.accumulate,
        "and": np.bitwise_and.accumulate,
        "or": np.bitwise_or.accumulate,
        "xor": np.bitwise_xor.accumulate,
    }
    for op, f in lib.items():
        ref_inc = f(x).astype(np.uint32)
        inc, tin = orc.scan_u32(x, op, inclusive=True)
        assert np.array_equal(inc, ref_inc), op
        ex, tex = orc.scan_u32(x, op, inclusive=False)
        assert ex[0] == IDENTITY[op] and np.array_equal(ex[1:], ref_inc[:-1]), op
        assert tin == tex == int(ref_inc[-1]), op


@pin
def pin_closed_forms(orc):
    for c in (1, 3, 0x9E3779B9, M32):
        n = 5000
        ex, total = orc.scan_u32(np.full(n, c, np.uint32), "sum", inclusive=False)
        assert ex.tolist() == [(c * i) & M32 for i in range(n)], c
        assert total == (c * n) & M32
    n = 1 << 17  # iota: exclusive[i] = i (i - 1) / 2, which wraps past 2^32
    ex, total = orc.scan_u32(np.arange(n, dtype=np.uint32), "sum", inclusive=False)
    i = np.arange(n, dtype=object)
    assert ex.tolist() == [int(v) & M32 for v in i * (i - 1) // 2]
    assert total == (n * (n - 1) // 2) & M32
    srt = np.sort(np.random.default_rng(7).integers(0, 1 << 32, 999, dtype=np.uint64)).astype(np.uint32)
    inc, _ = orc.scan_u32(srt, "max", inclusive=True)
    assert np.array_equal(inc, srt)
    inc, _ = orc.scan_u32(srt[::-1].copy(), "min", inclusive=True)
    assert np.array_equal(inc, srt[::-1])


# --------------------------------------------------------------------------
# Widening uint32 -> uint64 sum scan
# --------------------------------------------------------------------------
@pin
def pin_widening_worked_examples(orc):
    for name in ("p1_lead_scan.json", "p3_inclusive_exclusive.json", "p5_flat_example.json",
                 "p3_lengths_offsets.json"):
        g = golden(name)
        x = _u32(g["input"] if "input" in g else g["lengths"])
        ex, tex = orc.scan_u32_u64(x, inclusive=False)
        ref_ex = g["exclusive"] if "exclusive" in g else g["offsets"]
        assert ex.tolist() == ref_ex, name
        if "inclusive" in g:
            inc, tin = orc.scan_u32_u64(x, inclusive=True)
            assert inc.tolist() == g["inclusive"] and tin == tex == g["inclusive"][-1], name


@pin
def pin_widening_brute_force_and_numpy(orc):
    r = np.random.default_rng(505)
    for n in (0, 1, 2, 5, 64, 1000):
        x = r.integers(0, 1 << 32, size=n, dtype=np.uint64).astype(np.uint32)
        for inclusive in (False, True):
            y, total = orc.scan_u32_u64(x, inclusive)
            assert y.dtype == np.uint64
            assert y.tolist() == brute_force_wide(x.tolist(), inclusive), (n, inclusive)
            assert total == sum(int(v) for v in x.tolist())
    n = 200_003  # full-range values: the sums pass 2^32 after a couple of elements
    x = r.integers(0, 1 << 32, size=n, dtype=np.uint64).astype(np.uint32)
    ref_inc = np.cumsum(x.astype(np.uint64), dtype=np.uint64)
    inc, tin = orc.scan_u32_u64(x, inclusive=True)
    ex, tex = orc.scan_u32_u64(x, inclusive=False)
    assert np.array_equal(inc, ref_inc) and ex[0] == 0 and np.array_equal(ex[1:], ref_inc[:-1])
    assert tin == tex == int(ref_inc[-1]) == sum(int(v) for v in x.tolist())


@pin
def pin_widening_closed_forms(orc):
    n = 1 << 17
    for c in (1, 0x9E3779B9, M32):  # constant input: exclusive[i] = c * i, no wrap below 2^64
        ex, total = orc.scan_u32_u64(np.full(n, c, np.uint32), inclusive=False)
        assert ex.tolist() == [c * i for i in range(n)], c
        assert total == c * n
    ex, total = orc.scan_u32_u64(np.arange(n, dtype=np.uint32), inclusive=False)  # iota
    assert ex.tolist() == [i * (i - 1) // 2 for i in range(n)]
    assert total == n * (n - 1) // 2
    # the low 32 bits are the wrapping uint32 scan
    x = np.random.default_rng(606).integers(0, 1 << 32, size=50_000, dtype=np.uint64).astype(np.uint32)
    for inclusive in (False, True):
        wide, _ = orc.scan_u32_u64(x, inclusive)
        narrow, _ = orc.scan_u32(x, "sum", inclusive)
        assert np.array_equal((wide & np.uint64(M32)).astype(np.uint32), narrow)


@pin
def pin_invariants_u32(orc):
    r = np.random.default_rng(404)
    x = r.integers(0, 1 << 32, size=65_537, dtype=np.uint64).astype(np.uint32)
    ex, tex = orc.scan_u32(x, "sum", inclusive=False)
    inc, tin = orc.scan_u32(x, "sum", inclusive=True)
    assert tin == tex == int(inc[-1])
    assert np.array_equal((ex[1:] - ex[:-1]).astype(np.uint32), x[:-1])
    assert np.array_equal((ex + x).astype(np.uint32), inc)
    assert ex[0] == 0


@pin
def pin_affine16_semantics(orc):
    """The affine-pair scan composes maps h -> a h + b in input order: the
    inclusive output at i, applied to any h, equals applying maps 0..i."""
    r = np.random.default_rng(505)
    x = r.integers(0, 1 << 32, size=300, dtype=np.uint64).astype(np.uint32)
    inc, total = orc.scan_u32(x, "affine16", inclusive=True)
    for i in (0, 1, 2, 5, 50, 299):
        for h in (0, 1, 12345, 65535):
            a, b = int(inc[i]) >> 16, int(inc[i]) & 0xFFFF
            assert (a * h + b) & 0xFFFF == _affine_apply(x[: i + 1].tolist(), h), (i, h)
    assert total == int(inc[-1])


@pin
def pin_associativity_and_order(orc):
    """Random triples are associative for every operator; the affine pair is
    not commutative, so the scan must keep operands in order."""
    r = np.random.default_rng(606)

    def fold(op, v):
        return orc.scan_u32(_u32(v), op, inclusive=True)[1]

    for op in U32_OPS:
        for _ in range(200):
            a, b, c = (int(v) for v in r.integers(0, 1 << 32, size=3, dtype=np.uint64))
            left = fold(op, [fold(op, [a, b]), c])
            right = fold(op, [a, fold(op, [b, c])])
            assert left == right == fold(op, [a, b, c]), (op, a, b, c)
    swapped = 0
    for _ in range(50):
        a, b = (int(v) for v in r.integers(0, 1 << 32, size=2, dtype=np.uint64))
        swapped += fold("affine16", [a, b]) != fold("affine16", [b, a])
    assert swapped > 40


# --------------------------------------------------------------------------
# fp32 scans
# --------------------------------------------------------------------------
@pin
def pin_f32_sum_vs_numpy_fp64(orc):
    x = np.random.default_rng(707).standard_normal(200_001, dtype=np.float32)
    x64 = x.astype(np.float64)
    ref = np.cumsum(x64)  # sequential running sum in float64
    inc, ab, tin = orc.scan_f32_sum(x, inclusive=True)
    assert np.array_equal(inc, ref)
    assert np.array_equal(ab, np.cumsum(np.abs(x64)))
    ex, ab2, tex = orc.scan_f32_sum(x, inclusive=False)
    assert ex[0] == 0.0 and np.array_equal(ex[1:], ref[:-1])
    assert np.array_equal(ab2, ab)
    assert tin == tex == ref[-1]
    for i in (0, 1, 999, 77_777, 200_000):  # close to the exactly rounded prefix
        exact = math.fsum(x64[: i + 1].tolist())
        assert abs(inc[i] - exact) <= 1e-12 * ab[i] + 1e-300, i


@pin
def pin_f32_sum_small_integers_exact(orc):
    x = np.random.default_rng(808).integers(-8, 9, size=50_000).astype(np.float32)
    inc, _, _ = orc.scan_f32_sum(x, inclusive=True)
    ints = np.cumsum(x.astype(np.int64))
    assert np.array_equal(inc, ints.astype(np.float64))


@pin
def pin_f32_wide_accumulator_page_example(orc):
    g = golden("p2_fp16_accumulator.json")
    x = np.full(g["count"], np.float16(g["value"]), dtype=np.float32)
    inc, _, total = orc.scan_f32_sum(x, inclusive=True)
    assert total == g["wide_accumulator_sum"] and inc[-1] == g["wide_accumulator_sum"]
    h = np.float16(0.0)  # the page's float16 running sum, for contrast
    for v in x.astype(np.float16):
        h = np.float16(h + v)
    assert float(h) == g["fp16_running_sum"]


@pin
def pin_f32_minmax(orc):
    x = np.random.default_rng(909).standard_normal(100_000, dtype=np.float32)
    for op, f, ident in (("max", np.maximum.accumulate, -np.inf), ("min", np.minimum.accumulate, np.inf)):
        inc, tin = orc.scan_f32_minmax(x, op, inclusive=True)
        ref = f(x)
        assert np.array_equal(inc.view(np.uint32), ref.view(np.uint32)), op
        ex, tex = orc.scan_f32_minmax(x, op, inclusive=False)
        assert ex[0] == ident and np.array_equal(ex[1:].view(np.uint32), ref[:-1].view(np.uint32)), op
        assert tin == tex == float(ref[-1])
    # ties keep the earlier operand, so signed zeros resolve by position
    z = np.array([0.0, -0.0, 0.0], dtype=np.float32)
    for op in ("max", "min"):
        inc, _ = orc.scan_f32_minmax(z, op, inclusive=True)
        assert np.signbit(inc).tolist() == [False, False, False], op
        inc, _ = orc.scan_f32_minmax(-z, op, inclusive=True)
        assert np.signbit(inc).tolist() == [True, True, True], op


# --------------------------------------------------------------------------
# Linear recurrence h[t] = a[t] h[t-1] + b[t] as a scan of (a, b) pairs
# ("Parallel Prefix Sum (Scan), in depth", section "What scan builds")
# --------------------------------------------------------------------------
def _maps_fold_exact(pairs):
    """Compose the maps h -> a h + b of `pairs` in order with exact rationals
    and read the composition back as (A, B) by evaluating it at h = 0 (B) and
    h = 1 (A + B).  No use of the pair formula."""
    def apply(h):
        for a, b in pairs:
            h = Fraction(a) * h + Fraction(b)
        return h
    f0, f1 = apply(Fraction(0)), apply(Fraction(1))
    return f1 - f0, f0


def _linrec_closed_exact(a, b, t):
    """A_t = prod_{k<=t} a_k, B_t = sum_j b_j prod_{j<k<=t} a_k (exact), and
    the same sums over |a|, |b|."""
    A = math.prod((Fraction(float(v)) for v in a[: t + 1]), start=Fraction(1))
    B = Fraction(0)
    SB = Fraction(0)
    for j in range(t + 1):
        tail = math.prod((Fraction(float(v)) for v in a[j + 1: t + 1]), start=Fraction(1))
        B += Fraction(float(b[j])) * tail
        SB += abs(Fraction(float(b[j]))) * abs(tail)
    return A, B, abs(A), SB


def _linrec_tree_exact(pairs):
    """Inclusive scan by a balanced tree: each output folds a left and a right
    subtree's compositions, each computed by _maps_fold_exact.  Exact, so it
    must agree with any correct grouping."""
    out = []
    for t in range(len(pairs)):
        mid = (t + 1) // 2
        la, lb = _maps_fold_exact(pairs[:mid])
        ra, rb = _maps_fold_exact(pairs[mid: t + 1])
        out.append(_maps_fold_exact([(la, lb), (ra, rb)]))
    return out


@pin
def pin_linrec_page_example(orc):
    g = golden("p2_recurrence_example.json")
    ab = np.stack([np.array(g["a"], np.float32), np.array(g["b"], np.float32)], axis=1)
    A, B, sa, sb, tot = orc.scan_linrec_f32(ab, inclusive=True)
    # the page's decimals are the recurrence on a = 0.9, 0.1 exactly; the
    # float32 inputs differ from them by < 2^-24 relative
    assert np.allclose(B, g["h"], rtol=3e-7, atol=0), B
    assert np.allclose(A, np.cumprod(np.array(g["a"], np.float64)), rtol=3e-7, atol=0)
    pairs = [(float(x), float(y)) for x, y in ab]
    for t in range(len(pairs)):
        ea, eb = _maps_fold_exact(pairs[: t + 1])
        assert abs(B[t] - eb) <= 1e-15 * abs(eb) and abs(A[t] - ea) <= 1e-15 * abs(ea), t
    assert tot == (A[-1], B[-1])
    E_A, E_B, _, _, etot = orc.scan_linrec_f32(ab, inclusive=False)
    assert (E_A[0], E_B[0]) == (1.0, 0.0)
    assert np.array_equal(E_A[1:], A[:-1]) and np.array_equal(E_B[1:], B[:-1]) and etot == tot


@pin
def pin_linrec_brute_force_exact(orc):
    """Against exact closed forms and an exact tree grouping; the fp64 oracle
    must sit within the rounding bound 4 (t+1) 2^-53 of the magnitude sum."""
    r = np.random.default_rng(1301)
    for n in (0, 1, 2, 3, 7, 33, 70):
        a = r.uniform(-1.25, 1.25, size=n).astype(np.float32)
        b = r.standard_normal(n).astype(np.float32)
        ab = np.stack([a, b], axis=1).reshape(n, 2)
        A, B, sa, sb, (ta, tb) = orc.scan_linrec_f32(ab, inclusive=True)
        E_A, E_B, esa, esb, etot = orc.scan_linrec_f32(ab, inclusive=False)
        tree = _linrec_tree_exact([(float(x), float(y)) for x, y in ab])
        for t in range(n):
            xa, xb, xsa, xsb = _linrec_closed_exact(a, b, t)
            eps = 4 * (t + 1) * 2.0 ** -53
            assert tree[t] == (xa, xb), (n, t)
            assert abs(Fraction(A[t]) - xa) <= eps * xsa, (n, t)
            assert abs(Fraction(B[t]) - xb) <= eps * xsb, (n, t)
            assert abs(Fraction(sa[t]) - xsa) <= eps * xsa and abs(Fraction(sb[t]) - xsb) <= eps * xsb, (n, t)
            if t + 1 < n:
                assert (E_A[t + 1], E_B[t + 1], esa[t + 1], esb[t + 1]) == (A[t], B[t], sa[t], sb[t])
        if n:
            assert (E_A[0], E_B[0], esa[0], esb[0]) == (1.0, 0.0, 1.0, 0.0)
            assert (ta, tb) == etot == (A[-1], B[-1])
        else:
            assert (ta, tb) == etot == (1.0, 0.0)


@pin
def pin_linrec_closed_forms(orc):
    r = np.random.default_rng(1302)
    n = 100_000
    b = r.standard_normal(n).astype(np.float32)
    a = r.uniform(0.5, 1.0, size=n).astype(np.float32)
    # a = 1: plain prefix sums of b; products stay 1
    A, B, _, sb, _ = orc.scan_linrec_f32(np.stack([np.ones(n, np.float32), b], 1))
    assert np.array_equal(B, np.cumsum(b.astype(np.float64))) and np.all(A == 1.0)
    assert np.array_equal(sb, np.cumsum(np.abs(b.astype(np.float64))))
    # b = 0: h stays 0, A = prefix products of a
    A, B, sa, _, _ = orc.scan_linrec_f32(np.stack([a, np.zeros(n, np.float32)], 1))
    assert np.all(B == 0.0) and np.array_equal(A, np.cumprod(a.astype(np.float64)))
    assert np.array_equal(sa, A)
    # a = 0: the recurrence forgets, h[t] = b[t]
    A, B, _, _, _ = orc.scan_linrec_f32(np.stack([np.zeros(n, np.float32), b], 1))
    assert np.array_equal(B, b.astype(np.float64)) and np.all(A == 0.0)
    # constant (c, beta): geometric series beta (1 - c^(t+1)) / (1 - c)
    for c, beta in ((0.5, 1.0), (0.99951171875, -3.0), (-0.75, 2.0)):
        m = 5000
        A, B, _, _, _ = orc.scan_linrec_f32(np.tile(np.array([[c, beta]], np.float32), (m, 1)))
        t = np.arange(1, m + 1, dtype=np.float64)
        geo = beta * (1.0 - c ** t) / (1.0 - c)
        assert np.allclose(B, geo, rtol=1e-12, atol=1e-12 * abs(beta)), c
        assert np.allclose(A, c ** t, rtol=1e-11, atol=1e-300), c
    # nonnegative pairs: the magnitude scan is the scan itself
    ab = np.stack([a, np.abs(b)], 1)
    A, B, sa, sb, _ = orc.scan_linrec_f32(ab)
    assert np.array_equal(A, sa) and np.array_equal(B, sb)
    # signed inputs: the magnitude scan bounds the scan
    A, B, sa, sb, _ = orc.scan_linrec_f32(np.stack([-a, b], 1))
    assert np.all(np.abs(B) <= sb) and np.all(np.abs(A) <= sa)


@pin
def pin_linrec_order(orc):
    """The pair operator is associative but not commutative: folding two
    pairs must compose their maps in index order."""
    r = np.random.default_rng(1303)
    differ = 0
    for _ in range(100):
        x = r.uniform(-2, 2, size=2).astype(np.float32)
        y = r.uniform(-2, 2, size=2).astype(np.float32)
        _, _, _, _, xy = orc.scan_linrec_f32(np.stack([x, y]), want_abs=False)
        _, _, _, _, yx = orc.scan_linrec_f32(np.stack([y, x]), want_abs=False)
        ea, eb = _maps_fold_exact([(float(x[0]), float(x[1])), (float(y[0]), float(y[1]))])
        assert abs(Fraction(xy[0]) - ea) <= 2.0 ** -52 * abs(ea)
        assert abs(Fraction(xy[1]) - eb) <= 2.0 ** -51 * (abs(ea) + abs(eb) + 4)
        differ += xy != yx
    assert differ > 90


# --------------------------------------------------------------------------
# Segmented scan
# --------------------------------------------------------------------------
@pin
def pin_segmented_worked_example(orc):
    g = golden("p5_segmented_example.json")
    for inclusive, key in ((False, "exclusive"), (True, "inclusive")):
        y = orc.segmented_scan_u32(_u32(g["values"]), _u32(g["offsets"]), inclusive)
        assert y.tolist() == g[key], key


@pin
def pin_segmented_reduces_to_library(orc):
    r = np.random.default_rng(1001)
    sentinel = 0xDEADBEEF
    for trial in range(30):
        n = int(r.integers(0, 3000))
        nseg = int(r.integers(1, 60))
        x = r.integers(0, 1 << 32, size=n, dtype=np.uint64).astype(np.uint32)
        offs = _random_offsets(r, n, nseg, cover=bool(trial % 2))
        for inclusive in (False, True):
            y = orc.segmented_scan_u32(x, offs, inclusive, sentinel=sentinel)
            written = np.zeros(n, bool)
            for s in range(nseg):
                lo, hi = int(offs[s]), int(offs[s + 1])
                seg = np.cumsum(x[lo:hi], dtype=np.uint32)
                if not inclusive:
                    seg = np.concatenate(([0], seg[:-1])).astype(np.uint32) if hi > lo else seg
                assert np.array_equal(y[lo:hi], seg), (trial, s)
                if hi > lo:
                    if not inclusive:
                        assert y[lo] == 0
                    else:
                        assert y[hi - 1] == np.sum(x[lo:hi], dtype=np.uint32)
                written[lo:hi] = True
            assert np.all(y[~written] == sentinel), trial


def _random_offsets(r, n, nseg, cover=True):
    """Random non-decreasing offsets (about 30% empty segments); with
    cover=False the segments leave a gap at both ends of the array."""
    lo = 0 if cover else int(r.integers(0, n // 3 + 1))
    hi = n if cover else int(r.integers(lo, n + 1))
    b = np.concatenate(([lo], np.sort(r.integers(lo, hi + 1, size=nseg - 1)), [hi])).astype(np.int64)
    for k in range(1, nseg):
        if r.random() < 0.3:
            b[k] = b[k - 1]
    return b.astype(np.uint32)


@pin
def pin_segmented_special_cases(orc):
    r = np.random.default_rng(1102)
    x = r.integers(0, 1 << 32, size=777, dtype=np.uint64).astype(np.uint32)
    # one segment over everything is the flat scan (numpy.cumsum)
    one = _u32([0, 777])
    assert np.array_equal(orc.segmented_scan_u32(x, one, True), np.cumsum(x, dtype=np.uint32))
    # every segment of length 1: exclusive all zero, inclusive = x
    unit = np.arange(778, dtype=np.uint32)
    assert not orc.segmented_scan_u32(x, unit, False, sentinel=7).any()
    assert np.array_equal(orc.segmented_scan_u32(x, unit, True), x)
    # empty segments write nothing; all-empty offsets leave every row untouched
    empties = _u32([0, 0, 0, 300, 300, 777, 777])
    y = orc.segmented_scan_u32(x, empties, True, sentinel=5)
    assert np.array_equal(y[:300], np.cumsum(x[:300], dtype=np.uint32))
    assert np.array_equal(y[300:], np.cumsum(x[300:], dtype=np.uint32))
    assert np.all(orc.segmented_scan_u32(x, _u32([100, 100, 100]), False, sentinel=9) == 9)
    # zero segments: nothing written
    assert np.all(orc.segmented_scan_u32(x, _u32([0]), False, sentinel=3) == 3)


@pin
def pin_validate_offsets(orc):
    assert orc.validate_offsets(_u32([0, 2, 5, 6]), 6) == -1
    assert orc.validate_offsets(_u32([0, 0, 0]), 0) == -1
    assert orc.validate_offsets(_u32([0, 2, 2, 6]), 6) == -1
    assert orc.validate_offsets(_u32([0, 3, 2, 6]), 6) == 1
    assert orc.validate_offsets(_u32([0, 2, 5, 7]), 6) == 3
    assert orc.validate_offsets(_u32([5]), 4) == 0
    try:
        orc.segmented_scan_u32(_u32([1, 2, 3]), _u32([0, 2, 1, 3]), False)
    except ValueError:
        pass
    else:
        raise AssertionError("non-monotonic offsets must be rejected")


# --------------------------------------------------------------------------
# Compaction
# --------------------------------------------------------------------------
@pin
def pin_compaction_worked_examples(orc):
    g = golden("p2_compaction_example.json")
    x = np.array(g["input"], dtype=np.int32)
    flags = (x > 0).astype(np.uint8)
    assert flags.tolist() == g["flags"]
    off, total = orc.scan_u32(flags.astype(np.uint32), "sum", inclusive=False)
    assert off.tolist() == g["offsets"]
    out, count = orc.compact(x, flags)
    assert count == len(g["output"]) == total
    assert out[:count].tolist() == g["output"]

    g = golden("p3_flags_offsets.json")
    flags = np.array(g["flags"], np.uint8)
    off, _ = orc.scan_u32(flags.astype(np.uint32), "sum", inclusive=False)
    assert off.tolist() == g["offsets"]
    out, count = orc.compact(np.arange(len(flags), dtype=np.uint32), flags)
    assert out[:count].tolist() == g["kept_positions"]
    assert [int(off[p]) for p in g["kept_positions"]] == g["destinations"]
    assert count == int(off[-1]) + int(flags[-1])

    g = golden("p3_exercise_input.json")
    x = np.array(g["input"], dtype=np.uint32)
    keep = [v for v in g["input"] if v >= 5]  # stable CPU filter
    out, count = orc.compact(x, (x >= 5).astype(np.uint8))
    assert count == len(keep) and out[:count].tolist() == keep


@pin
def pin_compaction_vs_stable_filter(orc):
    r = np.random.default_rng(1203)
    g = golden("p3_exercise_input.json")
    for n in g["edge_lengths"]:
        for width in (1, 2, 4):
            rec = r.integers(0, 1 << 32, size=(n, width), dtype=np.uint64).astype(np.uint32)
            for kind in ("none", "all", "random", "clustered"):
                if kind == "none":
                    f = np.zeros(n, np.uint8)
                elif kind == "all":
                    f = np.ones(n, np.uint8)
                elif kind == "random":
                    f = (r.random(n) < 0.3).astype(np.uint8) * r.integers(1, 256, size=n).astype(np.uint8)
                else:
                    f = ((np.arange(n) // 37) % 2).astype(np.uint8)
                sentinel = np.full_like(rec, 0xA5A5A5A5)
                out, count = orc.compact(rec, f, out=sentinel)
                ref = rec[f != 0]
                assert count == ref.shape[0], (n, width, kind)
                assert np.array_equal(out[:count], ref), (n, width, kind)
                assert np.all(out[count:] == 0xA5A5A5A5), (n, width, kind)
