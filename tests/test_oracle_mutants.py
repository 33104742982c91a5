"""Plant plausible mistakes in copies of the oracle and check that the pins
catch every one (CPU only).

Each mutant copies oracle/oracle.c to a temporary directory, replaces one
snippet (the first occurrence after an anchor), compiles it with gcc and runs
the whole pin suite against it.  A mutant that no pin rejects means the pins
leave that part of the oracle unchecked.
"""
import os
import tempfile

import pytest

import oracle
from pins import PINS

# (name, anchor, snippet, replacement)
MUTANTS = [
    ("scan: exclusive writes after combining", "int oracle_scan_u32(",
     "            y[i] = acc;\n            acc = u32_combine(op, acc, xi);",
     "            acc = u32_combine(op, acc, xi);\n            y[i] = acc;"),
    ("scan: inclusive writes before combining", "int oracle_scan_u32(",
     "            acc = u32_combine(op, acc, xi);\n            y[i] = acc;",
     "            y[i] = acc;\n            acc = u32_combine(op, acc, xi);"),
    ("scan: operands of the combine swapped", "int oracle_scan_u32(",
     "acc = u32_combine(op, acc, xi);", "acc = u32_combine(op, xi, acc);"),
    ("scan: total is the last output", "int oracle_scan_u32(",
     "        *total = acc;", "        *total = n ? y[n - 1] : acc;"),
    ("widening: 32-bit accumulator", "int oracle_scan_u32_u64(",
     "    uint64_t acc = 0u;", "    uint32_t acc = 0u;"),
    ("widening: exclusive writes after adding", "int oracle_scan_u32_u64(",
     "            y[i] = acc;\n            acc = acc + xi;", "            acc = acc + xi;\n            y[i] = acc;"),
    ("widening: input truncated to 16 bits", "int oracle_scan_u32_u64(",
     "        uint64_t xi = (uint64_t)x[i];", "        uint64_t xi = (uint64_t)(x[i] & 0xFFFFu);"),
    ("widening: total misses the last element", "int oracle_scan_u32_u64(",
     "        *total = acc;", "        *total = n ? y[n - 1] : acc;"),
    ("linrec: b term with swapped roles", "int oracle_scan_linrec_f32(",
     "        pb = at * pb + bt;", "        pb = pa * bt + pb;"),
    ("linrec: dropped additive term", "int oracle_scan_linrec_f32(",
     "        pb = at * pb + bt;", "        pb = at * pb;"),
    ("linrec: float accumulator", "int oracle_scan_linrec_f32(",
     "    double pa = 1.0, pb = 0.0;", "    float pa = 1.0f, pb = 0.0f;"),
    ("linrec: exclusive form written inclusive", "int oracle_scan_linrec_f32(",
     "        if (inclusive) {\n            A[t] = pa;", "        if (1) {\n            A[t] = pa;"),
    ("linrec: identity (0, 0)", "int oracle_scan_linrec_f32(",
     "    double pa = 1.0, pb = 0.0;   /* running pair */", "    double pa = 0.0, pb = 0.0;   /* running pair */"),
    ("linrec: magnitudes without fabs", "int oracle_scan_linrec_f32(",
     "        qb = fabs(at) * qb + fabs(bt);", "        qb = at * qb + bt;"),
    ("sum: xor instead of add", "case ORC_SUM:", "return a + b;", "return a ^ b;"),
    ("max: picks the smaller", "case ORC_MAX:", "return (b > a) ? b : a;", "return (b > a) ? a : b;"),
    ("min: identity zero", "static uint32_t u32_identity", "    case ORC_MIN:\n        return 0xFFFFFFFFu;",
     "    case ORC_MIN:\n        return 0u;"),
    ("and: identity zero", "static uint32_t u32_identity", "    case ORC_AND:\n        return 0xFFFFFFFFu;",
     "    case ORC_AND:\n        return 0u;"),
    ("xor: or instead", "case ORC_XOR:", "return a ^ b;", "return a | b;"),
    ("affine16: b term with swapped roles", "case ORC_AFFINE16: {",
     "uint32_t rb = (a2 * b1 + b2) & 0xFFFFu;", "uint32_t rb = (a1 * b2 + b1) & 0xFFFFu;"),
    ("affine16: dropped additive term", "case ORC_AFFINE16: {",
     "uint32_t rb = (a2 * b1 + b2) & 0xFFFFu;", "uint32_t rb = (a2 * b1) & 0xFFFFu;"),
    ("affine16: wrong identity", "static uint32_t u32_identity",
     "return 0x00010000u;", "return 0x00000001u;"),
    ("f32 sum: float accumulator", "int oracle_scan_f32_sum(",
     "    double acc = 0.0;", "    float acc = 0.0f;"),
    ("f32 sum: absolute prefix without fabs", "int oracle_scan_f32_sum(",
     "absacc += fabs(xi);", "absacc += xi;"),
    ("f32 sum: exclusive off by one", "int oracle_scan_f32_sum(",
     "            if (y)\n                y[i] = acc;\n            acc += xi;",
     "            acc += xi;\n            if (y)\n                y[i] = acc;"),
    ("f32 max: ties take the later operand", "int oracle_scan_f32_minmax(",
     "next = (xi > acc) ? xi : acc;", "next = (xi >= acc) ? xi : acc;"),
    ("f32 min: wrong identity", "int oracle_scan_f32_minmax(",
     "float acc = (op == ORC_MAX) ? -INFINITY : INFINITY;", "float acc = (op == ORC_MAX) ? -INFINITY : 0.0f;"),
    ("validate: empty segments rejected", "int64_t oracle_validate_offsets(",
     "if (offsets[s] > offsets[s + 1])", "if (offsets[s] >= offsets[s + 1])"),
    ("validate: terminal offset equal to n rejected", "int64_t oracle_validate_offsets(",
     "if ((uint64_t)offsets[num_segments] > n)", "if ((uint64_t)offsets[num_segments] >= n)"),
    ("segmented: carry crosses the segment boundary", "int64_t oracle_segmented_scan_u32(",
     "        uint32_t acc = 0u;", "        uint32_t acc = (offsets[s] > 0) ? x[offsets[s] - 1] : 0u;"),
    ("segmented: first row of each segment skipped", "int64_t oracle_segmented_scan_u32(",
     "for (uint64_t i = offsets[s];", "for (uint64_t i = offsets[s] + 1;"),
    ("segmented: last row of each segment skipped", "int64_t oracle_segmented_scan_u32(",
     "i < (uint64_t)offsets[s + 1];", "i + 1 < (uint64_t)offsets[s + 1];"),
    ("segmented: inclusive writes before adding", "int64_t oracle_segmented_scan_u32(",
     "                acc += x[i];\n                y[i] = acc;",
     "                y[i] = acc;\n                acc += x[i];"),
    ("compact: destination off by one", "uint64_t oracle_compact(",
     "memcpy(dst + j * record_bytes", "memcpy(dst + (j + 1) * record_bytes"),
    ("compact: keeps the rejected records", "uint64_t oracle_compact(",
     "if (flags[i] != 0)", "if (flags[i] == 0)"),
    ("compact: only flag value 1 counts as keep", "uint64_t oracle_compact(",
     "if (flags[i] != 0)", "if (flags[i] == 1)"),
]


def _mutate(text, anchor, old, new):
    start = text.index(anchor)
    pos = text.index(old, start)
    return text[:pos] + new + text[pos + len(old):]


@pytest.mark.parametrize("mutant", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_reject_mutant(mutant):
    name, anchor, old, new = mutant
    src = open(oracle.SOURCE).read()
    assert anchor in src and old in src[src.index(anchor):], "mutation site vanished: " + name
    with tempfile.TemporaryDirectory() as tmp:
        path = os.path.join(tmp, "oracle_mutant.c")
        with open(path, "w") as f:
            f.write(_mutate(src, anchor, old, new))
        lib = oracle.build(source=path, output=os.path.join(tmp, "liboracle_mutant.so"))
        orc = oracle.Oracle(lib)
        caught = []
        for p in PINS:
            try:
                p(orc)
            except (AssertionError, ValueError):
                caught.append(p.__name__)
        assert caught, "no pin rejects the mutant: " + name
