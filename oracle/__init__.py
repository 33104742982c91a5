"""Sequential CPU oracle for the device-wide prefix scan (TEST INFRASTRUCTURE).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or calls it, and it never imports
the product path.

The arithmetic lives in ``oracle.c`` (plain C, one element at a time, in index
order); this module only marshals numpy arrays into it through ctypes and
builds the shared object with gcc when it is missing.  See ``oracle.c`` for
the page and section each routine follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "oracle.c")
LIBRARY = os.path.join(HERE, "liboracle.so")

# Operator codes of oracle.c (its own numbering, independent of the library).
_OPS = {"sum": 0, "max": 1, "min": 2, "and": 3, "or": 4, "xor": 5, "affine16": 6}

_build_lock = threading.Lock()


def build(source: str = SOURCE, output: str = LIBRARY) -> str:
    """Compile ``source`` with gcc -O2 into the shared object ``output``."""
    tmp = output + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
           "-o", tmp, source, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, output)
    return output


def _needs_build(lib: str, src: str) -> bool:
    return (not os.path.exists(lib)) or os.path.getmtime(lib) < os.path.getmtime(src)


def _ptr(a: np.ndarray | None):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


class Oracle:
    """ctypes view of one build of oracle.c (the real one, or a test mutant)."""

    def __init__(self, lib_path: str = LIBRARY):
        if lib_path == LIBRARY:
            with _build_lock:
                if _needs_build(LIBRARY, SOURCE):
                    build()
        self.path = lib_path
        lib = ctypes.CDLL(lib_path)
        vp, u64, i32 = ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int
        lib.oracle_scan_u32.argtypes = [i32, i32, vp, vp, u64, vp]
        lib.oracle_scan_u32.restype = i32
        lib.oracle_scan_u32_u64.argtypes = [i32, vp, vp, u64, vp]
        lib.oracle_scan_u32_u64.restype = i32
        lib.oracle_scan_linrec_f32.argtypes = [i32, vp, vp, vp, vp, vp, u64, vp, vp]
        lib.oracle_scan_linrec_f32.restype = i32
        lib.oracle_scan_f32_sum.argtypes = [i32, vp, vp, vp, u64, vp]
        lib.oracle_scan_f32_sum.restype = i32
        lib.oracle_scan_f32_minmax.argtypes = [i32, i32, vp, vp, u64, vp]
        lib.oracle_scan_f32_minmax.restype = i32
        lib.oracle_validate_offsets.argtypes = [vp, ctypes.c_uint32, u64]
        lib.oracle_validate_offsets.restype = ctypes.c_int64
        lib.oracle_segmented_scan_u32.argtypes = [i32, vp, u64, vp, ctypes.c_uint32, vp]
        lib.oracle_segmented_scan_u32.restype = ctypes.c_int64
        lib.oracle_compact.argtypes = [vp, ctypes.c_uint32, vp, u64, vp]
        lib.oracle_compact.restype = u64
        self.lib = lib

    # -- flat scans ---------------------------------------------------------
    def scan_u32(self, x, op: str = "sum", inclusive: bool = False, out=None):
        """Return (y, total) for a uint32 scan with operator ``op``."""
        x = np.ascontiguousarray(x, dtype=np.uint32)
        y = np.empty_like(x) if out is None else out
        total = np.zeros(1, dtype=np.uint32)
        rc = self.lib.oracle_scan_u32(_OPS[op], int(bool(inclusive)), _ptr(x), _ptr(y),
                                      x.size, _ptr(total))
        if rc != 0:
            raise ValueError("oracle_scan_u32: unknown operator %r" % op)
        return y, int(total[0])

    def scan_u32_u64(self, x, inclusive: bool = False):
        """Return (y uint64, total) for the widening uint32 -> uint64 sum scan."""
        x = np.ascontiguousarray(x, dtype=np.uint32)
        y = np.empty(x.size, dtype=np.uint64)
        total = np.zeros(1, dtype=np.uint64)
        self.lib.oracle_scan_u32_u64(int(bool(inclusive)), _ptr(x), _ptr(y), x.size, _ptr(total))
        return y, int(total[0])

    def scan_linrec_f32(self, ab, inclusive: bool = True, want_abs: bool = True):
        """Scan of (a, b) pairs under (a1,b1) then (a2,b2) = (a1 a2, a2 b1 + b2).
        ab: (n, 2) float32.  Returns (A, B, SA, SB, (ta, tb)) in fp64; SA/SB are
        the same scan over (|a|, |b|) (None unless want_abs)."""
        ab = np.ascontiguousarray(ab, dtype=np.float32).reshape(-1, 2)
        n = ab.shape[0]
        A = np.empty(n, np.float64)
        B = np.empty(n, np.float64)
        sa = np.empty(n, np.float64) if want_abs else None
        sb = np.empty(n, np.float64) if want_abs else None
        ta = np.zeros(1, np.float64)
        tb = np.zeros(1, np.float64)
        self.lib.oracle_scan_linrec_f32(int(bool(inclusive)), _ptr(ab), _ptr(A), _ptr(B), _ptr(sa), _ptr(sb), n,
                                        _ptr(ta), _ptr(tb))
        return A, B, sa, sb, (float(ta[0]), float(tb[0]))

    def scan_f32_sum(self, x, inclusive: bool = False, want_abs: bool = True):
        """Return (y_fp64, absprefix_fp64 or None, total_fp64) for an fp32 sum scan."""
        x = np.ascontiguousarray(x, dtype=np.float32)
        y = np.empty(x.size, dtype=np.float64)
        ab = np.empty(x.size, dtype=np.float64) if want_abs else None
        total = np.zeros(1, dtype=np.float64)
        self.lib.oracle_scan_f32_sum(int(bool(inclusive)), _ptr(x), _ptr(y), _ptr(ab),
                                     x.size, _ptr(total))
        return y, ab, float(total[0])

    def scan_f32_minmax(self, x, op: str = "max", inclusive: bool = True):
        """Return (y_fp32, total_fp32) for an fp32 max or min scan."""
        x = np.ascontiguousarray(x, dtype=np.float32)
        y = np.empty_like(x)
        total = np.zeros(1, dtype=np.float32)
        rc = self.lib.oracle_scan_f32_minmax(_OPS[op], int(bool(inclusive)), _ptr(x),
                                             _ptr(y), x.size, _ptr(total))
        if rc != 0:
            raise ValueError("oracle_scan_f32_minmax: operator must be max or min")
        return y, float(total[0])

    # -- segmented ------------------------------------------------------------
    def validate_offsets(self, offsets, n: int) -> int:
        offsets = np.ascontiguousarray(offsets, dtype=np.uint32)
        if offsets.size < 1:
            raise ValueError("offsets needs num_segments + 1 >= 1 entries")
        return int(self.lib.oracle_validate_offsets(_ptr(offsets), offsets.size - 1, n))

    def segmented_scan_u32(self, x, offsets, inclusive: bool = False, out=None,
                           sentinel: int = 0):
        """Segmented uint32 sum scan.  Rows outside every segment keep the
        contents of ``out`` (filled with ``sentinel`` when ``out`` is None)."""
        x = np.ascontiguousarray(x, dtype=np.uint32)
        offsets = np.ascontiguousarray(offsets, dtype=np.uint32)
        if out is None:
            out = np.full(x.size, sentinel, dtype=np.uint32)
        rc = self.lib.oracle_segmented_scan_u32(int(bool(inclusive)), _ptr(x), x.size,
                                                _ptr(offsets), offsets.size - 1, _ptr(out))
        if rc != 0:
            raise ValueError("offsets break the contract at index %d" % (rc - 1))
        return out

    # -- compaction -----------------------------------------------------------
    def compact(self, records, flags, out=None):
        """Stable compaction.  ``records`` is an (n, k) or (n,) array whose rows
        are the records; returns (out, count).  Rows of ``out`` past ``count``
        are untouched."""
        records = np.ascontiguousarray(records)
        flags = np.ascontiguousarray(flags, dtype=np.uint8)
        n = flags.size
        if records.shape[0] != n:
            raise ValueError("one flag per record")
        rb = records.nbytes // n if n else records.itemsize * int(np.prod(records.shape[1:]))
        if out is None:
            out = np.zeros_like(records)
        count = self.lib.oracle_compact(_ptr(records), rb, _ptr(flags), n, _ptr(out))
        return out, int(count)


_default = None


def default() -> Oracle:
    """The oracle built from oracle/oracle.c (compiled on first use)."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default
