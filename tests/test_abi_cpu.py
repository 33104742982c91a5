"""The C-ABI library on the CPU: it loads, exports every symbol the header
declares (and the binding wraps each), answers size queries and rejects bad
arguments before anything is launched.  No compute call is made here."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dwps.h")


def _lib():
    import device_wide_prefix_chained_amd as d
    if not os.path.exists(os.path.join(ROOT, "device_wide_prefix_chained_amd", "libdwps.so")):
        from device_wide_prefix_chained_amd import build
        build.build()
    return d.lib()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ps_[a-z0-9_]+)\s*\(", text)))


def test_header_lists_the_boundary():
    names = header_functions()
    for required in ("ps_scan_exclusive_u32", "ps_scan_inclusive_u32", "ps_scan_exclusive_f32",
                     "ps_scan_inclusive_f32", "ps_scan", "ps_segmented_scan_u32", "ps_compact"):
        assert required in names


def test_library_exports_every_declared_symbol():
    lib = _lib()
    so = lib._name
    out = subprocess.run(["nm", "-D", "--defined-only", so], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (ps_\w+)", out))
    for name in header_functions():
        assert name in exported, name
        assert hasattr(lib, name), name


def test_binding_wraps_every_declared_symbol():
    import device_wide_prefix_chained_amd as d
    for name in header_functions():
        assert callable(getattr(d, name, None)), name


def _wsq(lib, fn, *args):
    need = ctypes.c_size_t(0)
    st = getattr(lib, fn)(None, ctypes.byref(need), *args)
    return st, need.value


SMALL_N_CAP = 1 << 24   # inputs up to this size get a workspace that fits both forms


def _two_level_need(n, elem_bytes):
    """The header, then one tile total per 4096-element tile, stored as one
    8-byte descriptor word per 4 bytes of total (a word that reads as an
    unpublished descriptor)."""
    return 256 + -(-(-(-n // 4096)) * 2 * elem_bytes // 256) * 256


def _auto_need(n, single, elem_bytes):
    return max(single, _two_level_need(n, elem_bytes)) if n <= SMALL_N_CAP else single


def test_size_queries():
    lib = _lib()
    tile = lib.ps_tile_elements(0)
    assert tile == 12288
    for n in (0, 1, tile - 1, tile, tile + 1, 1 << 20, SMALL_N_CAP, SMALL_N_CAP + 1, (1 << 28) - 12345, 1 << 28):
        st, need = _wsq(lib, "ps_scan_exclusive_u32", None, None, n, None, None)
        tiles = -(-n // tile)
        single = 256 + -(-tiles * 8 // 256) * 256
        assert st == 0 and need == _auto_need(n, single, 4), n
        st2, need2 = _wsq(lib, "ps_scan", 3, 0, 1, None, None, n, None, None)
        assert st2 == 0 and need2 == need
        st3, need3 = _wsq(lib, "ps_scan_single_pass", 3, 0, 1, None, None, n, None, None)
        assert st3 == 0 and need3 == single
        assert lib.ps_lookback_tiles(n) == tiles
    wtile = lib.ps_tile_elements(2)
    assert wtile == 6144
    for n in (0, 1, wtile, wtile + 1, SMALL_N_CAP, 1 << 28):
        st, need = _wsq(lib, "ps_scan_exclusive_u32_u64", None, None, n, None, None)
        tiles = -(-n // wtile)
        # two descriptor words per tile for the 64-bit payload
        single = 256 + -(-tiles * 16 // 256) * 256
        assert st == 0 and need == _auto_need(n, single, 8), n
        st2, need2 = _wsq(lib, "ps_scan", 0, 2, 0, None, None, n, None, None)
        assert st2 == 0 and need2 == need
    ttile = lib.ps_two_level_tile_elements()
    assert ttile == 4096
    for n in (0, 1, ttile, ttile + 1, 1 << 28):
        tiles = -(-n // ttile)
        for dt, size in ((0, 4), (1, 4), (2, 8)):
            st, need = _wsq(lib, "ps_scan_two_level", 0, dt, 0, None, None, n, None, None)
            # the header, then one tile total per tile in descriptor words
            assert st == 0 and need == 256 + -(-tiles * 2 * size // 256) * 256, (n, dt)
    ltile = lib.ps_linrec_tile_elements()
    assert ltile == 6144
    for n in (0, 1, ltile, ltile + 1, SMALL_N_CAP + 1, 1 << 27):
        st, need = _wsq(lib, "ps_scan_linrec_f32", None, None, None, None, n, 1, None, None)
        tiles = -(-n // ltile)
        # two descriptor words per tile for the (a, b) payload
        assert st == 0 and need == _auto_need(n, 256 + -(-tiles * 16 // 256) * 256, 8), n
    stile = lib.ps_segmented_tile_elements()
    assert stile == 12288
    for n in (0, 1, stile, stile + 1, 1 << 26, (1 << 32) - 1):
        st, need = _wsq(lib, "ps_segmented_scan_u32", None, n, None, 1 << 16, None, 0, None)
        tiles = -(-n // stile)
        # header and one descriptor per tile (the start bitmaps stay in LDS)
        assert st == 0 and need == 256 + -(-tiles * 8 // 256) * 256, n
    for rb in (4, 8, 16):
        ctile = lib.ps_compact_tile_records(rb)
        assert ctile == 8 * 6 * 64 * (16 // rb)
        for n in (0, 1, ctile, ctile + 1, 1 << 26):
            st, need = _wsq(lib, "ps_compact", None, rb, None, n, None, None, None)
            tiles = -(-n // ctile)
            assert st == 0 and need == 256 + -(-tiles * 8 // 256) * 256, (rb, n)
    assert lib.ps_compact_tile_records(12) == 0
    for n in (0, 1, 1000, 1 << 26):
        # the flag scan's own workspace, the n offsets, the count
        st, scan = _wsq(lib, "ps_scan_exclusive_u32", None, None, n, None, None)
        st2, need = _wsq(lib, "ps_compact_staged", None, 16, None, n, None, None, None)
        assert st == st2 == 0 and need == scan + -(-n * 4 // 256) * 256 + 256, n


FAKE_WS = 0x10000000
A = 0x20000000          # fake, 256-byte aligned "device" addresses: never dereferenced
B = 0x40000000
C3 = 0x60000000


def _call_flat(lib, fn, ws_bytes, inp, out, n, total=None):
    wsb = ctypes.c_size_t(ws_bytes)
    return getattr(lib, fn)(ctypes.c_void_p(FAKE_WS), ctypes.byref(wsb), ctypes.c_void_p(inp) if inp else None,
                            ctypes.c_void_p(out) if out else None, n,
                            ctypes.c_void_p(total) if total else None, None)


def test_argument_errors_flat():
    lib = _lib()
    PS_ERR_NULL, PS_ERR_ALIAS, PS_ERR_SIZE, PS_ERR_WORKSPACE, PS_ERR_UNSUPPORTED, PS_ERR_ALIGNMENT = 1, 2, 3, 4, 5, 7
    big = 1 << 30
    for fn in ("ps_scan_exclusive_u32", "ps_scan_inclusive_u32", "ps_scan_exclusive_f32", "ps_scan_inclusive_f32"):
        assert _call_flat(lib, fn, big, A, B, 1 << 32) == PS_ERR_SIZE
        assert _call_flat(lib, fn, 16, A, B, 100000) == PS_ERR_WORKSPACE
        assert _call_flat(lib, fn, big, None, B, 10) == PS_ERR_NULL
        assert _call_flat(lib, fn, big, A, None, 10) == PS_ERR_NULL
        assert _call_flat(lib, fn, big, A + 2, B, 10) == PS_ERR_ALIGNMENT
        assert _call_flat(lib, fn, big, A, B + 1, 10) == PS_ERR_ALIGNMENT
        assert _call_flat(lib, fn, big, A, A + 4, 10) == PS_ERR_ALIAS       # partial overlap
        assert _call_flat(lib, fn, big, A + 36, A, 10) == PS_ERR_ALIAS
        # n == 0 without a total launches nothing and succeeds
        assert _call_flat(lib, fn, big, None, None, 0) == 0
    # ws_bytes == NULL
    assert lib.ps_scan_exclusive_u32(None, None, None, None, 5, None, None) == PS_ERR_NULL
    # unsupported operator / dtype pairs
    wsb = ctypes.c_size_t(big)
    for fn in (lib.ps_scan, lib.ps_scan_two_level):
        for op, dt in ((3, 1), (4, 1), (5, 1), (6, 1), (7, 0), (99, 0), (0, 3), (1, 2), (6, 2)):
            st = fn(ctypes.c_void_p(FAKE_WS), ctypes.byref(wsb), op, dt, 0, ctypes.c_void_p(A),
                    ctypes.c_void_p(B), 10, None, None)
            assert st == PS_ERR_UNSUPPORTED, (op, dt)
    # the two-level form checks its arguments like the single-pass one
    tl = lib.ps_scan_two_level
    for args, code in (((A, B, 1 << 32), PS_ERR_SIZE), ((None, B, 10), PS_ERR_NULL), ((A + 2, B, 10), PS_ERR_ALIGNMENT),
                       ((A, A + 4, 10), PS_ERR_ALIAS)):
        a, b, n = args
        st = tl(ctypes.c_void_p(FAKE_WS), ctypes.byref(wsb), 0, 0, 0, ctypes.c_void_p(a) if a else None,
                ctypes.c_void_p(b), n, None, None)
        assert st == code, args
    small = ctypes.c_size_t(16)
    assert tl(ctypes.c_void_p(FAKE_WS), ctypes.byref(small), 0, 0, 0, ctypes.c_void_p(A), ctypes.c_void_p(B),
              100000, None, None) == PS_ERR_WORKSPACE


def test_argument_errors_widening():
    lib = _lib()
    PS_ERR_ALIAS, PS_ERR_ALIGNMENT, PS_ERR_SIZE = 2, 7, 3
    big = 1 << 30
    for fn in ("ps_scan_exclusive_u32_u64", "ps_scan_inclusive_u32_u64"):
        assert _call_flat(lib, fn, big, A, B, 1 << 32) == PS_ERR_SIZE
        assert _call_flat(lib, fn, big, A, A, 10) == PS_ERR_ALIAS        # no in-place: sizes differ
        assert _call_flat(lib, fn, big, A, A + 32, 10) == PS_ERR_ALIAS   # out overlaps in's tail
        assert _call_flat(lib, fn, big, A + 48, A, 10) == PS_ERR_ALIAS   # in inside out
        assert _call_flat(lib, fn, big, A, B + 4, 10) == PS_ERR_ALIGNMENT  # out not 8-byte aligned
        assert _call_flat(lib, fn, big, A, B, 10, total=B + 4096 + 4) == PS_ERR_ALIGNMENT


def test_argument_errors_linrec():
    lib = _lib()
    PS_ERR_NULL, PS_ERR_ALIAS, PS_ERR_SIZE, PS_ERR_WORKSPACE, PS_ERR_ALIGNMENT = 1, 2, 3, 4, 7
    C, D = 0x60000000, 0x80000000
    big = 1 << 30

    def call(a, b, out_a, out_b, n, total=None, ws_bytes=big):
        wsb = ctypes.c_size_t(ws_bytes)
        v = lambda p: ctypes.c_void_p(p) if p else None  # noqa: E731
        return lib.ps_scan_linrec_f32(ctypes.c_void_p(FAKE_WS), ctypes.byref(wsb), v(a), v(b), v(out_a), v(out_b),
                                      n, 1, v(total), None)

    assert call(A, B, C, D, 1 << 32) == PS_ERR_SIZE
    assert call(A, B, C, D, 100000, ws_bytes=16) == PS_ERR_WORKSPACE
    assert call(None, B, C, D, 10) == PS_ERR_NULL
    assert call(A, None, C, D, 10) == PS_ERR_NULL
    assert call(A, B, C, None, 10) == PS_ERR_NULL          # out_b is required, out_a is not
    assert call(A + 2, B, C, D, 10) == PS_ERR_ALIGNMENT
    assert call(A, B, C + 1, D, 10) == PS_ERR_ALIGNMENT
    assert call(A, B, C, D, 10, total=D + 4096 + 2) == PS_ERR_ALIGNMENT
    assert call(A, B, C, A, 10) == PS_ERR_ALIAS            # B plane written over a
    assert call(A, B, B, D, 10) == PS_ERR_ALIAS            # A plane written over b
    assert call(A, B, None, B + 4, 10) == PS_ERR_ALIAS     # partial overlap with b
    assert call(A, B, C, C + 36, 10) == PS_ERR_ALIAS       # the two outputs overlap
    assert call(A, B, C, C, 10) == PS_ERR_ALIAS
    assert call(None, None, None, None, 0) == 0             # n == 0 without a total: nothing to do


def test_argument_errors_segmented_and_compact():
    lib = _lib()
    big = ctypes.c_size_t(1 << 30)
    ws = ctypes.c_void_p(FAKE_WS)
    seg = lib.ps_segmented_scan_u32
    C0 = 0x70000000
    # out overlapping values or offsets
    assert seg(ws, ctypes.byref(big), ctypes.c_void_p(A), 100, ctypes.c_void_p(B), 4, ctypes.c_void_p(A), 0, None) == 2
    assert seg(ws, ctypes.byref(big), ctypes.c_void_p(A), 100, ctypes.c_void_p(B), 4, ctypes.c_void_p(B - 16), 0, None) == 2
    assert seg(ws, ctypes.byref(big), None, 100, ctypes.c_void_p(B), 4, ctypes.c_void_p(A), 0, None) == 1
    assert seg(ws, ctypes.byref(big), ctypes.c_void_p(A), 1 << 32, ctypes.c_void_p(B), 4, ctypes.c_void_p(A), 0, None) == 3
    assert seg(ws, ctypes.byref(big), ctypes.c_void_p(A), 100, ctypes.c_void_p(B), 0xFFFFFFFF, ctypes.c_void_p(C0),
               0, None) == 3
    assert seg(ws, ctypes.byref(ctypes.c_size_t(8)), ctypes.c_void_p(A), 100000, ctypes.c_void_p(B), 4,
               ctypes.c_void_p(A + (1 << 20)), 0, None) == 4
    # zero segments or n == 0: nothing to do
    assert seg(ws, ctypes.byref(big), ctypes.c_void_p(A), 100, ctypes.c_void_p(B), 0, ctypes.c_void_p(B + 4096), 0, None) == 0
    C = 0x60000000
    for comp in (lib.ps_compact, lib.ps_compact_staged):
        _compact_errors(comp, ws, big, C)


def _compact_errors(comp, ws, big, C):
    for rb in (1, 2, 3, 12, 32):
        assert comp(ws, ctypes.byref(big), ctypes.c_void_p(A), rb, ctypes.c_void_p(B), 10, ctypes.c_void_p(C),
                    ctypes.c_void_p(C + 4096), None) == 5
    assert comp(ws, ctypes.byref(big), ctypes.c_void_p(A), 16, ctypes.c_void_p(B), 10, ctypes.c_void_p(A + 32),
                ctypes.c_void_p(C), None) == 2
    assert comp(ws, ctypes.byref(big), ctypes.c_void_p(A), 16, ctypes.c_void_p(B), 10, ctypes.c_void_p(C),
                None, None) == 1
    assert comp(ws, ctypes.byref(big), ctypes.c_void_p(A + 8), 16, ctypes.c_void_p(B), 10, ctypes.c_void_p(C),
                ctypes.c_void_p(C + 4096), None) == 7


def test_argument_errors_stream_helpers():
    lib = _lib()
    v = ctypes.c_void_p
    assert lib.ps_read_u32(None, 0, None, None) == 0 and lib.ps_fill_u32(None, 0, 0, None) == 0
    assert lib.ps_read_u32(None, 16, v(B), None) == 1 and lib.ps_read_u32(v(A), 16, None, None) == 1
    assert lib.ps_read_u32(v(A + 4), 16, v(B), None) == 7       # 16-byte alignment
    assert lib.ps_read_u32(v(A), 18, v(B), None) == 7           # whole 16-byte vectors only
    assert lib.ps_fill_u32(None, 16, 0, None) == 1
    assert lib.ps_fill_u32(v(A + 2), 16, 0, None) == 7
    assert lib.ps_fill_u32(v(A), 1 << 32, 0, None) == 3
    P = lib.ps_stream_planes_f32
    assert P(None, None, None, None, 0, None) == 0
    assert P(None, v(B), None, v(C3), 16, None) == 1 and P(v(A), v(B), None, None, 16, None) == 1
    assert P(v(A + 4), v(B), None, v(C3), 16, None) == 7       # 16-byte alignment
    assert P(v(A), v(B), None, v(C3), 18, None) == 7           # whole 16-byte vectors only
    assert P(v(A), v(B), None, v(A), 16, None) == 2           # an output over an input
    assert P(v(A), v(B), v(C3), v(C3), 16, None) == 2           # both outputs in one place
    assert P(v(A), v(B), None, v(C3), 1 << 32, None) == 3
    M = lib.ps_stream_mix_u32
    assert M(None, 0, None, 0, None) == 0
    assert M(None, 16, v(B), 16, None) == 1 and M(v(A), 16, None, 16, None) == 1
    assert M(v(A + 4), 16, v(B), 16, None) == 7 and M(v(A), 16, v(B), 6, None) == 7
    assert M(v(A), 16, v(A + 32), 16, None) == 2                     # overlapping
    assert M(v(A), 1 << 32, v(B), 16, None) == 3
    E = lib.ps_stream_mix_even_u32
    assert E(None, 0, None, 0, None) == 0
    assert E(v(A), 16, v(B), 32, None) == 5                          # more written than read
    assert E(None, 16, v(B), 16, None) == 1 and E(v(A), 16, None, 16, None) == 1
    assert E(v(A + 4), 16, v(B), 16, None) == 7 and E(v(A), 16, v(B), 6, None) == 7
    assert E(v(A), 32, v(A + 32), 16, None) == 2                     # overlapping
    assert E(v(A), 1 << 32, v(B), 16, None) == 3
    S = lib.ps_stream_shape
    W, CP, RD = 0, 1, 2
    assert S(CP, 128, 8, 1, 0, None, None, 0, 0, None) == 0          # n = 0: nothing to do
    for t, k in ((32, 8), (512, 8), (128, 2), (128, 32), (96, 4)):
        assert S(W, t, k, 1, 0, None, v(B), 16, 0, None) == 5       # shape not provided
    assert S(3, 128, 8, 1, 0, v(A), v(B), 16, 0, None) == 5          # no such stream
    assert S(CP, 128, 8, 1, 0, None, v(B), 16, 0, None) == 1         # a copy needs its input
    assert S(RD, 128, 8, 1, 0, None, v(B), 16, 0, None) == 1         # a read its input
    assert S(RD, 128, 8, 1, 0, v(A), None, 16, 0, None) == 1         # and its sink
    assert S(W, 128, 8, 1, 0, None, None, 16, 0, None) == 1
    assert S(CP, 256, 16, 0, 1, v(A + 4), v(B), 16, 0, None) == 7    # 16-byte alignment
    assert S(RD, 256, 16, 0, 1, v(A + 4), v(B), 16, 0, None) == 7
    assert S(W, 64, 4, 0, 0, None, v(B), 18, 0, None) == 7          # whole 16-byte vectors only
    assert S(CP, 64, 4, 1, 1, v(A), v(A + 16), 16, 0, None) == 2     # overlapping copy
    assert S(W, 64, 4, 1, 1, None, v(B), 1 << 32, 0, None) == 3


def test_status_strings():
    lib = _lib()
    for code in range(8):
        s = lib.ps_status_string(code).decode()
        assert s and s != "unknown status"
    assert lib.ps_status_string(1234).decode() == "unknown status"
    assert b"gfx950" in lib.ps_version()


def test_binding_refuses_cpu_tensors():
    import torch
    import device_wide_prefix_chained_amd as d
    x = torch.zeros(8, dtype=torch.uint32)
    with pytest.raises(ValueError):
        d.ps_scan_exclusive_u32(x, x.clone())


def test_small_n_config_roundtrip():
    """Host-side setting only: no GPU is touched."""
    import device_wide_prefix_chained_amd as d
    old = d.ps_small_n_config_get()
    assert old == 1 << 23
    try:
        d.ps_small_n_config(0)
        assert d.ps_small_n_config_get() == 0
        d.ps_small_n_config(SMALL_N_CAP)
        assert d.ps_small_n_config_get() == SMALL_N_CAP
        with pytest.raises(d.DwpsError):
            d.ps_small_n_config(SMALL_N_CAP + 1)
        assert d.ps_small_n_config_get() == SMALL_N_CAP
    finally:
        d.ps_small_n_config(old)
    # the size query of a flat entry point does not depend on the setting
    lib = _lib()
    sizes = []
    for setting in (0, 1 << 23, SMALL_N_CAP):
        d.ps_small_n_config(setting)
        sizes.append(_wsq(lib, "ps_scan_exclusive_u32", None, None, 5_000_000, None, None)[1])
    d.ps_small_n_config(old)
    assert len(set(sizes)) == 1


def test_lookback_config_roundtrip():
    """Host-side setting only: no GPU is touched."""
    import device_wide_prefix_chained_amd as d
    old = d.ps_lookback_config_get()
    assert old == (4096, 4)
    try:
        d.ps_lookback_config(0, 0)
        assert d.ps_lookback_config_get() == (0, 0)
        d.ps_lookback_config(12345, 3)
        assert d.ps_lookback_config_get() == (12345, 3)
    finally:
        d.ps_lookback_config(*old)
    assert d.ps_lookback_config_get() == old


@pytest.mark.parametrize("lang", ["c99", "c++17"])
def test_header_and_library_from_plain_c(tmp_path, lang):
    """tests/c/abi_from_c.c, built as C99 (and as C++17) with warnings as
    errors against include/dwps.h and linked to libdwps.so, runs its size
    queries and argument-error checks: the boundary needs neither Python nor
    torch."""
    import shutil
    lib = _lib()
    libdir = os.path.dirname(lib._name)
    cc = "gcc" if lang == "c99" else "g++"
    if shutil.which(cc) is None:
        pytest.skip("%s not installed" % cc)
    exe = str(tmp_path / "abi_from_c")
    cmd = [cc, "-std=" + lang, "-Wall", "-Wextra", "-Werror", "-I" + os.path.join(ROOT, "include")]
    if lang == "c99":
        cmd.append("-pedantic")
    else:
        cmd += ["-x", "c++"]
    cmd += [os.path.join(ROOT, "tests", "c", "abi_from_c.c"), "-L" + libdir, "-ldwps",
            "-Wl,-rpath," + libdir, "-Wl,-rpath-link,/opt/rocm/lib", "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    run = subprocess.run([exe], capture_output=True, text=True)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "FAIL" not in run.stdout and run.stdout.count("ok") >= 10


def test_kernel_timing_arguments():
    lib = _lib()
    assert lib.ps_kernel_timing(-1) == 3          # PS_ERR_SIZE
    assert lib.ps_kernel_timing(4) == 0 and lib.ps_kernel_timing(0) == 0
