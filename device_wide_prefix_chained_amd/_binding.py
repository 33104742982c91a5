"""ctypes binding of libdwps.so: argument marshalling only.

Each Python function has the name of the C entry point it wraps (see
``include/dwps.h`` for the contract).  Tensors are PyTorch CUDA (HIP) tensors;
PyTorch supplies device memory and streams.  A call that is given no
workspace uses one kept per (device, stream), allocated on that stream and
prepared once with ``ps_workspace_init``, so it is one kernel launch like
any other and its workspace is never handed to another stream while in use.
Every step of the computation runs in the library's HIP kernels; there is
no fallback: if the library is missing or a call fails, an exception is
raised.
"""
from __future__ import annotations

import ctypes
import os

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(PKG, "libdwps.so")

# enum values of include/dwps.h
PS_OK = 0
PS_U32, PS_F32, PS_U64 = 0, 1, 2
PS_OP_SUM, PS_OP_MAX, PS_OP_MIN, PS_OP_AND, PS_OP_OR, PS_OP_XOR, PS_OP_AFFINE16 = range(7)
OPS = {"sum": PS_OP_SUM, "max": PS_OP_MAX, "min": PS_OP_MIN, "and": PS_OP_AND,
       "or": PS_OP_OR, "xor": PS_OP_XOR, "affine16": PS_OP_AFFINE16}

# workspace header words and error bits (ps_ws_word, ps_ws_error)
PS_WS_HEADER_BYTES = 256
(PS_WS_ERROR, PS_WS_FALLBACKS, PS_WS_PARTIALS, PS_WS_TAG) = range(1, 5)
(PS_WS_MAGIC, PS_WS_CAPACITY, PS_WS_HIGH, PS_WS_DIRTY_LO, PS_WS_DIRTY_HI, PS_WS_READY, PS_WS_CALLS) = range(6, 13)
PS_WS_TICKET, PS_WS_DONE = 32, 33
PS_WS_ERR_SPIN, PS_WS_ERR_NOT_PREPARED, PS_WS_ERR_CAPACITY = 1, 2, 4
PS_DEBUG_WITHHOLD_AGGREGATES = 1
STATS_WORDS = 16  # uint32 per tile of the instrumented entry points

_U32_DTYPES = (torch.uint32, torch.int32)
_U64_DTYPES = (torch.uint64, torch.int64)

_lib = None


class DwpsError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__("%s failed: status %d (%s)" % (fn, status, msg))
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libdwps.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIBRARY):
        raise ImportError("libdwps.so is not built (%s); run "
                          "`python -m device_wide_prefix_chained_amd.build`" % LIBRARY)
    L = ctypes.CDLL(LIBRARY)
    vp, sz, u64, u32, i32 = (ctypes.c_void_p, ctypes.POINTER(ctypes.c_size_t), ctypes.c_uint64,
                             ctypes.c_uint32, ctypes.c_int)
    flat = [vp, sz, vp, vp, u64, vp, vp]
    for name in ("ps_scan_exclusive_u32", "ps_scan_inclusive_u32",
                 "ps_scan_exclusive_f32", "ps_scan_inclusive_f32",
                 "ps_scan_exclusive_u32_u64", "ps_scan_inclusive_u32_u64"):
        getattr(L, name).argtypes = flat
        getattr(L, name).restype = i32
    L.ps_scan_linrec_f32.argtypes = [vp, sz, vp, vp, vp, vp, u64, i32, vp, vp]
    L.ps_scan_linrec_f32.restype = i32
    L.ps_linrec_lookback_stats.argtypes = [vp, sz, vp, vp, vp, vp, u64, i32, vp, vp]
    L.ps_linrec_lookback_stats.restype = i32
    L.ps_linrec_tile_elements.argtypes = []
    L.ps_linrec_tile_elements.restype = u32
    L.ps_scan.argtypes = [vp, sz, i32, i32, i32, vp, vp, u64, vp, vp]
    L.ps_scan.restype = i32
    L.ps_scan_two_level.argtypes = [vp, sz, i32, i32, i32, vp, vp, u64, vp, vp]
    L.ps_scan_two_level.restype = i32
    L.ps_scan_single_pass.argtypes = [vp, sz, i32, i32, i32, vp, vp, u64, vp, vp]
    L.ps_scan_single_pass.restype = i32
    L.ps_small_n_config.argtypes = [u64]
    L.ps_small_n_config.restype = i32
    L.ps_small_n_config_get.argtypes = []
    L.ps_small_n_config_get.restype = u64
    L.ps_two_level_tile_elements.argtypes = []
    L.ps_two_level_tile_elements.restype = u32
    L.ps_segmented_scan_u32.argtypes = [vp, sz, vp, u64, vp, u32, vp, i32, vp]
    L.ps_segmented_scan_u32.restype = i32
    L.ps_validate_offsets.argtypes = [vp, u32, u64, vp, vp]
    L.ps_validate_offsets.restype = i32
    L.ps_compact.argtypes = [vp, sz, vp, u32, vp, u64, vp, vp, vp]
    L.ps_compact.restype = i32
    L.ps_compact_staged.argtypes = [vp, sz, vp, u32, vp, u64, vp, vp, vp]
    L.ps_compact_staged.restype = i32
    L.ps_copy_u32.argtypes = [vp, vp, u64, vp]
    L.ps_copy_u32.restype = i32
    L.ps_read_u32.argtypes = [vp, u64, vp, vp]
    L.ps_read_u32.restype = i32
    L.ps_fill_u32.argtypes = [vp, u64, u32, vp]
    L.ps_fill_u32.restype = i32
    L.ps_stream_planes_f32.argtypes = [vp, vp, vp, vp, u64, vp]
    L.ps_stream_planes_f32.restype = i32
    L.ps_stream_mix_u32.argtypes = [vp, u64, vp, u64, vp]
    L.ps_stream_mix_u32.restype = i32
    L.ps_stream_mix_even_u32.argtypes = [vp, u64, vp, u64, vp]
    L.ps_stream_mix_even_u32.restype = i32
    L.ps_stream_shape.argtypes = [i32, i32, i32, i32, i32, vp, vp, u64, u32, vp]
    L.ps_stream_shape.restype = i32
    L.ps_lookback_stats_u32.argtypes = [vp, sz, vp, vp, u64, vp, i32, vp]
    L.ps_lookback_stats_u32.restype = i32
    L.ps_scan_lookback_stats.argtypes = [vp, sz, i32, i32, i32, vp, vp, u64, vp, vp]
    L.ps_scan_lookback_stats.restype = i32
    L.ps_segmented_lookback_stats_u32.argtypes = [vp, sz, vp, u64, vp, u32, vp, i32, vp, vp]
    L.ps_segmented_lookback_stats_u32.restype = i32
    L.ps_compact_lookback_stats.argtypes = [vp, sz, vp, u32, vp, u64, vp, vp, vp, vp]
    L.ps_compact_lookback_stats.restype = i32
    L.ps_lookback_tiles.argtypes = [u64]
    L.ps_lookback_tiles.restype = u64
    L.ps_kernel_timing.argtypes = [i32]
    L.ps_kernel_timing.restype = i32
    L.ps_kernel_timing_read.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_uint64)]
    L.ps_kernel_timing_read.restype = i32
    L.ps_lookback_window.argtypes = []
    L.ps_lookback_window.restype = u32
    L.ps_lookback_group.argtypes = []
    L.ps_lookback_group.restype = u32
    L.ps_lookback_config.argtypes = [u32, u32]
    L.ps_lookback_config.restype = i32
    L.ps_lookback_config_get.argtypes = [ctypes.POINTER(ctypes.c_uint32), ctypes.POINTER(ctypes.c_uint32)]
    L.ps_lookback_config_get.restype = None
    L.ps_tile_elements.argtypes = [i32]
    L.ps_tile_elements.restype = u32
    L.ps_segmented_tile_elements.argtypes = []
    L.ps_segmented_tile_elements.restype = u32
    L.ps_compact_tile_records.argtypes = [u32]
    L.ps_compact_tile_records.restype = u32
    L.ps_scan_noalloc.argtypes = [i32, i32, i32, vp, vp, u64, vp, vp]
    L.ps_scan_noalloc.restype = i32
    L.ps_scan_noalloc_bytes.argtypes = []
    L.ps_scan_noalloc_bytes.restype = ctypes.c_size_t
    L.ps_workspace_init.argtypes = [vp, ctypes.c_size_t, vp]
    L.ps_workspace_init.restype = i32
    L.ps_lookback_debug.argtypes = [u32]
    L.ps_lookback_debug.restype = i32
    L.ps_lookback_debug_get.argtypes = []
    L.ps_lookback_debug_get.restype = u32
    L.ps_version.argtypes = []
    L.ps_version.restype = ctypes.c_char_p
    L.ps_status_string.argtypes = [i32]
    L.ps_status_string.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(fn: str, status: int) -> None:
    if status != PS_OK:
        raise DwpsError(fn, status, lib().ps_status_string(status).decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _torch_stream(device, stream):
    """The call's stream as a torch stream object (the current stream of
    ``device`` when None; raw hipStream_t handles are wrapped)."""
    if stream is None:
        return torch.cuda.current_stream(device)
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream), device=device)


# The raw handle of a device's current stream, read without building a
# torch stream object (which costs microseconds per call); None on a torch
# without it, where the stream object is built instead.
_CURRENT_RAW_STREAM = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _raw_stream(t, stream) -> int:
    """The call's stream as a raw hipStream_t (the current stream of t's
    device when None)."""
    if stream is None and _CURRENT_RAW_STREAM is not None:
        return int(_CURRENT_RAW_STREAM(t.get_device()))
    return int(_torch_stream(t.device, stream).cuda_stream)


def _stream(t, stream):
    return ctypes.c_void_p(_raw_stream(t, stream))


def _dev_tensor(name, t, dtypes=None, numel=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError("%s has dtype %s, expected one of %s" % (name, t.dtype, dtypes))
    if numel is not None and t.numel() < numel:
        raise ValueError("%s holds %d elements, needs %d" % (name, t.numel(), numel))
    return t


def ps_workspace_init(workspace, stream=None):
    """Prepare a workspace (a uint8 device tensor) for its first use."""
    _dev_tensor("workspace", workspace)
    _check("ps_workspace_init", lib().ps_workspace_init(
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(workspace, stream)))
    return workspace


def new_workspace(nbytes, device="cuda", stream=None):
    """A prepared workspace of at least ``nbytes`` bytes, allocated on the
    stream that will use it (the current stream when None)."""
    device = torch.device(device)
    ts = _torch_stream(device, stream)
    with torch.cuda.stream(ts):
        ws = torch.empty(max(int(nbytes), PS_WS_HEADER_BYTES), dtype=torch.uint8, device=device)
    return ps_workspace_init(ws, stream=ts)


_WS_CACHE = {}


def _cached_workspace(fn, need, t, stream):
    key = (t.get_device(), _raw_stream(t, stream))
    ws = _WS_CACHE.get(key)
    if ws is not None and ws.numel() >= need:
        return ws
    device = t.device
    ts = _torch_stream(device, stream)
    if torch.cuda.is_current_stream_capturing():
        raise RuntimeError("%s: pass a workspace (new_workspace) when capturing a graph" % fn)
    # grow geometrically; the old buffer was only ever used on this stream,
    # so the allocator may hand it out again in this stream's order
    size = max(int(need), 1 << 16)
    if ws is not None:
        size = max(size, 2 * ws.numel())
    ws = new_workspace(size, device, ts)
    _WS_CACHE[key] = ws
    return ws


def _workspace(fn: str, call, t, workspace, stream=None):
    """The call's workspace, or the prepared one kept for the device and
    stream of tensor t when none is given (sized by a CUB-style query).  A
    given workspace is not queried: the library itself refuses one that is
    too small (PS_ERR_WORKSPACE) before anything runs."""
    if workspace is None:
        need = ctypes.c_size_t(0)
        _check(fn, call(None, ctypes.byref(need)))
        workspace = _cached_workspace(fn, int(need.value), t, stream)
    else:
        _dev_tensor("workspace", workspace)
    have = ctypes.c_size_t(workspace.numel() * workspace.element_size())
    return workspace, have


# ---------------------------------------------------------------------------
# flat scans
# ---------------------------------------------------------------------------
def _flat(fn: str, inp, out, total, workspace, stream, dtypes, out_dtypes=None):
    out_dtypes = dtypes if out_dtypes is None else out_dtypes
    _dev_tensor("inp", inp, dtypes)
    _dev_tensor("out", out, out_dtypes, inp.numel())
    if total is not None:
        _dev_tensor("total", total, out_dtypes, 1)
    f = getattr(lib(), fn)
    n = inp.numel()
    s = _stream(inp, stream)
    call = lambda ws, wsb: f(ws, wsb, _ptr(inp), _ptr(out), n, _ptr(total), s)  # noqa: E731
    ws, have = _workspace(fn, call, inp, workspace, stream)
    _check(fn, call(_ptr(ws), ctypes.byref(have)))
    return out


def ps_scan_exclusive_u32(inp, out, total=None, workspace=None, stream=None):
    return _flat("ps_scan_exclusive_u32", inp, out, total, workspace, stream, _U32_DTYPES)


def ps_scan_inclusive_u32(inp, out, total=None, workspace=None, stream=None):
    return _flat("ps_scan_inclusive_u32", inp, out, total, workspace, stream, _U32_DTYPES)


def ps_scan_exclusive_f32(inp, out, total=None, workspace=None, stream=None):
    return _flat("ps_scan_exclusive_f32", inp, out, total, workspace, stream, (torch.float32,))


def ps_scan_inclusive_f32(inp, out, total=None, workspace=None, stream=None):
    return _flat("ps_scan_inclusive_f32", inp, out, total, workspace, stream, (torch.float32,))


def ps_scan_exclusive_u32_u64(inp, out, total=None, workspace=None, stream=None):
    """Widening sum: uint32 (or bit-identical int32) in, uint64/int64 out."""
    return _flat("ps_scan_exclusive_u32_u64", inp, out, total, workspace, stream, _U32_DTYPES, _U64_DTYPES)


def ps_scan_inclusive_u32_u64(inp, out, total=None, workspace=None, stream=None):
    return _flat("ps_scan_inclusive_u32_u64", inp, out, total, workspace, stream, _U32_DTYPES, _U64_DTYPES)


def ps_scan(op, inclusive, inp, out, total=None, workspace=None, stream=None, dtype=None):
    """Generic associative-operator scan; ``op`` is a PS_OP_* code or a name
    ('sum', 'max', 'min', 'and', 'or', 'xor', 'affine16')."""
    return _generic("ps_scan", op, inclusive, inp, out, total, workspace, stream, dtype)


def ps_scan_two_level(op, inclusive, inp, out, total=None, workspace=None, stream=None, dtype=None):
    """The two-level (reduce-then-scan, three launches) form of ps_scan."""
    return _generic("ps_scan_two_level", op, inclusive, inp, out, total, workspace, stream, dtype)


def ps_scan_single_pass(op, inclusive, inp, out, total=None, workspace=None, stream=None, dtype=None):
    """The single-pass chained form of ps_scan at every n."""
    return _generic("ps_scan_single_pass", op, inclusive, inp, out, total, workspace, stream, dtype)


def ps_scan_noalloc(op, inclusive, inp, out, total=None, stream=None, dtype=None):
    """ps_scan on the library's own per-device workspace (no allocation)."""
    opc = OPS[op] if isinstance(op, str) else int(op)
    if dtype is None:
        dtype = PS_F32 if inp.dtype == torch.float32 else PS_U32
    dtypes = (torch.float32,) if dtype == PS_F32 else _U32_DTYPES
    out_dtypes = _U64_DTYPES if dtype == PS_U64 else dtypes
    _dev_tensor("inp", inp, dtypes)
    _dev_tensor("out", out, out_dtypes, inp.numel())
    if total is not None:
        _dev_tensor("total", total, out_dtypes, 1)
    _check("ps_scan_noalloc", lib().ps_scan_noalloc(opc, dtype, int(bool(inclusive)), _ptr(inp), _ptr(out),
                                                    inp.numel(), _ptr(total), _stream(inp, stream)))
    return out


def ps_scan_noalloc_bytes() -> int:
    return int(lib().ps_scan_noalloc_bytes())


def ps_small_n_config(max_elements: int) -> None:
    """Largest n the flat entry points hand to the two-level form (0 = never)."""
    _check("ps_small_n_config", lib().ps_small_n_config(int(max_elements)))


def ps_small_n_config_get() -> int:
    return int(lib().ps_small_n_config_get())


def ps_two_level_tile_elements() -> int:
    return int(lib().ps_two_level_tile_elements())


def _generic(fn, op, inclusive, inp, out, total, workspace, stream, dtype):
    opc = OPS[op] if isinstance(op, str) else int(op)
    if dtype is None:
        dtype = PS_F32 if inp.dtype == torch.float32 else PS_U32
    dtypes = (torch.float32,) if dtype == PS_F32 else _U32_DTYPES
    out_dtypes = _U64_DTYPES if dtype == PS_U64 else dtypes
    _dev_tensor("inp", inp, dtypes)
    _dev_tensor("out", out, out_dtypes, inp.numel())
    if total is not None:
        _dev_tensor("total", total, out_dtypes, 1)
    n = inp.numel()
    s = _stream(inp, stream)
    L = lib()
    f = getattr(L, fn)
    call = lambda ws, wsb: f(ws, wsb, opc, dtype, int(bool(inclusive)), _ptr(inp),  # noqa: E731
                             _ptr(out), n, _ptr(total), s)
    ws, have = _workspace(fn, call, inp, workspace, stream)
    _check(fn, call(_ptr(ws), ctypes.byref(have)))
    return out


def ps_scan_linrec_f32(a, b, out_b, out_a=None, inclusive=True, total=None, workspace=None, stream=None):
    """Linear recurrence h[t] = a[t] h[t-1] + b[t] as a scan of (a, b) pairs:
    out_b receives B (= h for the inclusive form), out_a (optional) the
    products A; total (optional) two floats, the fold (A, B) of all pairs."""
    _dev_tensor("a", a, (torch.float32,))
    n = a.numel()
    _dev_tensor("b", b, (torch.float32,), n)
    _dev_tensor("out_b", out_b, (torch.float32,), n)
    if out_a is not None:
        _dev_tensor("out_a", out_a, (torch.float32,), n)
    if total is not None:
        _dev_tensor("total", total, (torch.float32,), 2)
    s = _stream(a, stream)
    L = lib()
    call = lambda ws, wsb: L.ps_scan_linrec_f32(ws, wsb, _ptr(a), _ptr(b), _ptr(out_a), _ptr(out_b),  # noqa: E731
                                                n, int(bool(inclusive)), _ptr(total), s)
    ws, have = _workspace("ps_scan_linrec_f32", call, a, workspace, stream)
    _check("ps_scan_linrec_f32", call(_ptr(ws), ctypes.byref(have)))
    return out_b


def ps_linrec_tile_elements() -> int:
    return int(lib().ps_linrec_tile_elements())


def ps_linrec_lookback_stats(a, b, out_b, stats, out_a=None, inclusive=True, workspace=None, stream=None):
    """ps_scan_linrec_f32 (single-pass form, no total) with per-tile look-back
    statistics: STATS_WORDS uint32 for each of ceil(n / ps_linrec_tile_elements())
    tiles."""
    _dev_tensor("a", a, (torch.float32,))
    n = a.numel()
    _dev_tensor("b", b, (torch.float32,), n)
    _dev_tensor("out_b", out_b, (torch.float32,), n)
    if out_a is not None:
        _dev_tensor("out_a", out_a, (torch.float32,), n)
    tiles = -(-n // ps_linrec_tile_elements())
    _dev_tensor("stats", stats, _U32_DTYPES, STATS_WORDS * tiles)
    s = _stream(a, stream)
    L = lib()
    call = lambda ws, wsb: L.ps_linrec_lookback_stats(ws, wsb, _ptr(a), _ptr(b), _ptr(out_a),  # noqa: E731
                                                      _ptr(out_b), n, int(bool(inclusive)), _ptr(stats), s)
    ws, have = _workspace("ps_linrec_lookback_stats", call, a, workspace, stream)
    _check("ps_linrec_lookback_stats", call(_ptr(ws), ctypes.byref(have)))
    return stats


def ps_lookback_stats_u32(inp, out, stats, aggregate_only=False, workspace=None, stream=None):
    _dev_tensor("inp", inp, _U32_DTYPES)
    _dev_tensor("out", out, _U32_DTYPES, inp.numel())
    n = inp.numel()
    _dev_tensor("stats", stats, _U32_DTYPES, STATS_WORDS * ps_lookback_tiles(n))
    s = _stream(inp, stream)
    L = lib()
    call = lambda ws, wsb: L.ps_lookback_stats_u32(ws, wsb, _ptr(inp), _ptr(out), n,  # noqa: E731
                                                   _ptr(stats), int(bool(aggregate_only)), s)
    ws, have = _workspace("ps_lookback_stats_u32", call, inp, workspace, stream)
    _check("ps_lookback_stats_u32", call(_ptr(ws), ctypes.byref(have)))
    return stats


def ps_scan_lookback_stats(op, inclusive, inp, out, stats, workspace=None, stream=None, dtype=None):
    """ps_scan (u32 sum, f32 sum, f32 max) with per-tile look-back statistics:
    stats holds STATS_WORDS uint32 per tile (the layout in dwps.h)."""
    opc = OPS[op] if isinstance(op, str) else int(op)
    if dtype is None:
        dtype = PS_F32 if inp.dtype == torch.float32 else PS_U32
    dtypes = (torch.float32,) if dtype == PS_F32 else _U32_DTYPES
    _dev_tensor("inp", inp, dtypes)
    _dev_tensor("out", out, dtypes, inp.numel())
    n = inp.numel()
    _dev_tensor("stats", stats, _U32_DTYPES, STATS_WORDS * ps_lookback_tiles(n))
    s = _stream(inp, stream)
    L = lib()
    call = lambda ws, wsb: L.ps_scan_lookback_stats(ws, wsb, opc, dtype, int(bool(inclusive)),  # noqa: E731
                                                    _ptr(inp), _ptr(out), n, _ptr(stats), s)
    ws, have = _workspace("ps_scan_lookback_stats", call, inp, workspace, stream)
    _check("ps_scan_lookback_stats", call(_ptr(ws), ctypes.byref(have)))
    return stats


def ps_segmented_lookback_stats_u32(values, offsets, out, stats, inclusive=False, workspace=None, stream=None):
    """ps_segmented_scan_u32 with per-tile look-back statistics."""
    _dev_tensor("values", values, _U32_DTYPES)
    _dev_tensor("offsets", offsets, _U32_DTYPES)
    _dev_tensor("out", out, _U32_DTYPES, values.numel())
    n = values.numel()
    tiles = -(-n // ps_segmented_tile_elements())
    _dev_tensor("stats", stats, _U32_DTYPES, STATS_WORDS * tiles)
    nseg = offsets.numel() - 1
    s = _stream(values, stream)
    L = lib()
    call = lambda ws, wsb: L.ps_segmented_lookback_stats_u32(ws, wsb, _ptr(values), n, _ptr(offsets),  # noqa
                                                             nseg, _ptr(out), int(bool(inclusive)), _ptr(stats), s)
    ws, have = _workspace("ps_segmented_lookback_stats_u32", call, values, workspace, stream)
    _check("ps_segmented_lookback_stats_u32", call(_ptr(ws), ctypes.byref(have)))
    return stats


def ps_compact_lookback_stats(records, flags, out, num_selected, stats, workspace=None, stream=None):
    """ps_compact of 16-byte records with per-tile look-back statistics."""
    _dev_tensor("records", records)
    _dev_tensor("flags", flags, (torch.uint8, torch.bool))
    _dev_tensor("out", out)
    _dev_tensor("num_selected", num_selected, (torch.int64, torch.uint64), 1)
    n = flags.numel()
    tiles = -(-n // ps_compact_tile_records(16))
    _dev_tensor("stats", stats, _U32_DTYPES, STATS_WORDS * tiles)
    row = 1
    for d in records.shape[1:]:
        row *= int(d)
    rb = records.element_size() * row
    s = _stream(flags, stream)
    L = lib()
    call = lambda ws, wsb: L.ps_compact_lookback_stats(ws, wsb, _ptr(records), rb, _ptr(flags), n,  # noqa
                                                       _ptr(out), _ptr(num_selected), _ptr(stats), s)
    ws, have = _workspace("ps_compact_lookback_stats", call, flags, workspace, stream)
    _check("ps_compact_lookback_stats", call(_ptr(ws), ctypes.byref(have)))
    return stats


def ps_lookback_tiles(n: int) -> int:
    return int(lib().ps_lookback_tiles(n))


# ---------------------------------------------------------------------------
# segmented scan
# ---------------------------------------------------------------------------
def ps_segmented_scan_u32(values, offsets, out, inclusive=False, workspace=None, stream=None):
    _dev_tensor("values", values, _U32_DTYPES)
    _dev_tensor("offsets", offsets, _U32_DTYPES)
    _dev_tensor("out", out, _U32_DTYPES, values.numel())
    if offsets.numel() < 1:
        raise ValueError("offsets needs num_segments + 1 >= 1 entries")
    n = values.numel()
    nseg = offsets.numel() - 1
    s = _stream(values, stream)
    L = lib()
    call = lambda ws, wsb: L.ps_segmented_scan_u32(ws, wsb, _ptr(values), n, _ptr(offsets),  # noqa: E731
                                                   nseg, _ptr(out), int(bool(inclusive)), s)
    ws, have = _workspace("ps_segmented_scan_u32", call, values, workspace, stream)
    _check("ps_segmented_scan_u32", call(_ptr(ws), ctypes.byref(have)))
    return out


def ps_validate_offsets(offsets, n, result, stream=None):
    _dev_tensor("offsets", offsets, _U32_DTYPES)
    _dev_tensor("result", result, (torch.int64,), 1)
    _check("ps_validate_offsets", lib().ps_validate_offsets(
        _ptr(offsets), offsets.numel() - 1, int(n), _ptr(result), _stream(offsets, stream)))
    return result


# ---------------------------------------------------------------------------
# compaction
# ---------------------------------------------------------------------------
def ps_compact(records, flags, out, num_selected, workspace=None, stream=None):
    """records: (n,) or (n, k) tensor whose rows are the records (4, 8 or 16
    bytes); flags: (n,) uint8/bool; out: same shape as records;
    num_selected: one int64/uint64 element on the device."""
    return _compact("ps_compact", records, flags, out, num_selected, workspace, stream)


def ps_compact_staged(records, flags, out, num_selected, workspace=None, stream=None):
    """ps_compact computed as a flag scan followed by a scatter (two passes)."""
    return _compact("ps_compact_staged", records, flags, out, num_selected, workspace, stream)


def _compact(fn, records, flags, out, num_selected, workspace, stream):
    _dev_tensor("records", records)
    _dev_tensor("flags", flags, (torch.uint8, torch.bool))
    _dev_tensor("out", out)
    _dev_tensor("num_selected", num_selected, (torch.int64, torch.uint64), 1)
    n = flags.numel()
    if records.shape[0] != n or (records.dim() > 1 and out.shape[1:] != records.shape[1:]):
        raise ValueError("records must have one row per flag and out the same row shape")
    if out.shape[0] < n:
        raise ValueError("out needs room for n records")
    row = 1
    for d in records.shape[1:]:
        row *= int(d)
    rb = records.element_size() * row
    s = _stream(flags, stream)
    L = lib()
    f = getattr(L, fn)
    call = lambda ws, wsb: f(ws, wsb, _ptr(records), rb, _ptr(flags), n,  # noqa: E731
                             _ptr(out), _ptr(num_selected), s)
    ws, have = _workspace(fn, call, flags, workspace, stream)
    _check(fn, call(_ptr(ws), ctypes.byref(have)))
    return out


# ---------------------------------------------------------------------------
# measurement helpers
# ---------------------------------------------------------------------------
def ps_copy_u32(inp, out, stream=None):
    _dev_tensor("inp", inp, _U32_DTYPES)
    _dev_tensor("out", out, _U32_DTYPES, inp.numel())
    _check("ps_copy_u32", lib().ps_copy_u32(_ptr(inp), _ptr(out), inp.numel(), _stream(inp, stream)))
    return out


def ps_read_u32(inp, sink, stream=None):
    _dev_tensor("inp", inp, _U32_DTYPES)
    _dev_tensor("sink", sink, _U32_DTYPES, 1)
    _check("ps_read_u32", lib().ps_read_u32(_ptr(inp), inp.numel(), _ptr(sink), _stream(inp, stream)))


def ps_fill_u32(out, value, stream=None):
    _dev_tensor("out", out, _U32_DTYPES)
    _check("ps_fill_u32", lib().ps_fill_u32(_ptr(out), out.numel(), int(value) & 0xFFFFFFFF, _stream(out, stream)))
    return out


def ps_stream_planes_f32(a, b, out_b, out_a=None, stream=None):
    """The recurrence's access shape as a plain stream: out_b = a * b and,
    when given, out_a = a + b (float planes, 16-byte aligned, n % 4 == 0)."""
    _dev_tensor("a", a, (torch.float32,))
    n = a.numel()
    _dev_tensor("b", b, (torch.float32,), n)
    _dev_tensor("out_b", out_b, (torch.float32,), n)
    if out_a is not None:
        _dev_tensor("out_a", out_a, (torch.float32,), n)
    _check("ps_stream_planes_f32", lib().ps_stream_planes_f32(_ptr(a), _ptr(b), _ptr(out_a), _ptr(out_b), n,
                                                              _stream(a, stream)))
    return out_b


def ps_stream_mix_u32(inp, out, stream=None):
    """A plain stream that reads inp and writes out: the words both have
    copied, then the rest of the longer one read or written alone (the
    ceiling of a kernel with that byte mix)."""
    _dev_tensor("inp", inp, _U32_DTYPES)
    _dev_tensor("out", out, _U32_DTYPES)
    _check("ps_stream_mix_u32", lib().ps_stream_mix_u32(_ptr(inp), inp.numel(), _ptr(out), out.numel(),
                                                        _stream(out, stream)))
    return out


def ps_stream_mix_even_u32(inp, out, stream=None):
    """The same byte mix spread evenly over the workgroups (read-heavy mixes:
    out no longer than inp): each workgroup reads a block of inp and writes
    its proportional share of out."""
    _dev_tensor("inp", inp, _U32_DTYPES)
    _dev_tensor("out", out, _U32_DTYPES)
    _check("ps_stream_mix_even_u32", lib().ps_stream_mix_even_u32(_ptr(inp), inp.numel(), _ptr(out), out.numel(),
                                                                  _stream(out, stream)))
    return out


def ps_stream_shape(kind, out, inp=None, *, threads=128, vecs=8, nontemporal=True, persistent=False, value=0,
                    stream=None):
    """One plain stream in a given access shape (the sweep behind the stream
    ceilings): kind "write" fills out with ``value``, "copy" copies inp to
    out, "read" reads inp (out: a one-word sink)."""
    code = {"write": 0, "copy": 1, "read": 2}[kind]
    if kind == "read":
        _dev_tensor("inp", inp, _U32_DTYPES)
        _dev_tensor("sink", out, _U32_DTYPES, 1)
        n = inp.numel()
    else:
        _dev_tensor("out", out, _U32_DTYPES)
        n = out.numel()
        if kind == "copy":
            _dev_tensor("inp", inp, _U32_DTYPES, n)
        else:
            inp = None
    _check("ps_stream_shape", lib().ps_stream_shape(code, int(threads), int(vecs), int(bool(nontemporal)),
                                                    int(bool(persistent)), _ptr(inp), _ptr(out), n,
                                                    int(value) & 0xFFFFFFFF, _stream(out, stream)))
    return out


def ps_kernel_timing(enable: bool, every: int = 1) -> None:
    """Start (enable) or stop kernel timing; ``every`` = N times every Nth call."""
    _check("ps_kernel_timing", lib().ps_kernel_timing(int(every) if enable else 0))


def ps_kernel_timing_read():
    """Return (total milliseconds, number of timed launches)."""
    ms = ctypes.c_double(0.0)
    cnt = ctypes.c_uint64(0)
    _check("ps_kernel_timing_read", lib().ps_kernel_timing_read(ctypes.byref(ms), ctypes.byref(cnt)))
    return ms.value, cnt.value


def ps_lookback_window() -> int:
    return int(lib().ps_lookback_window())


def ps_lookback_group() -> int:
    return int(lib().ps_lookback_group())


def ps_lookback_config(fallback_polls: int, partial_windows: int) -> None:
    """Look-back settings of every later call: fallback after this many
    stalled polls (0 = never); PARTIAL descriptors after this many windows
    walked without an inclusive prefix (0 = never)."""
    _check("ps_lookback_config", lib().ps_lookback_config(int(fallback_polls), int(partial_windows)))


def ps_lookback_debug(flags: int) -> None:
    """Debug settings of every later single-pass call (PS_DEBUG_* bits; 0 = off)."""
    _check("ps_lookback_debug", lib().ps_lookback_debug(int(flags)))


def ps_lookback_debug_get() -> int:
    return int(lib().ps_lookback_debug_get())


def workspace_header(workspace):
    """The header words of a workspace as Python ints (synchronises)."""
    import numpy as np
    torch.cuda.synchronize(workspace.device)
    h = workspace[:PS_WS_HEADER_BYTES].cpu().numpy().view(np.uint32)
    return [int(v) for v in h[:PS_WS_DONE + 1]]


def ps_lookback_config_get():
    """Current (fallback_polls, partial_windows) settings."""
    f = ctypes.c_uint32(0)
    p = ctypes.c_uint32(0)
    lib().ps_lookback_config_get(ctypes.byref(f), ctypes.byref(p))
    return int(f.value), int(p.value)


def ps_tile_elements(dtype=PS_U32) -> int:
    return int(lib().ps_tile_elements(dtype))


def ps_segmented_tile_elements() -> int:
    return int(lib().ps_segmented_tile_elements())


def ps_compact_tile_records(record_bytes: int) -> int:
    return int(lib().ps_compact_tile_records(record_bytes))


def ps_version() -> str:
    return lib().ps_version().decode()


def ps_status_string(status: int) -> str:
    return lib().ps_status_string(status).decode()


def workspace_bytes(fn: str, *args) -> int:
    """Size query of entry point ``fn`` for the given scalar arguments
    (as in the C call, with device pointers given as None)."""
    need = ctypes.c_size_t(0)
    _check(fn, getattr(lib(), fn)(None, ctypes.byref(need), *args))
    return int(need.value)
