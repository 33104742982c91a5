"""Device-wide single-pass prefix scan for AMD Instinct MI355X (gfx950).

The computation lives in the HIP library ``libdwps.so`` (sources in
``csrc/``, C ABI in ``include/dwps.h``); this package is its thin Python
binding.  Functions carry the names of the C entry points.
"""
from ._binding import (  # noqa: F401
    OPS,
    PS_F32,
    PS_OP_AFFINE16,
    PS_OP_AND,
    PS_OP_MAX,
    PS_OP_MIN,
    PS_OP_OR,
    PS_OP_SUM,
    PS_OP_XOR,
    PS_U32,
    DwpsError,
    lib,
    ps_compact,
    ps_compact_tile_records,
    ps_copy_u32,
    ps_kernel_timing,
    ps_kernel_timing_read,
    ps_lookback_stats_u32,
    ps_lookback_config,
    ps_lookback_config_get,
    ps_lookback_group,
    ps_lookback_tiles,
    ps_lookback_window,
    ps_scan,
    ps_scan_exclusive_f32,
    ps_scan_exclusive_u32,
    ps_scan_inclusive_f32,
    ps_scan_inclusive_u32,
    ps_segmented_scan_u32,
    ps_segmented_tile_elements,
    ps_status_string,
    ps_tile_elements,
    ps_validate_offsets,
    ps_version,
    workspace_bytes,
)
