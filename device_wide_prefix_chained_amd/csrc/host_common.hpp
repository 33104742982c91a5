// host_common.hpp -- host-side helpers shared by the entry points of the
// library: workspace layout, argument checks, launch error mapping and the
// optional kernel-timing events.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "dwps.h"
#include "dwps_device.hpp"
#include "ws_state.hpp"

namespace dwps {

// Workspace: a 256-byte header (ws_state.hpp) followed by the descriptor
// words, one or two 64-bit words per tile.  Prepared once by
// ps_workspace_init; every single-pass call leaves it ready for the next.
constexpr size_t kWsHeader = 256;
static_assert(kHdrWords * 4 <= (int)kWsHeader, "header words fit the header");

inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline uint64_t ceil_div(uint64_t a, uint64_t b) { return (a + b - 1) / b; }
inline size_t ws_bytes_for_tiles(uint64_t tiles) { return kWsHeader + round_up(tiles * 8, 256); }
inline uint32_t *ws_counter(void *ws) { return static_cast<uint32_t *>(ws); }
inline uint64_t *ws_desc(void *ws) {
    return reinterpret_cast<uint64_t *>(static_cast<char *>(ws) + kWsHeader);
}

inline bool ranges_overlap(const void *a, size_t abytes, const void *b, size_t bbytes) {
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return abytes && bbytes && a0 < b0 + bbytes && b0 < a0 + abytes;
}
inline bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Size query / workspace check of the CUB two-call pattern.  Returns PS_OK
// with *done = true when the call was a size query.
inline ps_status workspace_protocol(void *ws, size_t *ws_bytes, size_t need, bool *done) {
    *done = false;
    if (!ws_bytes) return PS_ERR_NULL;
    if (!ws) {
        *ws_bytes = need;
        *done = true;
        return PS_OK;
    }
    if (*ws_bytes < need) return PS_ERR_WORKSPACE;
    return PS_OK;
}

// Prepare the header of a workspace of `bytes` bytes on `stream` (a kernel,
// not hipMemsetAsync, so that a caller may capture it in a graph).
hipError_t launch_ws_init(void *ws, size_t bytes, hipStream_t stream);

inline ps_status launch_status() {
    return hipGetLastError() == hipSuccess ? PS_OK : PS_ERR_HIP;
}

// Grid of a persistent kernel: the number of its workgroups the current
// device keeps resident (occupancy x compute units, cached per kernel and
// device), capped at `work_items`.  0 on a HIP error.
uint32_t persistent_grid(const void *kernel, int block_threads, uint32_t work_items);

// Process-wide look-back settings (ps_lookback_config), read at launch:
// stalled polls in a row before a fallback (0 = never) and whether tiles
// publish PARTIAL descriptors.
uint32_t lookback_fallback_after();
uint32_t lookback_partial();
uint32_t lookback_debug_flags();

// The look-back settings of a launch.  An in-place call runs without the
// fallback: a fallback reduces a predecessor from its input, which in place
// may already hold that predecessor's outputs.
inline LookbackCfg lookback_cfg(bool in_place) {
    return LookbackCfg{in_place ? 0u : lookback_fallback_after(), lookback_partial(), lookback_debug_flags(), 0u};
}

// Largest n that the flat entry points hand to the two-level form
// (ps_small_n_config), and the cap of that setting.
constexpr uint64_t kSmallNCap = 1ull << 24;
uint64_t small_n_max();

// Kernel timing hooks: when enabled (ps_kernel_timing), timing_begin/end
// record a HIP event pair around the main kernel of the call on `stream`.
void timing_begin(hipStream_t stream);
void timing_end(hipStream_t stream);

}  // namespace dwps
