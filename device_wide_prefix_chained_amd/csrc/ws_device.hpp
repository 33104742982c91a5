// ws_device.hpp -- the start and the end of a single-pass kernel's use of
// its workspace (header layout and hand-over rules: ws_state.hpp).
//
// Start (every thread of a workgroup): thread 0 reads the header and takes
// the workgroup's first ticket; if the call needs dirty descriptor words
// cleaned, the workgroup holding tile 0 zeroes them and raises the ready
// word.  Before its first descriptor access the control wave of every
// workgroup waits for that word (ws_wait_clean).  End: once its last
// descriptor access is done, the control wave counts the workgroup as
// finished; the last one to finish writes the header for the next call.
#pragma once

#include "dwps_device.hpp"
#include "ws_state.hpp"

namespace dwps {

__device__ __forceinline__ uint32_t hdr_load(uint32_t *hdr, int i) {
    return __hip_atomic_load(hdr + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void hdr_store(uint32_t *hdr, int i, uint32_t v) {
    __hip_atomic_store(hdr + i, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void hdr_raise(uint32_t *hdr, uint32_t bits) {
    __hip_atomic_fetch_or(hdr + kHdrError, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t uniform_u32(uint32_t v) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)v); }

// LDS copy of what thread 0 read.
struct WsShared {
    uint32_t begin[6];  // WsBegin
    uint32_t t0;        // the workgroup's first tile (num_tiles: none)
    uint32_t entry;     // the real-time counter (low 32 bits) at the workgroup's start
};

// What a workgroup knows about its call's workspace, uniform across it.
struct WsCall {
    WsBegin begin;
    WsPlan plan;
    uint32_t need;  // descriptor words of this call
    __device__ bool must_clean() const { return plan.clean_lo < plan.clean_hi; }
};

__device__ __forceinline__ WsBegin ws_shared_begin(const WsShared &sh) {
    return WsBegin{uniform_u32(sh.begin[0]), uniform_u32(sh.begin[1]), uniform_u32(sh.begin[2]),
                   uniform_u32(sh.begin[3]), uniform_u32(sh.begin[4]), uniform_u32(sh.begin[5])};
}

__device__ __forceinline__ WsBegin ws_read_begin(uint32_t *hdr) {
    return WsBegin{hdr_load(hdr, kHdrMagic), hdr_load(hdr, kHdrCapacity), hdr_load(hdr, kHdrTag),
                   hdr_load(hdr, kHdrHigh),  hdr_load(hdr, kHdrDirtyLo),  hdr_load(hdr, kHdrDirtyHi)};
}

// Called by every thread at kernel start.  `t0` receives the workgroup's
// first tile: G consecutive tiles per ticket, num_tiles when none is left
// or when the workspace is not usable (then nothing else happens).
template <int G>
__device__ __forceinline__ WsCall ws_start(uint32_t *hdr, uint64_t *desc, uint32_t need, uint32_t num_tiles,
                                           WsShared &sh, uint32_t &t0) {
    if (threadIdx.x == 0) {
        sh.entry = (uint32_t)__builtin_amdgcn_s_memrealtime();
        // the ticket is taken together with the header reads (one round
        // trip, not two) and given back if the workspace is refused, which
        // leaves the counter of a prepared workspace as it was
        const uint32_t g = take_ticket(hdr + kHdrTicket);
        const WsBegin b = ws_read_begin(hdr);
        const WsPlan p = ws_plan(b, need);
        uint32_t first = num_tiles;
        if (p.ok) {
            first = (g < (num_tiles + G - 1u) / G) ? g * G : num_tiles;
        } else {
            __hip_atomic_fetch_sub(hdr + kHdrTicket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            hdr_raise(hdr, p.error);
        }
        sh.begin[0] = b.magic;
        sh.begin[1] = b.capacity;
        sh.begin[2] = b.tag;
        sh.begin[3] = b.high;
        sh.begin[4] = b.dirty_lo;
        sh.begin[5] = b.dirty_hi;
        sh.t0 = first;
    }
    __syncthreads();
    WsCall c;
    c.begin = ws_shared_begin(sh);
    c.plan = ws_plan(c.begin, need);
    c.need = need;
    t0 = uniform_u32(sh.t0);
    if (c.plan.ok && c.must_clean() && t0 == 0u) {
        // the workgroup holding tile 0 zeroes the dirty words this call
        // uses, before any workgroup touches a descriptor
        for (uint32_t i = c.plan.clean_lo + threadIdx.x; i < c.plan.clean_hi; i += blockDim.x)
            __hip_atomic_store(desc + i, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __threadfence();
        __syncthreads();
        if (threadIdx.x == 0) hdr_store(hdr, kHdrReady, 1u);
    }
    return c;
}

// The control wave, before its first descriptor access: wait until the
// dirty words are clean.  The cleaning workgroup is running (it holds tile
// 0), so the wait ends; a limit far beyond any cleaning time turns a broken
// header into an error bit instead of a hung GPU.
__device__ __forceinline__ void ws_wait_clean(const WsCall &c, uint32_t *hdr) {
    if (!c.must_clean()) return;
    for (uint32_t spins = 0; hdr_load(hdr, kHdrReady) == 0u; ++spins) {
        if (spins >= kSpinLimit) {
            if ((threadIdx.x & 63u) == 0u) hdr_raise(hdr, kErrSpin);
            break;
        }
        __builtin_amdgcn_s_sleep(2);
    }
    __threadfence();
}

// Counts the workgroup done; the last one writes the header for the next
// call.  Called by ONE wave (lane 0 does the work): the control wave right
// after its last descriptor access -- the data waves' last stores need not
// be waited for, since no later part of this call reads them, and the last
// ticket (taken by a data wave) was consumed before the barrier the control
// wave passed in that phase -- or the first wave of a workgroup that got no
// tile.  What the call read at its start is taken again from LDS, so that
// nothing of it stays live in registers across the pipeline.  No fence: the
// counters are atomics at agent scope, and descriptor words are read only
// by later kernels (ordered by the kernel boundary); an agent-scope fence
// here would write back the XCD's L2 at the exit of every workgroup.
__device__ __forceinline__ void ws_done(const WsShared &sh, uint32_t need, uint32_t *hdr, uint32_t lane) {
    WsCall c;
    c.begin = ws_shared_begin(sh);
    c.plan = ws_plan(c.begin, need);
    c.need = need;
    if (!c.plan.ok || lane != 0u) return;
    const uint32_t done = __hip_atomic_fetch_add(hdr + kHdrDone, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (done == gridDim.x - 1u) {
        const WsEnd e = ws_end(c.begin, c.plan, c.need);
        hdr_store(hdr, kHdrTicket, 0u);
        hdr_store(hdr, kHdrDone, 0u);
        hdr_store(hdr, kHdrReady, 0u);
        hdr_store(hdr, kHdrHigh, e.high);
        hdr_store(hdr, kHdrDirtyLo, e.dirty_lo);
        hdr_store(hdr, kHdrDirtyHi, e.dirty_hi);
        hdr_store(hdr, kHdrTag, e.tag);
        __hip_atomic_fetch_add(hdr + kHdrCalls, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

}  // namespace dwps
