/*
 * dwps.h -- device-wide prefix scan for AMD Instinct MI355X (gfx950).
 *
 * A single-pass chained scan with decoupled look-back, its CSR-segmented
 * variant and flag-driven stable stream compaction, behind a plain C ABI.
 *
 * Sources (page title, section):
 *   [P1] "Single-Pass Prefix Scan with Decoupled Look-Back": lead section
 *        (what an exclusive/inclusive prefix sum is); "Three states in a
 *        per-block descriptor"; "The publication protocol in code";
 *        "Where the algorithm meets the hardware".
 *   [P2] "Parallel Prefix Sum (Scan), in depth": "Inclusive, exclusive and
 *        associative"; "Scanning a whole array: three grid strategies";
 *        "Use the library" (size query with a null temporary buffer);
 *        "What scan builds" (compaction, recurrence pairs); "Failure
 *        modes".
 *   [P3] "Prefix scans and compaction": "Scan as an index generator";
 *        "Worked example: Stable stream compaction".
 *   [P5] "GPUSegmentedScan": "Prefix scans and segmented scans", "Contract",
 *        "Limitations".
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers named in/out/values/offsets/records/flags/total/num_selected
 *    are DEVICE pointers (hipMalloc'd or torch CUDA tensors) unless stated.
 *    `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *  - Calls only enqueue work on `stream` and return at once; results are
 *    visible in stream order.  The library never synchronises and never
 *    allocates device memory.
 *  - Workspace (the CUB-style two-call pattern of [P2] "Use the library"):
 *    call with ws == NULL to receive the byte count in *ws_bytes (nothing is
 *    launched, no GPU is touched); then call again with a device buffer of at
 *    least that many bytes (16-byte aligned), passing its size in *ws_bytes.
 *    The caller owns it.  A workspace is prepared ONCE, before its first use,
 *    with ps_workspace_init (which takes its full size); every call then
 *    leaves it ready for the next call of any entry point, so a call is a
 *    single kernel launch with no separate clear.  One workspace may serve
 *    calls of every size up to the size it was prepared with.  Two calls in
 *    flight at once must not share a workspace (two streams need two), and a
 *    call that does not complete (the process or the device fails mid-call)
 *    leaves it to be prepared again.  Layout: a PS_WS_HEADER_BYTES header of
 *    32-bit words (ps_ws_word), then the tile descriptors.  Diagnostics in
 *    the header: PS_WS_ERROR holds sticky ps_ws_error bits (nonzero: some
 *    call since preparation did not produce valid results); PS_WS_FALLBACKS
 *    and PS_WS_PARTIALS count look-back fallbacks and PARTIAL descriptors
 *    (the latter by the instrumented entry points only), cumulatively;
 *    PS_WS_CALLS counts completed single-pass calls.  A call on a workspace
 *    that was never prepared computes nothing and sets
 *    PS_WS_ERR_NOT_PREPARED; one on a workspace prepared smaller than it
 *    needs sets PS_WS_ERR_CAPACITY.
 *  - Argument errors are returned synchronously before anything is
 *    launched: PS_ERR_NULL (a required pointer is NULL while n > 0),
 *    PS_ERR_SIZE (n >= 2^32, or offsets beyond the supported range),
 *    PS_ERR_WORKSPACE (*ws_bytes smaller than required), PS_ERR_UNSUPPORTED
 *    (operator / dtype / record size not provided), PS_ERR_ALIAS (forbidden
 *    overlap of input and output), PS_ERR_ALIGNMENT (a pointer is not
 *    aligned to its element size).  A failed launch returns PS_ERR_HIP.
 *    Device faults surface at the caller's next synchronisation.
 *  - n == 0 is valid: nothing is written except *total (the identity) or
 *    *num_selected (0).
 *  - Arithmetic: uint32 sums wrap modulo 2^32.  fp32 operations use IEEE
 *    fp32 round-to-nearest with an fp32 accumulator; the grouping of a
 *    floating-point sum depends on run-time scheduling, so fp32 sums are not
 *    bitwise reproducible ([P1] "When not to use it").  Integer results,
 *    max/min and compaction are exact and deterministic.
 */
#ifndef DWPS_H
#define DWPS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 32-bit words of the workspace header. */
#define PS_WS_HEADER_BYTES 256
typedef enum ps_ws_word {
    PS_WS_ERROR = 1,     /* sticky ps_ws_error bits */
    PS_WS_FALLBACKS = 2, /* look-back fallbacks installed, cumulative */
    PS_WS_PARTIALS = 3,  /* PARTIAL descriptors published (instrumented entry points), cumulative */
    PS_WS_TAG = 4,       /* 9-bit tag of the next call; descriptors carry their call's tag */
    PS_WS_MAGIC = 6,     /* set by ps_workspace_init */
    PS_WS_CAPACITY = 7,  /* descriptor words the workspace holds */
    PS_WS_HIGH = 8,      /* descriptor words any call has tagged */
    PS_WS_DIRTY_LO = 9,  /* descriptor words [lo, hi) that may hold anything; */
    PS_WS_DIRTY_HI = 10, /* the next call that uses them zeroes them first */
    PS_WS_READY = 11,    /* nonzero once the call in flight has zeroed its dirty words */
    PS_WS_CALLS = 12,    /* single-pass calls completed, modulo 2^32 */
    /* the two counters every workgroup updates, on a 128-byte line of their
     * own, away from the words every workgroup reads at its start */
    PS_WS_TICKET = 32,   /* tile tickets handed out by the call in flight (0 between calls) */
    PS_WS_DONE = 33      /* workgroups of the call in flight that have finished */
} ps_ws_word;
typedef enum ps_ws_error {
    PS_WS_ERR_SPIN = 1,         /* a look-back hit its spin limit: results not valid */
    PS_WS_ERR_NOT_PREPARED = 2, /* the workspace was not prepared: nothing computed */
    PS_WS_ERR_CAPACITY = 4      /* prepared smaller than the call needs: nothing computed */
} ps_ws_error;

typedef enum ps_status {
    PS_OK = 0,
    PS_ERR_NULL = 1,
    PS_ERR_ALIAS = 2,
    PS_ERR_SIZE = 3,
    PS_ERR_WORKSPACE = 4,
    PS_ERR_UNSUPPORTED = 5,
    PS_ERR_HIP = 6,
    PS_ERR_ALIGNMENT = 7
} ps_status;

/* Element types.  PS_U64 names the widening sum: uint32 inputs, uint64
 * outputs and total (ps_scan with PS_OP_SUM only). */
typedef enum ps_dtype { PS_U32 = 0, PS_F32 = 1, PS_U64 = 2 } ps_dtype;

/* Associative operators ([P2] "Inclusive, exclusive and associative": any
 * associative operator, commutativity not required).  Operands are always
 * combined as (earlier) (+) (later).
 *   SUM      u32: a + b mod 2^32, identity 0;  f32: a + b, identity +0.0f
 *   MAX      u32: identity 0;          f32: identity -inf
 *   MIN      u32: identity 0xFFFFFFFF; f32: identity +inf
 *            (max/min keep the earlier operand on ties; f32 inputs must not
 *             hold NaN)
 *   AND/OR/XOR  u32 only; identities 0xFFFFFFFF / 0 / 0
 *   AFFINE16 u32 only: the linear-recurrence pair of [P2] "What scan builds"
 *            over the integers mod 2^16, packed (a << 16) | b:
 *            (a1,b1) (+) (a2,b2) = (a1*a2, a2*b1 + b2); identity 0x00010000.
 *            Not commutative. */
typedef enum ps_op {
    PS_OP_SUM = 0,
    PS_OP_MAX = 1,
    PS_OP_MIN = 2,
    PS_OP_AND = 3,
    PS_OP_OR = 4,
    PS_OP_XOR = 5,
    PS_OP_AFFINE16 = 6
} ps_op;

/* Prepare a workspace of ws_bytes bytes (16-byte aligned, at least
 * PS_WS_HEADER_BYTES) on `stream`: one small kernel that writes its header
 * (no call in flight, tag 0, every descriptor word marked dirty, the
 * capacity).  The descriptor words themselves are zeroed lazily, by the
 * first call that uses them.  Needed once per workspace, before its first
 * use; again only after a call failed to complete.  Calls made in the
 * same stream order afterwards see the prepared header.  Returns
 * PS_ERR_NULL, PS_ERR_ALIGNMENT or PS_ERR_WORKSPACE (too small) before
 * launching anything. */
ps_status ps_workspace_init(void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * Flat scans.  [P2] "Inclusive, exclusive and associative":
 *   inclusive  out[i] = in[0] (+) ... (+) in[i]
 *   exclusive  out[0] = identity, out[i] = in[0] (+) ... (+) in[i-1]
 * computed in one pass by the chained scan with decoupled look-back
 * ([P1] "Three states in a per-block descriptor"; [P2] "Scanning a whole
 * array: three grid strategies").
 *   in, out : n elements each; in == out (exact in-place) is allowed, any
 *             other overlap returns PS_ERR_ALIAS.  4-byte alignment
 *             required; 16-byte alignment of both selects the vector path.
 *   n       : element count, 0 <= n < 2^32.
 *   total   : optional (may be NULL) device pointer to ONE element that
 *             receives the fold of all n inputs (identity when n == 0) --
 *             the allocation size when offsets are built from lengths
 *             ([P3] "Scan as an index generator").
 * ------------------------------------------------------------------------- */
ps_status ps_scan_exclusive_u32(void *ws, size_t *ws_bytes, const uint32_t *in,
                                uint32_t *out, uint64_t n, uint32_t *total,
                                void *stream);
ps_status ps_scan_inclusive_u32(void *ws, size_t *ws_bytes, const uint32_t *in,
                                uint32_t *out, uint64_t n, uint32_t *total,
                                void *stream);
ps_status ps_scan_exclusive_f32(void *ws, size_t *ws_bytes, const float *in,
                                float *out, uint64_t n, float *total,
                                void *stream);
ps_status ps_scan_inclusive_f32(void *ws, size_t *ws_bytes, const float *in,
                                float *out, uint64_t n, float *total,
                                void *stream);

/* Widening uint32 -> uint64 sum scan (the 64-bit results [P2] "Failure
 * modes" asks for when 32-bit sums overflow; [P3] "Scan as an index
 * generator": offsets over billions of flags).  Same contract as the flat
 * scans, except:
 *   in    : n uint32 values (4-byte aligned);
 *   out   : n uint64 sums, exact (no wrap below 2^64), 8-byte aligned; out
 *           must not overlap in at all (the element sizes differ);
 *   total : optional, one uint64.
 * Each tile's 64-bit aggregate and prefix travel as two descriptor words
 * that both carry the state; a reader takes a tile only when the two agree.
 * Tiles hold 6144 elements (ps_tile_elements(PS_U64)), so the parked
 * 64-bit outputs fit the same LDS as the 32-bit scans'. */
ps_status ps_scan_exclusive_u32_u64(void *ws, size_t *ws_bytes, const uint32_t *in,
                                    uint64_t *out, uint64_t n, uint64_t *total,
                                    void *stream);
ps_status ps_scan_inclusive_u32_u64(void *ws, size_t *ws_bytes, const uint32_t *in,
                                    uint64_t *out, uint64_t n, uint64_t *total,
                                    void *stream);

/* Linear recurrence h[t] = a[t] h[t-1] + b[t] (h[-1] = 0) as one scan of
 * the pairs (a[t], b[t]) under (a1, b1) then (a2, b2) = (a1 a2, a2 b1 + b2),
 * identity (1, 0) ([P2] "What scan builds"; the operator is associative but
 * not commutative, so operands keep index order, [P2] "Failure modes").
 *   a, b         : n floats each, the coefficients as two separate arrays
 *                  (they may be the same array).
 *   out_a, out_b : n floats each, the two components of the scanned pair:
 *                  inclusive  (A[t], B[t]) = (a0,b0) (+) ... (+) (at,bt),
 *                  so B[t] = h[t] and A[t] = a[0] ... a[t];
 *                  exclusive  (A[0], B[0]) = (1, 0), then the inclusive
 *                  pair of t-1.  h from another start value h0 is
 *                  A[t] h0 + B[t].  out_a may be NULL (only B is written,
 *                  4 bytes less traffic per element); out_b is required.
 *                  out_a == a and/or out_b == b (exact in-place) is
 *                  allowed; any other overlap among the four arrays, or
 *                  between out_a and out_b, returns PS_ERR_ALIAS.
 *   total        : optional, TWO floats (A, B) of the fold of all n pairs;
 *                  (1, 0) when n == 0.
 * 4-byte alignment required, 16-byte alignment of every array selects the
 * vector path.  Arithmetic is fp32: A by products, B by fused
 * multiply-adds, in a grouping that depends on scheduling (not bitwise
 * reproducible).  Descriptors carry the pair as two words, like the
 * widening scan; tiles hold ps_linrec_tile_elements() pairs.  Not
 * reachable through ps_scan, whose one input array cannot hold two
 * planes. */
ps_status ps_scan_linrec_f32(void *ws, size_t *ws_bytes, const float *a,
                             const float *b, float *out_a, float *out_b,
                             uint64_t n, int inclusive, float *total,
                             void *stream);
uint32_t ps_linrec_tile_elements(void);

/* Generic associative-operator scan: the same pass for any (op, dtype) pair
 * listed under ps_op, and (PS_OP_SUM, PS_U64) for the widening sum.  `in`,
 * `out` and `total` point to elements of `dtype` (uint32_t or float; for
 * PS_U64 uint32_t in, uint64_t out and total); inclusive != 0 selects the
 * inclusive form.  Pairs not listed return PS_ERR_UNSUPPORTED. */
ps_status ps_scan(void *ws, size_t *ws_bytes, ps_op op, ps_dtype dtype,
                  int inclusive, const void *in, void *out, uint64_t n,
                  void *total, void *stream);

/* ps_scan for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.
 * Same arguments, results and errors as ps_scan without ws / ws_bytes: the
 * workspace is a fixed array of ps_scan_noalloc_bytes() bytes (4 MiB)
 * inside the library, one per device, held until the process ends.  Its
 * address is looked up, and its header prepared with one small kernel on
 * `stream`, by the first call on each device; later calls launch only the
 * scan.  Every call on a device shares that device's array, which keeps
 * itself ready between calls: calls that overlap on one device (two
 * streams, or the first call on one stream with a later one on another
 * before the first has run) race and give wrong results.  An n whose
 * workspace would exceed the array returns PS_ERR_SIZE (every 32-bit and
 * fp32 scan fits; the widening sum fits n up to about 1.6e9).  Allocates
 * nothing on the device or the host. */
ps_status ps_scan_noalloc(ps_op op, ps_dtype dtype, int inclusive, const void *in,
                          void *out, uint64_t n, void *total, void *stream);
size_t ps_scan_noalloc_bytes(void);

/* The two forms behind every flat entry point, callable on their own.
 *
 * ps_scan_single_pass: the chained scan with decoupled look-back, at every
 * n.
 *
 * ps_scan_two_level: the two-level (reduce-then-scan) form ([P1] the
 * two-level form and "When not to use it"; [P2] "Scanning a whole array:
 * three grid strategies"): fold each tile of ps_two_level_tile_elements()
 * elements, scan the tile totals, scan each tile again from its total's
 * prefix.  Up to 1024 tiles the tile totals are folded by the final pass
 * itself (two launches; one launch for a single tile); beyond, one
 * workgroup scans them in between (three launches).  It reads the input
 * twice (12 instead of 8 bytes per 32-bit element) but has no descriptors
 * and no look-back, so on small inputs it finishes sooner.  It keeps its
 * tile totals in the descriptor area of the workspace, as words that read
 * as unpublished descriptors, and does not touch the header: it needs no
 * preparation, and a prepared workspace stays ready.
 *
 * Both take the arguments of ps_scan and give the same results.  The flat
 * entry points (ps_scan, ps_scan_{ex,in}clusive_{u32,f32,u32_u64},
 * ps_scan_linrec_f32) run the two-level form for n up to the
 * ps_small_n_config setting and the single-pass form above it. */
ps_status ps_scan_single_pass(void *ws, size_t *ws_bytes, ps_op op, ps_dtype dtype,
                              int inclusive, const void *in, void *out, uint64_t n,
                              void *total, void *stream);
ps_status ps_scan_two_level(void *ws, size_t *ws_bytes, ps_op op, ps_dtype dtype,
                            int inclusive, const void *in, void *out, uint64_t n,
                            void *total, void *stream);
uint32_t ps_two_level_tile_elements(void);

/* Largest n that the flat entry points hand to the two-level form, for
 * every later call of this process (default 2^23, the measured crossover on
 * MI355X; 0 = always single-pass; above 2^24 returns PS_ERR_SIZE).  The size
 * queries of the flat entry points do not depend on it: up to 2^24
 * elements they report a workspace that fits either form. */
ps_status ps_small_n_config(uint64_t max_elements);
uint64_t ps_small_n_config_get(void);

/* ---------------------------------------------------------------------------
 * Segmented uint32 sum scan over CSR offsets ([P5] "Prefix scans and
 * segmented scans", "Contract", "Limitations"; the carried segment flag of
 * [P2] "What scan builds").
 *   values       : n uint32 inputs.
 *   offsets      : num_segments + 1 uint32 offsets; segment s is
 *                  [offsets[s], offsets[s+1]).  The terminal offset is
 *                  mandatory; repeated offsets are empty segments.  Offsets
 *                  must be non-decreasing with offsets[num_segments] <= n:
 *                  this is ASSUMED, not checked, on this hot path (use
 *                  ps_validate_offsets when unsure).
 *   out          : n uint32 outputs.  For every row i of segment s:
 *                  exclusive  out[i] = sum of values[offsets[s] .. i-1]
 *                  inclusive  out[i] = sum of values[offsets[s] .. i]
 *                  (mod 2^32).  Rows outside [offsets[0],
 *                  offsets[num_segments]) belong to no segment and are NOT
 *                  written; empty segments write nothing.
 *   inclusive    : nonzero for the inclusive form.
 * Any overlap of out with values or offsets returns PS_ERR_ALIAS.
 * num_segments may be 0 (nothing is written); num_segments = 2^32 - 1 (an
 * offsets array of 2^32 entries) returns PS_ERR_SIZE, as does n >= 2^32.
 * One kernel runs per call: the single-pass scan, which reads the values
 * and, per tile, the offsets that fall into it (its segment starts) once,
 * and writes every row of a segment once.  The workspace holds the header
 * and one descriptor per tile. */
ps_status ps_segmented_scan_u32(void *ws, size_t *ws_bytes,
                                const uint32_t *values, uint64_t n,
                                const uint32_t *offsets, uint32_t num_segments,
                                uint32_t *out, int inclusive, void *stream);

/* Optional check of the offsets contract above, on the device.  Writes to
 * *result (device int64): -1 when valid, else the first index s with
 * offsets[s] > offsets[s+1], or num_segments when offsets[num_segments] > n.
 * Needs no workspace. */
ps_status ps_validate_offsets(const uint32_t *offsets, uint32_t num_segments,
                              uint64_t n, int64_t *result, void *stream);

/* ---------------------------------------------------------------------------
 * Stable stream compaction ([P3] "Worked example: Stable stream compaction";
 * [P2] "What scan builds"): every record whose flag is nonzero is copied,
 * bitwise and in input order, to out[0], out[1], ...  The positions are the
 * exclusive scan of the flags, fused into the same pass (never materialised);
 * *num_selected (device uint64) receives the count = last offset + last flag.
 * Slots of out at or past the count are not touched.
 *   records      : n records of record_bytes bytes each (4, 8 or 16),
 *                  aligned to record_bytes.
 *   flags        : n bytes, 0 = drop, anything else = keep.
 *   out          : room for n records (the count is not known in advance).
 * out must not overlap records or flags (PS_ERR_ALIAS). */
ps_status ps_compact(void *ws, size_t *ws_bytes, const void *records,
                     uint32_t record_bytes, const uint8_t *flags, uint64_t n,
                     void *out, uint64_t *num_selected, void *stream);

/* Staged compaction: the same contract and results as ps_compact, computed
 * as two separate passes instead of one fused kernel ([P3] "Worked example:
 * Stable stream compaction": flags -> exclusive scan -> scatter): the flat
 * scan of the keep flags (nonzero counts as 1) into uint32 offsets in the
 * workspace, then a scatter of every kept record to its offset.  It moves
 * 1 + 4 + 1 + 4 + record_bytes bytes per record (plus record_bytes per kept
 * record) against the fused kernel's 1 + record_bytes, and exists to
 * measure what the fusion saves.  The workspace holds the scan's own, n
 * offsets and the count; the offsets' words are left marked dirty, so the
 * next single-pass call that needs them zeroes them first.  The scatter
 * writes no record to a position at or past n (a guard against offsets
 * left unwritten when the workspace was not prepared). */
ps_status ps_compact_staged(void *ws, size_t *ws_bytes, const void *records,
                            uint32_t record_bytes, const uint8_t *flags, uint64_t n,
                            void *out, uint64_t *num_selected, void *stream);
/* Records per tile of the compaction kernel for a record width (4, 8 or
 * 16 bytes; 0 for any other width). */
uint32_t ps_compact_tile_records(uint32_t record_bytes);

/* ---------------------------------------------------------------------------
 * Measurement and diagnostics (not part of the scan itself).
 * ------------------------------------------------------------------------- */

/* Plain streaming copy of n uint32 (16-byte vector path when aligned): the
 * practical HBM ceiling next to which the scans are read, and the reference
 * kernel of known size used to scale the hardware byte counters. */
ps_status ps_copy_u32(const uint32_t *in, uint32_t *out, uint64_t n, void *stream);

/* The two halves of that ceiling: a stream that only reads n uint32, with
 * the copy's access shape (in 16-byte aligned, n a multiple of 4, else
 * PS_ERR_ALIGNMENT; *sink, one device word, is written only in the
 * practically impossible case that the fold of the data hits a fixed
 * constant), and one that only writes (fills n uint32 with `value`, in the
 * fastest write shape of ps_stream_shape: 64 threads x 4 vectors, plain
 * stores; also a plain fill that records no memset node when captured in a
 * graph). */
ps_status ps_read_u32(const uint32_t *in, uint64_t n, uint32_t *sink, void *stream);
ps_status ps_fill_u32(uint32_t *out, uint64_t n, uint32_t value, void *stream);

/* The linear recurrence's access shape as a plain stream, the practical
 * ceiling of ps_scan_linrec_f32: reads the float planes a and b (n each)
 * and writes out_b[i] = a[i] * b[i] and, when out_a is not null, out_a[i] =
 * a[i] + b[i] -- two planes read, one or two written, with the copy's
 * 16-byte vectors.  Every array 16-byte aligned and n a multiple of 4, else
 * PS_ERR_ALIGNMENT; overlapping arrays: PS_ERR_ALIAS. */
ps_status ps_stream_planes_f32(const float *a, const float *b, float *out_a, float *out_b,
                               uint64_t n, void *stream);

/* A plain stream with a given mix of read and written bytes, the practical
 * ceiling of a kernel that reads n_in uint32 and writes n_out: the 16-byte
 * vectors both sides have (the first min(n_in, n_out) / 4) are copied in the
 * copy's access shape, then the rest of the longer side is read alone or
 * written alone.  out receives in's first min(n_in, n_out) words, then
 * zeros up to n_out.  Arrays 16-byte aligned and n_in, n_out multiples of 4,
 * else PS_ERR_ALIGNMENT; in and out overlapping: PS_ERR_ALIAS. */
ps_status ps_stream_mix_u32(const uint32_t *in, uint64_t n_in, uint32_t *out, uint64_t n_out,
                            void *stream);

/* The same byte mix spread evenly, for read-heavy mixes (n_out <= n_in, else
 * PS_ERR_UNSUPPORTED): workgroup b of ceil(n_in / 4096) reads the 16-byte
 * vectors [1024 b, 1024 (b + 1)) of in and writes the vectors [oc b,
 * oc (b + 1)) of out, oc = ceil(1024 (n_out / 4) / (n_in / 4)); output
 * vector oc b + j is input vector min(1024 b + j, n_in / 4 - 1).  It shows
 * what a kernel that
 * stores between its loads in every workgroup can reach.  Arrays 16-byte
 * aligned and n_in, n_out multiples of 4, else PS_ERR_ALIGNMENT; in and out
 * overlapping: PS_ERR_ALIAS. */
ps_status ps_stream_mix_even_u32(const uint32_t *in, uint64_t n_in, uint32_t *out, uint64_t n_out,
                                 void *stream);

/* The three plain streams in one of several access shapes, for a sweep that
 * shows whether the stream helpers above run at the memory's rate:
 * PS_STREAM_WRITE fills n uint32 of out with `value` (in unused),
 * PS_STREAM_COPY copies in to out, PS_STREAM_READ reads n uint32 of in (out
 * is a one-word sink, written only in the practically impossible case that
 * the fold of the data hits a fixed constant).  Shape: `threads` per
 * workgroup (64, 128 or 256), `vecs` 16-byte vectors per thread and block
 * (4, 8 or 16), non-temporal or plain loads and stores, one workgroup per
 * block of threads * vecs vectors or (persistent != 0) the resident grid
 * striding over the blocks.  Any other kind, threads or vecs:
 * PS_ERR_UNSUPPORTED; streamed arrays 16-byte aligned and n a multiple of 4,
 * else PS_ERR_ALIGNMENT; n >= 2^32: PS_ERR_SIZE; overlapping copy:
 * PS_ERR_ALIAS. */
enum { PS_STREAM_WRITE = 0, PS_STREAM_COPY = 1, PS_STREAM_READ = 2 };
ps_status ps_stream_shape(int kind, int threads, int vecs, int nontemporal, int persistent,
                          const uint32_t *in, uint32_t *out, uint64_t n, uint32_t value,
                          void *stream);

/* Exclusive uint32 sum scan (same kernel as ps_scan_exclusive_u32, built
 * with per-tile instrumentation of the look-back of [P1] "Why the work
 * stays linear").  stats: device buffer of 16 * tiles uint32, tiles
 * reported by ps_lookback_tiles(n); per tile, times in ticks of the 100 MHz
 * real-time counter:
 *   [0] poll rounds of its look-back, [1] windows of ps_lookback_window()
 *   predecessors walked, [2] look-back time after the barrier its first
 *   poll straddles, [3] polls that found an unpublished predecessor;
 *   [4]-[7] the phase that scanned the tile as the pipeline's control wave
 *   saw it: from the start of the phase to its first barrier, waiting
 *   there, from there to its second barrier, waiting there (they add up to
 *   the phase; a long wait means the data waves came later);
 *   [8]-[12] a timeline, low 32 bits of the counter: [8] start of the
 *   tile's scan phase, [9] start of the phase that stored it, [10] the
 *   workgroup (blockIdx), [11] that workgroup's start, [12] for the last
 *   tile a workgroup stored, the time the workgroup's control wave
 *   finished (0 for other tiles); [13], [14] when the phase that stored
 *   the tile scanned no tile (the pipeline's drain), that phase's parts
 *   as in [4]-[7], two 16-bit values per word (low half first); [15]
 *   (flat scan and recurrence) the phase that scanned the tile as the
 *   first data wave saw it, three 10-bit fields in ticks (saturating at
 *   1023), low bits first: from leaving the second barrier of the phase
 *   before to the end of the scan, from leaving the first barrier to the
 *   last store of the stored tile issued, from leaving the first barrier to
 *   reaching the second; (segmented scan) when the data waves reached the
 *   first barrier of that phase, in ticks after the control wave's start of
 *   the phase (0 for a data wave that came before it, at most 1023): bits
 *   0-9 the first data wave, bits 10-19 the last, bits 20-23 the last
 *   one's index, bits 24-27 the first one's; (compaction) 0.
 * aggregate_only != 0 (a test of the sliding window): tiles after tile 0
 * never publish their inclusive prefix, so every look-back walks back to
 * tile 0 -- quadratic in the tile count, meant for small n only. */
ps_status ps_lookback_stats_u32(void *ws, size_t *ws_bytes, const uint32_t *in,
                                uint32_t *out, uint64_t n, uint32_t *stats,
                                int aggregate_only, void *stream);
uint64_t ps_lookback_tiles(uint64_t n);

/* The same per-tile statistics for the other single-pass kernels, each the
 * kernel of its ordinary entry point built with the instrumentation (same
 * results; a few percent slower).  `stats` holds 16 uint32 per tile of
 * that kernel, in the layout above; tiles that do not look back (the
 * second of a ticket group; in the segmented scan also tiles whose first
 * element starts a segment, and tile 0) show zero polls.  Every array must
 * be 16-byte aligned (the instrumented build has only the vector path),
 * else PS_ERR_ALIGNMENT.
 *   ps_scan_lookback_stats: ps_scan for (PS_OP_SUM, PS_U32), (PS_OP_SUM,
 *     PS_F32) and (PS_OP_MAX, PS_F32), single-pass form at every n;
 *     ps_lookback_tiles(n) tiles.  Other pairs: PS_ERR_UNSUPPORTED.
 *   ps_segmented_lookback_stats_u32: ps_segmented_scan_u32;
 *     ceil(n / ps_segmented_tile_elements()) tiles.
 *   ps_compact_lookback_stats: ps_compact for 16-byte records only (else
 *     PS_ERR_UNSUPPORTED); ceil(n / ps_compact_tile_records(16)) tiles.
 *   ps_linrec_lookback_stats: ps_scan_linrec_f32 (no total), single-pass
 *     form at every n; ceil(n / ps_linrec_tile_elements()) tiles. */
ps_status ps_scan_lookback_stats(void *ws, size_t *ws_bytes, ps_op op, ps_dtype dtype,
                                 int inclusive, const void *in, void *out, uint64_t n,
                                 uint32_t *stats, void *stream);
ps_status ps_segmented_lookback_stats_u32(void *ws, size_t *ws_bytes,
                                          const uint32_t *values, uint64_t n,
                                          const uint32_t *offsets, uint32_t num_segments,
                                          uint32_t *out, int inclusive, uint32_t *stats,
                                          void *stream);
ps_status ps_compact_lookback_stats(void *ws, size_t *ws_bytes, const void *records,
                                    uint32_t record_bytes, const uint8_t *flags, uint64_t n,
                                    void *out, uint64_t *num_selected, uint32_t *stats,
                                    void *stream);
ps_status ps_linrec_lookback_stats(void *ws, size_t *ws_bytes, const float *a, const float *b,
                                   float *out_a, float *out_b, uint64_t n, int inclusive,
                                   uint32_t *stats, void *stream);
/* Predecessor descriptors read per look-back poll (64 lanes x K words). */
uint32_t ps_lookback_window(void);
/* Tiles claimed per ticket of the flat scan: a workgroup scans that many
 * consecutive tiles, and only the first of each group looks back (the others
 * take the inclusive prefix of the tile before them, which the same
 * workgroup computed); their stats rows show zero polls. */
uint32_t ps_lookback_group(void);

/* Look-back settings of every later call of this process (calls already
 * enqueued keep theirs); not synchronised with calls made at the same time
 * from other threads.
 *   fallback_polls  : after this many polls in a row that find an
 *                     unpublished predecessor, the waiting tile reduces that
 *                     predecessor's input itself and installs the result
 *                     with a compare-and-swap, so the first of several such
 *                     tiles wins ([P4] "Decoupled Fallback").  0 = never.
 *                     Default 4096 (milliseconds of waiting; the protocol
 *                     already guarantees progress on this GPU, so the
 *                     fallback is a safety valve).
 *   partial_windows : a tile whose look-back has walked this many windows of
 *                     ps_lookback_window() predecessors without reaching an
 *                     inclusive prefix publishes a PARTIAL descriptor after
 *                     every further window -- the fold of the tiles it has
 *                     covered, itself included, and their count -- which
 *                     later look-backs jump in one read ([P1] "Why the work
 *                     stays linear", the bounded-window variant with W =
 *                     partial_windows windows).  0 = never.  Default 4:
 *                     ordinary look-backs end within two windows and never
 *                     publish; a threshold of 1 would publish on ordinary
 *                     walks, and the extra store and the short jumps it
 *                     offers slow the scans by 10-20%.
 * Calls whose output is their input (exact in-place) never fall back: the
 * input of a stalled predecessor may already hold its outputs.  Integer
 * results do not depend on either setting; fp32 results stay within the
 * same bounds (a fallback changes the grouping). */
ps_status ps_lookback_config(uint32_t fallback_polls, uint32_t partial_windows);
void ps_lookback_config_get(uint32_t *fallback_polls, uint32_t *partial_windows);

/* Debug settings of every later single-pass call of this process (a test
 * aid, like ps_lookback_config; not for production use).
 *   PS_DEBUG_WITHHOLD_AGGREGATES: no tile publishes its AGGREGATE (a tile
 *     publishes only its inclusive PREFIX, and PARTIALs), so a look-back
 *     that reaches a tile whose prefix is not yet known stalls there; with
 *     a fallback configured (ps_lookback_config), the fallback reduces that
 *     tile's input and installs the aggregate its owner withheld ([P4]
 *     "Decoupled Fallback").  Results must be unchanged; PS_WS_FALLBACKS
 *     shows how many were installed.  Without a fallback the chain of
 *     prefixes still completes, only serially.
 * Other bits return PS_ERR_UNSUPPORTED.  0 = off (default). */
typedef enum ps_debug_flag { PS_DEBUG_WITHHOLD_AGGREGATES = 1 } ps_debug_flag;
ps_status ps_lookback_debug(uint32_t flags);
uint32_t ps_lookback_debug_get(void);

/* Kernel timing with HIP events placed around the main scan kernel of a
 * call.  every = 0 turns timing
 * off; every = N >= 1 starts a new measurement that times the 1st, (N+1)th,
 * (2N+1)th ... call from now on (1 = every call); a negative value returns
 * PS_ERR_SIZE.  ps_kernel_timing_read synchronises on the recorded events
 * and returns the summed milliseconds and the number of timed launches.
 * The events are created with hipEventDisableSystemFence (recording one
 * writes back and invalidates no cache) and are recycled across
 * measurements, so a timed call creates none once a first measurement has
 * run; each timed call still carries two event packets (a few µs), which
 * timing a sample of the calls spreads thin. */
ps_status ps_kernel_timing(int every);
ps_status ps_kernel_timing_read(double *total_ms, uint64_t *launches);

/* Elements per tile of the flat scan kernel for `dtype` (PS_U64: the
 * widening scan), of the segmented
 * scan kernel, and the library version string. */
uint32_t ps_tile_elements(ps_dtype dtype);
uint32_t ps_segmented_tile_elements(void);
const char *ps_version(void);
const char *ps_status_string(ps_status status);

#ifdef __cplusplus
}
#endif

#endif /* DWPS_H */
