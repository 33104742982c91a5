/*
 * oracle.c -- plain, sequential CPU reference for the device-wide prefix scan,
 * the CSR-segmented scan and stable stream compaction.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code, header, table or constant with the
 * GPU library: every operator, identity and loop below is written out here on
 * its own from the definitions on the pages.
 *
 * Every routine is the textbook definition executed one element at a time, in
 * index order, with no blocking, fusion or reordering.  Sources (page title,
 * section):
 *   [P1] "Single-Pass Prefix Scan with Decoupled Look-Back" -- lead section
 *        (exclusive/inclusive worked example).
 *   [P2] "Parallel Prefix Sum (Scan), in depth" -- "Inclusive, exclusive and
 *        associative" (definitions, any associative operator, commutativity
 *        not required); "What scan builds" (compaction, recurrence pair);
 *        "Numerics and determinism" (fp32 accumulation); "Failure modes"
 *        (identity padding, operand order, overflow).
 *   [P3] "Prefix scans and compaction" -- "Inclusive and exclusive scan"
 *        (identities), "Scan as an index generator" and "Worked example:
 *        Stable stream compaction" (flags -> exclusive offsets -> scatter).
 *   [P5] "GPUSegmentedScan" -- "Prefix scans and segmented scans" (segment s
 *        is [offsets[s], offsets[s+1]), N+1 offsets, reset at every segment),
 *        "Contract" (empty segments write no rows), "Limitations" (uint32
 *        addition; offsets monotonic and in bounds).
 *
 * Parity status: every exported function is pinned by the CPU test-suite
 * (worked examples printed on the pages, closed forms, library routines,
 * an O(n^2) brute force, an independent Blelloch up/down-sweep and
 * invariants).  No function here is "parity unpinned".
 *
 * Build: gcc -O2 -shared -fPIC -o liboracle.so oracle.c -lm
 * (no OpenMP, no intrinsics, no fast-math: IEEE round-to-nearest-even).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

/* Operator codes of this file (the Python wrapper maps names onto them). */
#define ORC_SUM 0
#define ORC_MAX 1
#define ORC_MIN 2
#define ORC_AND 3
#define ORC_OR 4
#define ORC_XOR 5
#define ORC_AFFINE16 6

/*
 * a (+) b, with a the EARLIER operand and b the LATER one.  [P2] "Inclusive,
 * exclusive and associative": any associative operator; commutativity is not
 * required, so the order (earlier, later) is kept everywhere.
 *   SUM       : a + b modulo 2^32 (uint32 wrap-around).
 *   MAX / MIN : keep the earlier operand unless the later one is strictly
 *               larger / smaller.
 *   AND/OR/XOR: bitwise.
 *   AFFINE16  : the pair operator for h[t] = a[t] h[t-1] + b[t] of [P2] "What
 *               scan builds", over the integers modulo 2^16, packed as
 *               (a << 16) | b.  Applying (a1,b1) first and (a2,b2) second
 *               maps h to a2 (a1 h + b1) + b2 = (a1 a2) h + (a2 b1 + b2).
 */
static uint32_t u32_combine(int op, uint32_t a, uint32_t b)
{
    switch (op) {
    case ORC_SUM:
        return a + b;
    case ORC_MAX:
        return (b > a) ? b : a;
    case ORC_MIN:
        return (b < a) ? b : a;
    case ORC_AND:
        return a & b;
    case ORC_OR:
        return a | b;
    case ORC_XOR:
        return a ^ b;
    case ORC_AFFINE16: {
        uint32_t a1 = a >> 16, b1 = a & 0xFFFFu;
        uint32_t a2 = b >> 16, b2 = b & 0xFFFFu;
        uint32_t ra = (a1 * a2) & 0xFFFFu;
        uint32_t rb = (a2 * b1 + b2) & 0xFFFFu;
        return (ra << 16) | rb;
    }
    default:
        return 0;
    }
}

/* Identity of each operator: [P3] "Inclusive and exclusive scan" (zero for
 * addition; the lowest representable value for a maximum), [P2] "Failure
 * modes" (the pad value must be the operator's identity). */
static uint32_t u32_identity(int op)
{
    switch (op) {
    case ORC_SUM:
        return 0u;
    case ORC_MAX:
        return 0u;
    case ORC_MIN:
        return 0xFFFFFFFFu;
    case ORC_AND:
        return 0xFFFFFFFFu;
    case ORC_OR:
        return 0u;
    case ORC_XOR:
        return 0u;
    case ORC_AFFINE16:
        return 0x00010000u; /* a = 1, b = 0: the map h -> h */
    default:
        return 0u;
    }
}

static int u32_op_known(int op) { return op >= ORC_SUM && op <= ORC_AFFINE16; }

/*
 * Flat scan over uint32.  [P2] "Inclusive, exclusive and associative":
 *   inclusive  y[i] = x[0] (+) ... (+) x[i]
 *   exclusive  y[0] = identity, y[i] = x[0] (+) ... (+) x[i-1]
 * written as one running accumulator.  *total (optional) receives the fold of
 * the whole input (identity when n == 0).  Returns 0, or -1 for an unknown op.
 * in == out is allowed (each x[i] is read before y[i] is written).
 */
int oracle_scan_u32(int op, int inclusive, const uint32_t *x, uint32_t *y,
                    uint64_t n, uint32_t *total)
{
    if (!u32_op_known(op))
        return -1;
    uint32_t acc = u32_identity(op);
    for (uint64_t i = 0; i < n; ++i) {
        uint32_t xi = x[i];
        if (inclusive) {
            acc = u32_combine(op, acc, xi);
            y[i] = acc;
        } else {
            y[i] = acc;
            acc = u32_combine(op, acc, xi);
        }
    }
    if (total)
        *total = acc;
    return 0;
}

/*
 * Widening sum scan: uint32 inputs, uint64 running sums ([P2] "Failure modes":
 * a 32-bit accumulator overflows on long inputs; [P3] "Scan as an index
 * generator": offsets over billions of flags need 64 bits).  The same running
 * accumulator as above, 64 bits wide, so no sum below 2^64 wraps.  *total
 * (optional) receives the sum of the whole input (0 when n == 0).
 */
int oracle_scan_u32_u64(int inclusive, const uint32_t *x, uint64_t *y,
                        uint64_t n, uint64_t *total)
{
    uint64_t acc = 0u;
    for (uint64_t i = 0; i < n; ++i) {
        uint64_t xi = (uint64_t)x[i];
        if (inclusive) {
            acc = acc + xi;
            y[i] = acc;
        } else {
            y[i] = acc;
            acc = acc + xi;
        }
    }
    if (total)
        *total = acc;
    return 0;
}

/*
 * Linear recurrence h[t] = a[t] h[t-1] + b[t] as a scan of (a, b) pairs
 * ([P2] "What scan builds": (a1, b1) then (a2, b2) combine to
 * (a1 a2, a2 b1 + b2); identity (1, 0); not commutative).  fp32 inputs,
 * fp64 accumulation, one running pair in index order:
 *   inclusive  out[t] = (a_0, b_0) (+) ... (+) (a_t, b_t)
 *   exclusive  out[0] = (1, 0), out[t] = (a_0, b_0) (+) ... (+) (a_{t-1}, b_{t-1})
 * so with h[-1] = 0 the second component of the inclusive pair is h[t].
 * ab holds n interleaved pairs; A, B receive the two components (fp64).
 * sa, sb (optional) receive the same scan over (|a|, |b|): the magnitudes
 * that scale the tolerance of an fp32 evaluation in any grouping.
 * *ta, *tb (optional) receive the fold of all n pairs.
 */
int oracle_scan_linrec_f32(int inclusive, const float *ab, double *A, double *B,
                           double *sa, double *sb, uint64_t n, double *ta, double *tb)
{
    double pa = 1.0, pb = 0.0;   /* running pair */
    double qa = 1.0, qb = 0.0;   /* running pair of magnitudes */
    for (uint64_t t = 0; t < n; ++t) {
        double at = (double)ab[2 * t], bt = (double)ab[2 * t + 1];
        if (!inclusive) {
            A[t] = pa;
            B[t] = pb;
            if (sa) sa[t] = qa;
            if (sb) sb[t] = qb;
        }
        /* (pa, pb) then (at, bt) */
        pb = at * pb + bt;
        pa = pa * at;
        qb = fabs(at) * qb + fabs(bt);
        qa = qa * fabs(at);
        if (inclusive) {
            A[t] = pa;
            B[t] = pb;
            if (sa) sa[t] = qa;
            if (sb) sb[t] = qb;
        }
    }
    if (ta) *ta = pa;
    if (tb) *tb = pb;
    return 0;
}

/*
 * fp32 sum scan, accumulated in fp64 from the fp32 inputs ([P2] "Numerics and
 * determinism": keep the accumulator in float32 or wider; the float64 answer
 * is the reference).  Also returns absprefix[i] = sum_{j<=i} |x[j]| in fp64,
 * the scale of the tolerance  |gpu_i - y_i| <= 1e-5 * absprefix[i].
 * Either output pointer may be NULL.
 */
int oracle_scan_f32_sum(int inclusive, const float *x, double *y,
                        double *absprefix, uint64_t n, double *total)
{
    double acc = 0.0;
    double absacc = 0.0;
    for (uint64_t i = 0; i < n; ++i) {
        double xi = (double)x[i];
        absacc += fabs(xi);
        if (inclusive) {
            acc += xi;
            if (y)
                y[i] = acc;
        } else {
            if (y)
                y[i] = acc;
            acc += xi;
        }
        if (absprefix)
            absprefix[i] = absacc;
    }
    if (total)
        *total = acc;
    return 0;
}

/*
 * fp32 max / min scan (op = ORC_MAX or ORC_MIN).  Exact in any grouping: the
 * result is always one of the inputs.  Ties keep the earlier operand, as in
 * the uint32 operator, so signed zeros are resolved the same way in every
 * grouping.  Identities are -inf (max) and +inf (min) ([P3] "Inclusive and
 * exclusive scan": the lowest representable value for a maximum).
 */
int oracle_scan_f32_minmax(int op, int inclusive, const float *x, float *y,
                           uint64_t n, float *total)
{
    if (op != ORC_MAX && op != ORC_MIN)
        return -1;
    float acc = (op == ORC_MAX) ? -INFINITY : INFINITY;
    for (uint64_t i = 0; i < n; ++i) {
        float xi = x[i];
        float next;
        if (op == ORC_MAX)
            next = (xi > acc) ? xi : acc;
        else
            next = (xi < acc) ? xi : acc;
        if (inclusive) {
            acc = next;
            y[i] = acc;
        } else {
            y[i] = acc;
            acc = next;
        }
    }
    if (total)
        *total = acc;
    return 0;
}

/*
 * Offsets check for the segmented scan ([P5] "Prefix scans and segmented
 * scans", "Limitations"): N segments need N+1 offsets, non-decreasing, with
 * offsets[N] <= n.  Returns -1 when valid, else the first index s at which the
 * contract breaks (offsets[s] > offsets[s+1], or s = N when offsets[N] > n).
 */
int64_t oracle_validate_offsets(const uint32_t *offsets, uint32_t num_segments,
                                uint64_t n)
{
    for (uint32_t s = 0; s < num_segments; ++s)
        if (offsets[s] > offsets[s + 1])
            return (int64_t)s;
    if ((uint64_t)offsets[num_segments] > n)
        return (int64_t)num_segments;
    return -1;
}

/*
 * Segmented uint32 sum scan ([P5] "Prefix scans and segmented scans",
 * "Contract"): for each segment s, the running total restarts at zero at
 * offsets[s] and covers [offsets[s], offsets[s+1]).  Rows that belong to no
 * segment (before offsets[0] or from offsets[N] on) and the rows of empty
 * segments (there are none) are not written.  Returns 0, or 1 + the index
 * reported by oracle_validate_offsets when the offsets break the contract
 * (nothing is written then).
 */
int64_t oracle_segmented_scan_u32(int inclusive, const uint32_t *x, uint64_t n,
                                  const uint32_t *offsets,
                                  uint32_t num_segments, uint32_t *y)
{
    int64_t bad = oracle_validate_offsets(offsets, num_segments, n);
    if (bad >= 0)
        return bad + 1;
    for (uint32_t s = 0; s < num_segments; ++s) {
        uint32_t acc = 0u;
        for (uint64_t i = offsets[s]; i < (uint64_t)offsets[s + 1]; ++i) {
            if (inclusive) {
                acc += x[i];
                y[i] = acc;
            } else {
                y[i] = acc;
                acc += x[i];
            }
        }
    }
    return 0;
}

/*
 * Stable stream compaction ([P3] "Worked example: Stable stream compaction";
 * [P2] "What scan builds"): records whose flag is nonzero are copied, bitwise
 * and in their original order, to out[0], out[1], ...; the count of kept
 * records is returned.  Slots of out past the count are not touched.
 */
uint64_t oracle_compact(const void *records, uint32_t record_bytes,
                        const uint8_t *flags, uint64_t n, void *out)
{
    const unsigned char *src = (const unsigned char *)records;
    unsigned char *dst = (unsigned char *)out;
    uint64_t j = 0;
    for (uint64_t i = 0; i < n; ++i) {
        if (flags[i] != 0) {
            memcpy(dst + j * record_bytes, src + i * record_bytes, record_bytes);
            ++j;
        }
    }
    return j;
}
