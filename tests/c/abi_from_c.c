/* The C ABI used from plain C (and, compiled again, from C++): size queries
 * and argument errors only -- nothing here launches work, so it runs on a
 * machine without a GPU.  Prints one line per check and exits non-zero on
 * the first failure. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "dwps.h"

static int failures = 0;

static void expect(int ok, const char *what) {
    printf("%s %s\n", ok ? "ok  " : "FAIL", what);
    if (!ok) ++failures;
}

int main(void) {
    size_t need = 0;
    const uint64_t n = (uint64_t)1 << 28;
    const uint32_t tile = ps_tile_elements(PS_U32);
    const uint64_t tiles = (n + tile - 1) / tile;
    char *fake = (char *)(uintptr_t)0x40000000u; /* never dereferenced on these paths */
    size_t have;

    expect(ps_scan_exclusive_u32(NULL, &need, NULL, NULL, n, NULL, NULL) == PS_OK, "size query, 2^28 u32");
    /* header, then one 8-byte descriptor per tile, each part rounded to 256 bytes */
    expect(need == 256 + ((tiles * 8 + 255) / 256) * 256, "size = header + descriptors");
    expect(ps_scan(NULL, &need, PS_OP_AFFINE16, PS_F32, 0, NULL, NULL, 16, NULL, NULL) == PS_ERR_UNSUPPORTED,
           "AFFINE16 on fp32 is unsupported");
    have = 1u << 20;
    expect(ps_scan_inclusive_f32(fake, &have, NULL, (float *)fake, 100, NULL, NULL) == PS_ERR_NULL,
           "NULL input with n > 0");
    have = 8;
    expect(ps_scan_exclusive_u32(fake, &have, (const uint32_t *)fake, (uint32_t *)(fake + (1u << 24)), 100000,
                                 NULL, NULL) == PS_ERR_WORKSPACE,
           "workspace too small");
    have = 1u << 20;
    expect(ps_scan_exclusive_u32(fake, &have, (const uint32_t *)(fake + 2), (uint32_t *)(fake + (1u << 24)), 100,
                                 NULL, NULL) == PS_ERR_ALIGNMENT,
           "misaligned input");
    expect(ps_segmented_scan_u32(NULL, &need, NULL, (uint64_t)1 << 32, NULL, 4, NULL, 0, NULL) == PS_ERR_SIZE,
           "n = 2^32 rejected");
    expect(ps_compact(NULL, &need, NULL, 12, NULL, 10, NULL, NULL, NULL) == PS_ERR_UNSUPPORTED,
           "12-byte records are unsupported");
    expect(strlen(ps_status_string(PS_ERR_ALIAS)) > 0, "status strings");
    expect(strlen(ps_version()) > 0, "version string");
    return failures ? 1 : 0;
}
