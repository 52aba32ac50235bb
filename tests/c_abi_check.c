/* C11 client of libprism: exercises the parts of the C ABI that are decided
 * on the host (workspace sizes, status strings, the candidate-shape table, the
 * Hilbert zone order and argument checks made before any launch), so it runs
 * without a GPU.  Built and run by tests/test_c_abi.py; exit status 0 when
 * every check holds, else the number of the first failing check. */
#include <stdio.h>
#include <string.h>

#include "prism.h"

#define CHECK(n, cond)                                                       \
    do {                                                                     \
        if (!(cond)) {                                                       \
            fprintf(stderr, "check %d failed: %s\n", (n), #cond);           \
            return (n);                                                      \
        }                                                                    \
    } while (0)

int main(void) {
    /* workspace sizes: positive, and larger for more heads */
    const int ops[] = {PRISM_OP_SELECT, PRISM_OP_ATTN_FWD, PRISM_OP_ATTN_BWD, PRISM_OP_ROUTED_FWD,
                       PRISM_OP_ROUTED_BWD, PRISM_OP_SELECT_SUB};
    for (size_t i = 0; i < sizeof ops / sizeof ops[0]; ++i) {
        const size_t one = prism_workspace_size(ops[i], 4096, 1, 64, 16, 256);
        const size_t two = prism_workspace_size(ops[i], 4096, 2, 64, 16, 256);
        CHECK(1, one > 0 && two > one);
    }
    CHECK(2, prism_workspace_size(PRISM_OP_SELECT, 0, 1, 64, 16, 256) == 0);
    CHECK(3, prism_workspace_size(PRISM_OP_FLAT_ROUTE, 0, 2, 0, 16, 0) >= 2 * 16 * sizeof(double));

    /* status strings */
    for (int s = PRISM_OK; s <= PRISM_E_HIP; ++s) CHECK(4, strlen(prism_status_string((prism_status)s)) > 0);

    /* the 16 candidate shapes: power-of-two edges in {2, 4, 8}, volumes 64 / 128 / 256 in order */
    int32_t c[16][3];
    prism_candidate_shapes(c);
    int last = 0;
    for (int i = 0; i < 16; ++i) {
        const int vol = c[i][0] * c[i][1] * c[i][2];
        CHECK(5, vol == 64 || vol == 128 || vol == 256);
        CHECK(6, vol >= last);
        last = vol;
        for (int a = 0; a < 3; ++a) CHECK(7, c[i][a] == 2 || c[i][a] == 4 || c[i][a] == 8);
    }

    /* Hilbert zone order of a 2 x 2 x 2 zone grid: a permutation that starts at
     * zone 0 and moves one zone along one axis at each step */
    int32_t order[8], seen[8] = {0};
    CHECK(8, prism_hilbert_zone_order(16, 16, 16, order) == PRISM_OK);
    CHECK(9, order[0] == 0);
    for (int i = 0; i < 8; ++i) {
        CHECK(10, order[i] >= 0 && order[i] < 8 && !seen[order[i]]);
        seen[order[i]] = 1;
        if (i) {
            const int a = order[i - 1], b = order[i];
            const int d = (a / 4 != b / 4) + ((a / 2) % 2 != (b / 2) % 2) + (a % 2 != b % 2);
            CHECK(11, d == 1);
        }
    }
    CHECK(12, prism_hilbert_zone_order(12, 16, 16, order) == PRISM_E_GRID);

    /* argument checks before any launch (no device memory is touched) */
    int32_t so[17], si[256];
    int64_t total;
    CHECK(13, prism_select(NULL, NULL, PRISM_BF16, 4096, 1, 64, 64, 64, NULL, 16, 4, 0.9, 0.125f, so, si, 256,
                           &total, NULL, NULL, 0, 0) == PRISM_E_ARG);
    CHECK(14, strlen(prism_last_error()) > 0);
    const prism_raster_layout bad = {8, 8, 12, (const uint8_t*)0x1000, NULL, 128, 64};
    CHECK(15, prism_sparse_attn_fwd((void*)0x10000, (void*)0x20000, (void*)0x30000, (void*)0x40000,
                                    (float*)0x50000, NULL, PRISM_BF16, 768, 1, 64, 64, 64, (const int32_t*)0x60000, 12,
                                    (const int32_t*)0x70000, (const int32_t*)0x80000, 144, 0.125f, &bad, NULL, 0,
                                    0) == PRISM_E_GRID);
    printf("c abi ok\n");
    return 0;
}
