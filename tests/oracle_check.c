/* Host build of the C oracle under the address and undefined-behaviour
 * sanitizers (with OpenMP, as the oracle runs): every entry point on small
 * inputs and on its edge cases -- K above the number of items, empty and
 * fully masked sets, ids outside the catalog, duplicate ids, mask bits past
 * M, bf16 and fp32 inputs -- with the padding and counts those cases must
 * give.  Exit status 0 = all checks passed. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../oracle/oracle.c"

static int fails = 0;
#define CHECK(c, msg)                              \
    do {                                           \
        if (!(c)) {                                \
            printf("check failed: %s\n", msg);     \
            ++fails;                               \
        }                                          \
    } while (0)

static uint16_t bf16_of(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16); /* truncation: any bf16 value will do here */
}

int main(void) {
    enum { B = 3, D = 5, M = 4, K = 6 };
    float Hf[B * D], Ef[M * D];
    uint16_t Hb[B * D], Eb[M * D];
    for (int i = 0; i < B * D; ++i) { Hf[i] = (float)((i * 7) % 11) / 8.0f - 0.5f; Hb[i] = bf16_of(Hf[i]); }
    for (int i = 0; i < M * D; ++i) { Ef[i] = (float)((i * 5) % 13) / 16.0f - 0.25f; Eb[i] = bf16_of(Ef[i]); }
    int64_t users[B] = {2, 0, 1};
    for (int dt = 0; dt < 2; ++dt) {
        const void* H = dt == ORACLE_BF16 ? (const void*)Hb : (const void*)Hf;
        const void* E = dt == ORACLE_BF16 ? (const void*)Eb : (const void*)Ef;
        double S[B * M], sc[B * K], ls[B];
        int64_t idx[B * K];
        /* K > M: M real entries, then padding */
        oracle_full(H, E, dt, D, M, K, users, B, S, idx, sc, ls);
        for (int r = 0; r < B; ++r) {
            for (int j = 0; j < M; ++j) CHECK(idx[r * K + j] >= 0 && idx[r * K + j] < M, "full: real entry");
            for (int j = M; j < K; ++j) CHECK(idx[r * K + j] == -1 && isinf(sc[r * K + j]) && sc[r * K + j] < 0, "full: padding");
            for (int j = 1; j < M; ++j) CHECK(sc[r * K + j] <= sc[r * K + j - 1], "full: order");
            CHECK(isfinite(ls[r]), "full: lse");
        }
        /* masks: nothing allowed for user 0, items 1 and 3 for user 1 (bits past M set), all for user 2 */
        uint32_t mask[B] = {0u, 0xFFFFFFF0u | 0xAu, 0xFu};
        oracle_full_masked(H, E, dt, D, M, K, mask, 1, (int64_t[]){0, 1, 2}, B, S, idx, sc, ls);
        CHECK(isinf(ls[0]) && ls[0] < 0 && idx[0] == -1, "masked: nothing allowed");
        CHECK(((idx[K] == 1 && idx[K + 1] == 3) || (idx[K] == 3 && idx[K + 1] == 1)) && idx[K + 2] == -1, "masked: two allowed");
        CHECK(idx[2 * K + 3] >= 0 && idx[2 * K + 4] == -1, "masked: all allowed");
        /* candidate lists: user 0 empty, user 1 with bad ids and a duplicate, user 2 all items */
        int64_t off[B + 1] = {0, 0, 5, 9};
        int32_t ids[9] = {-1, 2, 2, 7, 0, 0, 1, 2, 3};
        double es[9];
        int64_t bad = oracle_cand(H, E, dt, D, M, K, off, ids, (int64_t[]){0, 1, 2}, B, es, idx, sc, ls);
        CHECK(bad == 2, "cand: two ids outside the catalog");
        CHECK(isnan(es[0]) && isnan(es[3]) && !isnan(es[1]), "cand: entry scores");
        CHECK(isinf(ls[0]) && ls[0] < 0 && idx[0] == -1, "cand: empty list");
        CHECK(idx[K + 3] == -1 && idx[K + 2] >= 0, "cand: three valid entries, duplicate kept");
        CHECK(es[1] == es[2], "cand: duplicate scored alike");
    }
    /* one row: lse of an empty set, top-K of a row with ties */
    CHECK(isinf(oracle_lse(NULL, 0)), "lse of nothing");
    double row[5] = {1.0, 3.0, 3.0, -2.0, 3.0};
    int64_t ti[7];
    double ts[7];
    oracle_topk_row(row, 5, 7, ti, ts);
    CHECK(ti[0] == 1 && ti[1] == 2 && ti[2] == 4 && ti[3] == 0 && ti[4] == 3 && ti[5] == -1 && ti[6] == -1, "topk ties and padding");
    if (fails) {
        printf("%d oracle checks failed\n", fails);
        return 1;
    }
    printf("oracle ok\n");
    return 0;
}
