// Host check of the MFMA kernel's tile geometry (mfma_layout.hpp): every DMA
// write lands where the fragment reads look for it, every source row is in
// bounds for every partial-tile size, and the per-lane 32-bit fast-path
// offset equals the 64-bit row offset.  Exit status 0 = all checks passed.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "../full_catalog_ranking_amd/csrc/mfma_layout.hpp"

using namespace genrec;

static int fails = 0;
#define CHECK(c, ...)                                 \
    do {                                              \
        if (!(c)) {                                   \
            if (fails < 20) printf(__VA_ARGS__), printf("\n"); \
            ++fails;                                  \
        }                                             \
    } while (0)

int main() {
    // 1. write/read agreement and coverage of one operand stage
    static int owner[MF_TI * MF_ROWB / 16];
    memset(owner, -1, sizeof owner);
    for (int w = 0; w < MF_NW; ++w)
        for (int lane = 0; lane < 64; ++lane)
            for (int j = 0; j < MF_DMA; ++j) {
                const int row = mf_dma_row(w, lane, j);
                const int kc = mf_dma_kchunk(w, lane);
                CHECK(row >= 0 && row < MF_TI, "row %d out of tile", row);
                CHECK(kc >= 0 && kc < MF_BK / 8, "k-chunk %d out of stage", kc);
                CHECK(kc == ((lane & 3) ^ mf_swz(row)), "swizzle depends on op: w%d l%d j%d", w, lane, j);
                const int wr = mf_dma_lds_byte(w, lane, j);
                CHECK(wr == mf_dma_lds_byte(w, 0, j) + lane * 16, "DMA is not wave-contiguous");
                CHECK(wr == mf_frag_lds_byte(row, kc), "DMA byte %d != fragment byte %d (row %d kc %d)", wr,
                      mf_frag_lds_byte(row, kc), row, kc);
                const int slot = wr / 16;
                CHECK(slot >= 0 && slot < MF_TI * MF_ROWB / 16, "slot out of stage");
                if (slot >= 0 && slot < MF_TI * MF_ROWB / 16) {
                    CHECK(owner[slot] == -1, "slot %d written twice", slot);
                    owner[slot] = row * 4 + kc;
                }
            }
    for (int s = 0; s < MF_TI * MF_ROWB / 16; ++s) CHECK(owner[s] != -1, "slot %d never written", s);
    // every (row, k-chunk) pair is read from a distinct slot
    static int seen[MF_TI * MF_ROWB / 16];
    memset(seen, 0, sizeof seen);
    for (int row = 0; row < MF_TI; ++row)
        for (int kc = 0; kc < MF_BK / 8; ++kc) {
            const int b = mf_frag_lds_byte(row, kc);
            CHECK(b >= 0 && b + 16 <= MF_TI * MF_ROWB && b % 16 == 0, "fragment byte %d out of stage", b);
            if (b >= 0 && b + 16 <= MF_TI * MF_ROWB) ++seen[b / 16];
        }
    for (int s = 0; s < MF_TI * MF_ROWB / 16; ++s) CHECK(seen[s] == 1, "slot %d read %d times", s, seen[s]);

    // 2. DMA byte offsets stay inside one operand tile (256 rows of D elements)
    //    for the k-chunks of a stage, and fit the 32-bit buffer offset
    const int Ds[] = {8, 64, 200, 256, 2048, 4096, 65536};
    for (int D : Ds)
        for (int w = 0; w < MF_NW; ++w)
            for (int lane = 0; lane < 64; ++lane)
                for (int j = 0; j < MF_DMA; ++j) {
                    const long long off = mf_dma_voff(w, lane, j, D);
                    const long long row = mf_dma_row(w, lane, j);
                    CHECK(off >= 0 && off < (1LL << 31), "offset overflows 32 bits");
                    CHECK(off / 2 - row * D == mf_dma_kchunk(w, lane) * 8, "offset is not row*D + k-chunk");
                    CHECK(row >= 0 && row < MF_TI, "row outside the tile");
                    // with the stage's k0 added: the 16 bytes stay inside the tile
                    // unless they run past D (the k tail, zero-masked at use)
                    const long long k0_max = ((D - 1) / MF_BK) * MF_BK;
                    CHECK(off + 2LL * k0_max + 16 <= (long long)MF_TI * D * 2 + 2LL * MF_BK,
                          "offset past the tile");
                }
    // 3. sampled tiles: one full tile inside each window of G, distinct, in order
    long long sample_cases = 0;
    const long long Gs[] = {1, 2, 32, 33, 62, 1000};
    const long long Fs[] = {1, 31, 32, 33, 390, 3906, 4095, 1000000};
    for (long long G : Gs)
        for (long long F : Fs) {
            const long long T = (F + G - 1) / G;  // sampled tiles
            long long prev = -1;
            for (long long t = 0; t < T; ++t) {
                const long long c = mf_sample_tile(t, G, F);
                ++sample_cases;
                CHECK(c >= t * G && c < t * G + G && c < F, "G %lld F %lld: window %lld -> tile %lld", G, F, t, c);
                CHECK(c > prev, "G %lld F %lld: tiles out of order", G, F);
                if (G == 1) CHECK(c == t, "G = 1 must keep the tile");
                prev = c;
            }
        }
    printf("sampled tiles: %lld checked\n", sample_cases);
    if (fails) {
        printf("%d layout checks failed\n", fails);
        return 1;
    }
    printf("layout ok\n");
    return 0;
}
