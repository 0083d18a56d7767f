// Host build of the library's HIP-free halves -- argument validation
// (validate.hpp) and planning (plan.hpp) -- run under the address and
// undefined-behaviour sanitizers.  For a grid of shapes up to and past the
// supported limits it checks that every workspace region is aligned, lies
// inside the reported total and does not overlap another, that the work
// split covers the catalog exactly, and that the index ranges the kernels
// derive from a plan (chunks, pieces, candidate regions, rows, flags) stay
// inside the regions the plan reserved; shapes too large for one launch or
// one workspace must be reported unsupported, never wrapped around.
// Exit status 0 = all checks passed.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "../full_catalog_ranking_amd/csrc/plan.hpp"
#include "../full_catalog_ranking_amd/csrc/validate.hpp"

using namespace genrec;

static long fails = 0, checks = 0;
#define CHECK(c, ...)                                                \
    do {                                                             \
        ++checks;                                                    \
        if (!(c)) {                                                  \
            if (fails < 30) printf(__VA_ARGS__), printf("\n");      \
            ++fails;                                                 \
        }                                                            \
    } while (0)

struct Region {
    size_t off;
    unsigned __int128 bytes;
    const char* name;
};

// Regions sorted by offset: aligned, disjoint, inside the total.
static void check_regions(std::vector<Region> r, size_t total, const char* what) {
    // empty regions hold nothing (their offsets need not be set)
    r.erase(std::remove_if(r.begin(), r.end(), [](const Region& x) { return x.bytes == 0; }), r.end());
    std::sort(r.begin(), r.end(), [](const Region& a, const Region& b) { return a.off < b.off; });
    for (size_t i = 0; i < r.size(); ++i) {
        CHECK(r[i].off % 256 == 0, "%s: region %s offset %zu not 256-aligned", what, r[i].name, r[i].off);
        const unsigned __int128 end = (unsigned __int128)r[i].off + r[i].bytes;
        CHECK(end <= total, "%s: region %s ends past the total", what, r[i].name);
        if (i + 1 < r.size() && r[i].bytes > 0)
            CHECK(end <= r[i + 1].off, "%s: region %s overlaps %s", what, r[i].name, r[i + 1].name);
    }
}

static unsigned __int128 u128(int64_t a) { return (unsigned __int128)a; }

static void check_dense(int B, int D, int64_t M, int K, int dt) {
    char what[128];
    snprintf(what, sizeof what, "dense B=%d D=%d M=%lld K=%d dt=%d", B, D, (long long)M, K, dt);
    const DensePlan p = plan_dense(B, D, M, K, dt);
    const unsigned __int128 full_keys = u128(B) * u128(p.key_stride) * 8;
    const unsigned __int128 keys_bytes =
        p.bounded ? (u128(p.n_pieces) * u128(p.cap) + u128(B) * u128(p.ovf_cap)) * 8 : full_keys;
    const unsigned __int128 n_rec = u128(B) * u128(p.rec_stride);
    if (!p.ok) {
        CHECK(p.total == 0, "%s: unsupported plan with a workspace size", what);
        // unsupported only when something really is too large
        const bool big = keys_bytes > kMaxWorkspace || u128(B) * u128(M) * 4 > kMaxWorkspace ||
                         (int64_t)p.main.UT * p.main.P > kMaxGrid || p.n_pieces > kMaxGrid ||
                         (p.sample && u128(B) * u128(p.n_sample) * 4 > kMaxWorkspace) ||
                         (p.sample && !p.mfma && (int64_t)B * p.pre.P > kMaxGrid);
        CHECK(big, "%s: unsupported without cause", what);
        return;
    }
    CHECK(p.total > 0 && p.total <= kMaxWorkspace, "%s: total", what);
    CHECK(p.n_pieces == (int64_t)B * p.main.P * p.pieces_per_chunk, "%s: piece count", what);
    if (p.mfma) {
        // chunks cover the catalog's tiles exactly, in order
        const int64_t nt = ceil_div(M, kMfmaTileItems);
        int64_t t = 0;
        for (int c = 0; c < p.main.P; ++c) {
            const int64_t tile0 = (int64_t)c * p.main.base + std::min(c, p.main.rem);
            const int64_t ntiles = p.main.base + (c < p.main.rem ? 1 : 0);
            CHECK(tile0 == t, "%s: chunk %d starts at tile %lld, expected %lld", what, c, (long long)tile0, (long long)t);
            CHECK(ntiles >= 1, "%s: empty chunk %d", what, c);
            // candidate sub-regions of the chunk's four lane groups (64 rows of each tile)
            const int64_t item0 = tile0 * kMfmaTileItems;
            CHECK(item0 + 4 * 64 * ntiles <= p.key_stride, "%s: chunk %d's candidate regions pass the user's", what, c);
            t += ntiles;
        }
        CHECK(t == nt, "%s: chunks cover %lld of %lld tiles", what, (long long)t, (long long)nt);
        CHECK(p.key_stride >= M, "%s: key stride", what);
        CHECK((int64_t)p.main.UT * kMfmaTileUsers >= B, "%s: user tiles", what);
        // bounded regions: only past the key budget, with a sampled fast
        // threshold, pieces smaller than their items, a collect region that
        // holds K keys and more
        CHECK(!p.bounded || (full_keys > kDefaultKeyBudget && p.fast), "%s: bounded without cause", what);
        if (p.bounded)
            CHECK(p.cap >= kCapMin && p.cap < 64 * (p.main.base + (p.main.rem ? 1 : 0)) && p.ccol > K &&
                  p.ccol % 256 == 0 && p.ovf_cap >= 2 * p.ccol, "%s: bounded sizes", what);
        CHECK(p.rec_stride == (int64_t)p.main.P * 4 + (p.bounded ? 1 : 0), "%s: records per user", what);
    } else if (!p.fused) {
        CHECK((int64_t)p.main.P * p.main.CH >= M && (int64_t)(p.main.P - 1) * p.main.CH < M, "%s: VALU chunks", what);
        CHECK(p.key_stride == M, "%s: VALU key stride", what);
    }
    if (p.sample) {
        // a split sample: splits a power of two dividing the reduction into whole k-steps, only
        // for a sample pass that would fill few CUs, and then no exact threshold
        const int64_t ke = dt == 0 ? kMfmaBlockK : kMfmaBlockK / 2;
        const int S = p.sample_splits;
        CHECK(S >= 1 && S <= kSampleMaxSplits && (S & (S - 1)) == 0 && (S == 1 || D % (ke * S) == 0), "%s: sample splits", what);
        CHECK(S == 1 || D / (ke * S) >= kSampleMinSteps, "%s: sample splits of at least the minimum k-steps", what);
        CHECK(S == 1 || (p.mfma && (int64_t)p.pre.UT * p.pre.P * S <= kNumCU), "%s: split sample fills the GPU", what);
        CHECK(p.safe_exact == (S == 1), "%s: safe threshold exact iff unsplit", what);
        CHECK(p.n_sample <= kSampleMaxItems, "%s: sample above the threshold kernel's capacity", what);
        CHECK((p.sample_tiles - 1) * p.stride * kMfmaTileItems + kMfmaTileItems <= M, "%s: sampled tile past M", what);
        CHECK(p.r_fast >= 1 && p.r_fast <= K, "%s: fast rank", what);
    }
    if (p.fused) {
        CHECK(M <= kFusedMaxM && p.main.P <= 256 && p.main.CH >= 32, "%s: fused limits", what);
        CHECK((int64_t)p.main.P * p.main.CH >= M && (int64_t)(p.main.P - 1) * p.main.CH < M, "%s: fused chunks", what);
        check_regions({{p.off_hdr, 256, "hdr"},
                       {p.off_arrive, u128(p.n_pieces) * 8, "flags"},
                       {p.off_elect, u128(B) * 8, "elect"},
                       {p.off_pm, u128(p.n_pieces) * 4, "pm"},
                       {p.off_pl, u128(p.n_pieces) * 4, "pl"},
                       {p.off_rows, u128(B) * u128(M) * 4, "rows"}},
                      p.total, what);
        return;
    }
    check_regions({{p.off_hdr, 256, "hdr"},
                   {p.off_theta, u128(B) * 4, "theta"},
                   {p.off_theta_safe, u128(B) * 4, "theta_safe"},
                   {p.off_uflag, u128(B) * 4, "uflag"},
                   {p.off_tflag, u128(ceil_div(B, kMfmaTileUsers)) * 4, "tflag"},
                   {p.off_sample, p.sample ? u128(p.sample_splits) * u128(B) * u128(p.n_sample) * 4 : 0, "sample"},
                   {p.off_pm, n_rec * 4, "pm"},
                   {p.off_pl, n_rec * 4, "pl"},
                   {p.off_pcnt, n_rec * 4, "pcnt"},
                   {p.off_preg, n_rec * 8, "preg"},
                   {p.off_keys, keys_bytes, "keys"},
                   {p.off_nst, p.bounded ? u128(B) * 32 : 0, "narrow state"},
                   {p.off_hist, p.bounded ? u128(B) * kNarrowBinsPlan * 4 : 0, "hist"},
                   {p.off_coll, p.bounded ? u128(B) * u128(p.ccol) * 8 : 0, "collect"},
                   {p.off_ccnt, p.bounded ? u128(B) * 4 : 0, "collect counts"},
                   {p.off_cbase, p.bounded ? u128(B) * 8 : 0, "collect bases"},
                   {p.off_rc, p.bounded ? 256 : 0, "rescue counts"},
                   {p.off_hgat, p.bounded ? u128(B) * u128(D) * (dt == 0 ? 2 : 4) : 0, "gathered rows"},
                   {p.off_map, p.bounded ? u128(B) * 4 : 0, "gathered users"}},
                  p.total, what);
}

static void check_cand(int B, int D, int64_t M, int64_t nnz, int dt) {
    char what[128];
    snprintf(what, sizeof what, "cand B=%d D=%d M=%lld nnz=%lld dt=%d", B, D, (long long)M, (long long)nnz, dt);
    const CandPlan p = plan_cand(B, D, M, nnz, dt);
    if (!p.ok) {
        CHECK(p.total == 0, "%s: unsupported plan with a workspace size", what);
        return;
    }
    // every list of L entries takes ceil(L / 256) pieces: at most nnz / 256 + B
    CHECK(p.n_pieces_max >= nnz / kCandPiece + B, "%s: piece bound", what);
    std::vector<Region> r = {{p.off_hdr, 256, "hdr"},
                             {p.off_begin, (u128(B) + 1) * 4, "begin"},
                             {p.off_table, u128(p.n_pieces_max) * 16, "table"},
                             {p.off_pm, u128(p.n_pieces_max) * 4, "pm"},
                             {p.off_pl, u128(p.n_pieces_max) * 4, "pl"},
                             {p.off_pcnt, u128(p.n_pieces_max) * 4, "pcnt"},
                             {p.off_preg, u128(p.n_pieces_max) * 8, "preg"},
                             {p.off_keys, u128(std::max<int64_t>(nnz, 1)) * 8, "keys"}};
    if (p.hot) {
        CHECK(p.t_max % kMfmaTileItems == 0 && p.t_max >= kMfmaTileItems, "%s: hot rows", what);
        CHECK((int64_t)p.hot_chunks.P * p.hot_chunks.UT <= kMaxGrid, "%s: hot grid", what);
        CHECK(p.n_hblk * kHotBlock >= M, "%s: hot blocks", what);
        r.push_back({p.off_cnt, u128(M) * 4, "cnt"});
        r.push_back({p.off_hot_idx, u128(M) * 4, "hot_idx"});
        r.push_back({p.off_hist, u128(kHotBins) * 4, "hist"});
        r.push_back({p.off_meta, 256, "meta"});
        r.push_back({p.off_hblk, u128(p.n_hblk) * 4, "hblk"});
        r.push_back({p.off_hot_ids, u128(p.t_max) * 4, "hot_ids"});
        r.push_back({p.off_ehot, u128(p.t_max) * u128(D) * 2, "e_hot"});
        r.push_back({p.off_shot, u128(B) * u128(p.t_max) * 4, "s_hot"});
    }
    check_regions(r, p.total, what);
}

static void check_topk(int R, int64_t N, int K) {
    char what[96];
    snprintf(what, sizeof what, "topk R=%d N=%lld K=%d", R, (long long)N, K);
    const TopkPlan p = plan_topk(R, N, K);
    if (!p.ok) {
        CHECK(p.workspace == 0, "%s: unsupported with a workspace", what);
        CHECK((int64_t)R * p.nchunk > kMaxGrid || u128(R) * u128(p.nchunk) * u128(K) * 8 > kMaxWorkspace,
              "%s: unsupported without cause", what);
        return;
    }
    CHECK((int64_t)p.nchunk * p.C >= N && (int64_t)(p.nchunk - 1) * p.C < N, "%s: chunks cover the row", what);
    if (p.filt) {
        const int64_t rs = N / 256;
        CHECK(N > kTopkSeg && K <= kTopkBoundMaxK && !p.reg && !p.row && p.C == kTopkFiltCols, "%s: filter plan", what);
        CHECK(p.filt >= kTopkFiltMinRank && p.filt < 256, "%s: the bound's rank", what);
        CHECK(255 * rs + 63 < N, "%s: sample runs inside the row", what);
        const double e = topk_filt_expect(N, p.filt);
        CHECK(e >= 3.0 * K && e <= kTopkFiltCap / 2, "%s: expected list length", what);
        CHECK(p.filt == kTopkFiltMinRank || topk_filt_expect(N, p.filt - 1) < 3.0 * K, "%s: the smallest rank", what);
        std::vector<Region> r = {{0, u128(R) * kTopkFiltCap * 8, "lists"},
                                 {p.off_thr, u128(R) * 4, "bounds"},
                                 {p.off_cnt, u128(R) * kTopkFiltParts * 4, "counts"}};
        check_regions(r, p.workspace, what);
        return;
    }
    CHECK(topk_filt_rank(N, K) == 0, "%s: the filter route whenever it applies", what);
    if (p.row) {
        CHECK(p.reg && N <= kTopkSeg && K <= kTopkRowMaxK && p.nchunk == 1 && p.C == N && p.workspace == 0,
              "%s: one-block row plan", what);
    } else if (p.reg) {
        CHECK(p.C == kTopkSeg && p.nchunk >= 2 && (int64_t)p.nchunk * K <= kTopkMergeKeys, "%s: reg plan", what);
    } else if (p.nchunk > 1) {
        CHECK((int64_t)p.nchunk * std::min<int64_t>(K, p.C) <= kTopkGather, "%s: merge gather", what);
    }
    CHECK(p.row == (N <= kTopkSeg && K <= kTopkRowMaxK), "%s: one-block rows exactly for short rows and K <= 512", what);
    if (p.nchunk > 1) CHECK(p.workspace == u128(R) * u128(p.nchunk) * u128(K) * 8, "%s: workspace", what);
}

static void check_ce(int B, int D, int64_t M) {
    char what[96];
    snprintf(what, sizeof what, "ce B=%d D=%d M=%lld", B, D, (long long)M);
    const CePlan p = plan_ce(B, D, M);
    if (!p.ok) {
        CHECK(p.bwd_total == 0, "%s: unsupported backward with a workspace", what);
    } else {
        CHECK(p.chunk >= 1 && p.n_chunks * p.chunk >= M && (p.n_chunks - 1) * p.chunk < M, "%s: chunks", what);
        CHECK(p.Mcp % kMfmaTileItems == 0 && p.Mcp >= p.chunk && p.Mcp - p.chunk < kMfmaTileItems, "%s: Mcp", what);
        // each k-blocked operand stays under 1 GiB (32-bit buffer offsets)
        CHECK(u128(p.Mcp) * u128(std::max<int64_t>(D, p.Bp)) * 2 <= (unsigned __int128)kCeBlockedMaxBytes,
              "%s: blocked operand too large", what);
        CHECK(p.splits >= 1 && p.splits <= kCeMaxSplits && (p.splits & (p.splits - 1)) == 0 && p.Mcp % p.splits == 0 &&
                  (p.Mcp / p.splits) % kMfmaBlockK == 0,
              "%s: splits", what);
        CHECK(ce_depth_h(p) == p.Mcp / p.splits + p.n_chunks + p.splits && ce_depth_e(p) == p.Bp, "%s: depths", what);
        check_regions({{p.off_hdr, 256, "hdr"},
                       {p.off_w, u128(B) * 4, "w"},
                       {p.off_ht, u128(D) * u128(p.Bp) * 2, "ht"},
                       {p.off_et, u128(D) * u128(p.Mcp) * 2, "et"},
                       {p.off_grows, u128(p.Bp) * u128(p.Mcp) * 2, "grows"},
                       {p.off_gcols, u128(p.Mcp) * u128(p.Bp) * 2, "gcols"},
                       {p.off_dhp, u128(p.splits) * u128(B) * u128(D) * 4, "dhp"}},
                      p.bwd_total, what);
    }
    if (p.fwd_ok)
        check_regions({{p.off_hdr, 256, "hdr"},
                       {p.off_w, u128(B) * 4, "w"},
                       {p.off_pm, u128(p.n_pieces) * 4, "pm"},
                       {p.off_pl, u128(p.n_pieces) * 4, "pl"},
                       {p.off_pcnt, u128(p.n_pieces) * 4, "pcnt"},
                       {p.off_preg, u128(p.n_pieces) * 8, "preg"}},
                      p.fwd_total, what);
}

static void check_validation() {
    alignas(16) static char buf[64];
    const void* A = buf;        // 16-byte aligned
    const void* A8 = buf + 8;   // 8-byte aligned only
    const int32_t* I = (const int32_t*)buf;
    const float* F = (const float*)buf;
    CHECK(check_common(A, A, GENREC_BF16, 4, 64, 100, 10, I, F, F) == GENREC_OK, "valid call rejected");
    CHECK(check_common(A, A, 2, 4, 64, 100, 10, I, F, F) == GENREC_ERR_INVALID_ARG, "dtype");
    CHECK(check_common(nullptr, A, 0, 4, 64, 100, 10, I, F, F) == GENREC_ERR_INVALID_ARG, "null H");
    CHECK(check_common(A8, A, 0, 4, 64, 100, 10, I, F, F) == GENREC_ERR_INVALID_ARG, "misaligned H");
    CHECK(check_common(A, A, 0, 0, 64, 100, 10, I, F, F) == GENREC_ERR_INVALID_ARG, "B = 0");
    CHECK(check_common(A, A, 0, -1, 64, 100, 10, I, F, F) == GENREC_ERR_INVALID_ARG, "B < 0");
    CHECK(check_common(A, A, 0, 4, 64, 0, 10, I, F, F) == GENREC_ERR_INVALID_ARG, "M = 0");
    CHECK(check_common(A, A, 0, 4, 64, 100, 0, I, F, F) == GENREC_ERR_INVALID_ARG, "K = 0");
    CHECK(check_common(A, A, 0, 4, 64, 100, GENREC_KMAX, I, F, F) == GENREC_OK, "K = KMAX");
    CHECK(check_common(A, A, 0, 4, 64, 100, GENREC_KMAX + 1, I, F, F) == GENREC_ERR_UNSUPPORTED, "K > KMAX");
    CHECK(check_common(A, A, 0, 4, 64, ((int64_t)1 << 31) - 1, 10, I, F, F) == GENREC_OK, "M = 2^31 - 1");
    CHECK(check_common(A, A, 0, 4, 64, (int64_t)1 << 31, 10, I, F, F) == GENREC_ERR_UNSUPPORTED, "M = 2^31");
    CHECK(check_common(A, A, 0, 4, 12, 100, 10, I, F, F) == GENREC_ERR_UNSUPPORTED, "bf16 D %% 8");
    CHECK(check_common(A, A, 1, 4, 12, 100, 10, I, F, F) == GENREC_OK, "fp32 D %% 4");
    CHECK(check_common(A, A, 1, 4, 6, 100, 10, I, F, F) == GENREC_ERR_UNSUPPORTED, "fp32 D %% 4 != 0");
    CHECK(check_common(A, A, 0, 4, GENREC_DMAX + 8, 100, 10, I, F, F) == GENREC_ERR_UNSUPPORTED, "D > DMAX");
    CHECK(check_ce(A, A, 4, 64, 100, I, nullptr) == GENREC_OK, "ce valid");
    CHECK(check_ce(A, A, 4, 64, 100, nullptr, F) == GENREC_ERR_INVALID_ARG, "ce null labels");
    CHECK(check_ce(A, A, 4, 60, 100, I, F) == GENREC_ERR_UNSUPPORTED, "ce D %% 8");
    CHECK(check_ce(A, A, 4, 64, (int64_t)1 << 31, I, F) == GENREC_ERR_UNSUPPORTED, "ce M");
}

int main() {
    check_validation();
    const int Bs[] = {1, 2, 3, 63, 64, 255, 256, 257, 1023, 1024, 4096, 65537, 1 << 20, 2147483647};
    const int Ds[] = {4, 8, 200, 256, 2048, 4096, 65536};
    const int64_t Ms[] = {1, 2, 255, 256, 257, 5000, 8192, 8193, 65535, 65536, 100000, 1000000, 1000001, (int64_t)1 << 26,
                          ((int64_t)1 << 31) - 1};
    const int Ks[] = {1, 10, 100, 500, 1024};
    for (int B : Bs)
        for (int D : Ds)
            for (int64_t M : Ms)
                for (int K : Ks)
                    for (int dt = 0; dt < 2; ++dt) {
                        if (dt == 0 && D % 8) continue;
                        check_dense(B, D, M, K, dt);
                    }
    const int64_t nnzs[] = {0, 1, 255, 256, 257, 6393195, (int64_t)1 << 35};
    for (int B : Bs)
        for (int D : {8, 2048})
            for (int64_t M : Ms)
                for (int64_t nnz : nnzs)
                    for (int dt = 0; dt < 2; ++dt) check_cand(B, D, M, nnz, dt);
    const int Rs[] = {1, 7, 64, 256, 100000, 2147483647};
    const int64_t Ns[] = {1, 1023, 4096, 4097, 16384, 16385, 262144, 1000000, ((int64_t)1 << 31) - 1};
    for (int R : Rs)
        for (int64_t N : Ns)
            for (int K : Ks) check_topk(R, N, K);
    for (int B : Bs)
        for (int D : {8, 40, 4096, 16384, 65536})
            for (int64_t M : Ms) check_ce(B, D, M);
    if (fails) {
        printf("%ld of %ld plan checks failed\n", fails, checks);
        return 1;
    }
    printf("plans ok: %ld checks\n", checks);
    return 0;
}
