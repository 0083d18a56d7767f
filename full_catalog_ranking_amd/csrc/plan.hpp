// Host-side planning for the ranking head: variant choice, work split and
// workspace layout.  Pure C++ (no HIP), so it can be unit-tested on any host.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <algorithm>

namespace genrec {

constexpr int kNumCU = 256;            // MI355X compute units
constexpr int kMfmaTileItems = 256;    // items per MFMA tile
constexpr int kMfmaTileUsers = 256;    // users per MFMA tile
constexpr int kMfmaBlockK = 32;        // reduction elements per k-step (and per k-block of a blocked operand)
constexpr int kStreamMaxB = 1;         // bf16 batches up to this size use the VALU path (a half-empty MFMA tile still beats re-reading E per user)
constexpr int64_t kSampleMinM = 65536; // smaller catalogs skip the threshold pre-pass
constexpr int64_t kSampleMinStride = 32; // sample every G-th catalog tile, G >= 32
constexpr int64_t kSampleMaxTiles = 128; // sampled items per user at most 128 * 256
constexpr int64_t kSampleMaxItems = 32768;  // = kSampleMaxTiles * 256: one user's sample fits the threshold kernel
constexpr int kFastOversample = 4;     // fast threshold: expected candidates ~ 4 K
// MFMA path: the sample only has to place the fast threshold at rank >= 32 of
// the sampled scores.  The number of catalog items above the r-th largest of
// n sampled scores is about M r / n with a Gamma(r)-shaped spread, so at
// r = 32 and 4 K expected the chance of fewer than K (a rescue) is ~1e-9 per
// user.  A larger sample buys nothing there and costs a pass over more tiles.
constexpr int64_t kFastMinRank = 32;
constexpr int64_t kStreamPieces = 2048;  // target work pieces of the VALU path
constexpr int64_t kStreamChunkAlign = 32;
constexpr int kCandPiece = 256;        // candidate entries per piece (matches the kernels)

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

struct Chunking {
    int UT = 1, P = 1, base = 0, rem = 0;  // MFMA: P chunks of base(+1) tiles over UT user tiles
    int64_t CH = 0;                        // VALU: items per chunk (P chunks)
};

// The merge's smaller build (LDS gather of 2,048 keys, 512-piece batches)
// serves users expected to hold at most that many candidates and pieces.
constexpr int kMergeSmallGather = 2048;
constexpr int kMergeSmallPieces = 512;

struct DensePlan {
    bool mfma = false;
    bool sample = false;
    int64_t stride = 1;        // G: the sample holds catalog tiles 0, G, 2G, ... (full tiles only)
    int64_t sample_tiles = 0;  // number of sampled 256-row tiles
    int64_t n_sample = 0;      // sampled items = 256 * sample_tiles
    // Fast threshold (MFMA path): the r_fast-th largest sampled score instead
    // of the K-th, r_fast ~ 4 K n_sample / M, so that about 4 K catalog items
    // are expected to pass.  A user with fewer than K candidates is detected
    // by the merge and recomputed by the rescue pass with the K-th sampled
    // score, which at least K catalog items always reach.
    int r_fast = 0;
    bool fast = false;
    Chunking main, pre;
    int pieces_per_chunk = 1;  // MFMA: one piece per (user, chunk, lane group) = 4
    int64_t n_pieces = 0;
    int64_t key_stride = 0;    // candidate-region elements per user
    bool merge_small = false;  // the merge's smaller build serves this shape (a speed choice)
    size_t off_hdr = 0, off_theta = 0, off_theta_safe = 0, off_uflag = 0, off_tflag = 0, off_sample = 0,
           off_pm = 0, off_pl = 0, off_pcnt = 0, off_preg = 0, off_keys = 0, total = 0;
};

inline Chunking chunk_mfma(int B, int64_t n_tiles) {
    Chunking c;
    c.UT = (int)ceil_div(B, kMfmaTileUsers);
    const int64_t nt = n_tiles;
    const int64_t want = std::max<int64_t>(1, kNumCU / c.UT);
    c.P = (int)std::max<int64_t>(1, std::min(nt, want));
    c.base = (int)(nt / c.P);
    c.rem = (int)(nt % c.P);
    return c;
}

inline Chunking chunk_stream(int B, int64_t n_items) {
    Chunking c;
    int64_t ch = ceil_div(n_items * (int64_t)B, kStreamPieces);
    ch = std::max<int64_t>(kStreamChunkAlign, ceil_div(ch, kStreamChunkAlign) * kStreamChunkAlign);
    c.CH = ch;
    c.P = (int)ceil_div(n_items, ch);
    return c;
}

// dtype: 0 = bf16, 1 = f32.
inline DensePlan plan_dense(int B, int D, int64_t M, int K, int dtype) {
    (void)D;
    DensePlan p;
    p.mfma = dtype == 0 && B > kStreamMaxB;
    const int64_t full_tiles = M / kMfmaTileItems;
    int64_t want_tiles = kSampleMaxTiles;
    if (p.mfma && K > 0)
        want_tiles = std::min<int64_t>(
            kSampleMaxTiles,
            std::max<int64_t>(1, ceil_div(ceil_div(kFastMinRank * M, (int64_t)kFastOversample * K), kMfmaTileItems)));
    p.stride = std::max<int64_t>(kSampleMinStride, ceil_div(full_tiles, want_tiles));
    p.sample_tiles = ceil_div(full_tiles, p.stride);
    p.n_sample = p.sample_tiles * kMfmaTileItems;
    p.sample = M >= kSampleMinM && p.n_sample >= 4 * (int64_t)K;
    p.r_fast = (int)std::min<int64_t>(K, std::max<int64_t>(1, ceil_div((int64_t)kFastOversample * K * p.n_sample, M)));
    p.fast = p.mfma && p.sample && p.r_fast < K;
    p.main = p.mfma ? chunk_mfma(B, ceil_div(M, kMfmaTileItems)) : chunk_stream(B, M);
    if (p.sample) p.pre = p.mfma ? chunk_mfma(B, p.sample_tiles) : chunk_stream(B, p.n_sample);
    p.pieces_per_chunk = p.mfma ? 4 : 1;
    p.n_pieces = (int64_t)B * p.main.P * p.pieces_per_chunk;
    p.key_stride = p.mfma ? ceil_div(M, kMfmaTileItems) * kMfmaTileItems : M;
    {
        // expected candidates per user: ~4K past the fast threshold, ~K M / n
        // past the K-th sampled score, every item without a sample
        const int64_t expect = p.fast ? (int64_t)kFastOversample * K
                                      : (p.sample ? ceil_div((int64_t)K * M, p.n_sample) : M);
        p.merge_small = (int64_t)p.main.P * p.pieces_per_chunk <= kMergeSmallPieces && expect <= kMergeSmallGather;
    }
    size_t o = 0;
    p.off_hdr = o;
    o += 256;
    p.off_theta = o;
    o = align_up(o + sizeof(float) * (size_t)B, 256);
    p.off_theta_safe = o;
    o = align_up(o + sizeof(float) * (size_t)B, 256);
    p.off_uflag = o;
    o = align_up(o + sizeof(int) * (size_t)B, 256);
    p.off_tflag = o;
    o = align_up(o + sizeof(int) * (size_t)ceil_div(B, kMfmaTileUsers), 256);
    p.off_sample = o;
    if (p.sample) o = align_up(o + sizeof(float) * (size_t)B * (size_t)p.n_sample, 256);
    p.off_pm = o;
    o = align_up(o + sizeof(float) * (size_t)p.n_pieces, 256);
    p.off_pl = o;
    o = align_up(o + sizeof(float) * (size_t)p.n_pieces, 256);
    p.off_pcnt = o;
    o = align_up(o + sizeof(int) * (size_t)p.n_pieces, 256);
    p.off_preg = o;
    o = align_up(o + sizeof(int64_t) * (size_t)p.n_pieces, 256);
    p.off_keys = o;
    o = align_up(o + sizeof(uint64_t) * (size_t)B * (size_t)p.key_stride, 256);
    p.total = o;
    return p;
}

struct CandPlan {
    int64_t n_pieces_max = 0;
    // Hot head (bf16, B >= 64): catalog items listed at least c times over all
    // lists (in sampled counts; c >= c_min, raised until at most t_max items
    // qualify) are scored
    // densely for every user on the MFMA path into s_hot[B][t_max]; the list
    // pass looks their scores up and gathers only the other rows.
    bool hot = false;
    int t_max = 0, c_min = 0;
    int64_t n_hblk = 0;  // blocks of kHotBlock catalog ids
    Chunking hot_chunks;
    size_t off_hdr = 0, off_begin = 0, off_table = 0, off_pm = 0, off_pl = 0, off_pcnt = 0,
           off_preg = 0, off_keys = 0, off_cnt = 0, off_hot_idx = 0, off_hist = 0, off_meta = 0, off_hblk = 0,
           off_hot_ids = 0, off_ehot = 0, off_shot = 0, total = 0;
};

constexpr int kHotMinUsers = 64;             // fewer users: no item can reach the break-even count
constexpr int kHotMaxRows = 16384;           // hot rows at most
constexpr int64_t kHotMaxEBytes = 256ll << 20;  // ... and at most this much gathered catalog
constexpr int64_t kHotMaxSBytes = 1ll << 30;    // ... and this much of dense scores
constexpr int kHotBins = 4096;               // histogram of per-item list counts
constexpr int kHotBlock = 4096;              // catalog ids per block of the hot compaction
constexpr int kHotSample = 16;               // list counts are estimated from every 16th entry

// Header of every workspace: int64 bad-id count, int64 bad-offset count,
// int32 piece count (candidate calls); int64 rescued-user count (dense calls).
constexpr size_t kHdrErrIds = 0, kHdrErrOffsets = 8, kHdrPieces = 16, kHdrRescued = 24;

inline CandPlan plan_cand(int B, int D, int64_t M, int64_t nnz, int dtype) {
    CandPlan p;
    p.n_pieces_max = nnz / kCandPiece + B;
    if (dtype == 0 && B >= kHotMinUsers && nnz > 0) {
        const int64_t bpad = ceil_div(B, kMfmaTileUsers) * kMfmaTileUsers;
        int64_t t = std::min<int64_t>(kHotMaxRows, ceil_div(M, kMfmaTileItems) * kMfmaTileItems);
        t = std::min<int64_t>(t, kHotMaxEBytes / (2 * (int64_t)D));
        t = std::min<int64_t>(t, kHotMaxSBytes / (4 * (int64_t)B));
        t = t / kMfmaTileItems * kMfmaTileItems;
        if (t >= kMfmaTileItems) {
            p.hot = true;
            p.t_max = (int)t;
            // break-even: scoring a row densely for B_pad users on the matrix
            // cores costs about as much as gathering it ~B_pad / 128 times;
            // in sampled counts (every kHotSample-th entry) that is / 16
            p.c_min = (int)std::max<int64_t>(2, ceil_div(std::max<int64_t>(4, bpad / 128), kHotSample));
            p.n_hblk = ceil_div(M, kHotBlock);
            p.hot_chunks = chunk_mfma(B, t / kMfmaTileItems);
        }
    }
    size_t o = 0;
    p.off_hdr = o;
    o += 256;
    p.off_begin = o;
    o = align_up(o + sizeof(int) * ((size_t)B + 1), 256);
    p.off_table = o;
    o = align_up(o + 16 * (size_t)p.n_pieces_max, 256);
    p.off_pm = o;
    o = align_up(o + sizeof(float) * (size_t)p.n_pieces_max, 256);
    p.off_pl = o;
    o = align_up(o + sizeof(float) * (size_t)p.n_pieces_max, 256);
    p.off_pcnt = o;
    o = align_up(o + sizeof(int) * (size_t)p.n_pieces_max, 256);
    p.off_preg = o;
    o = align_up(o + sizeof(int64_t) * (size_t)p.n_pieces_max, 256);
    p.off_keys = o;
    o = align_up(o + sizeof(uint64_t) * (size_t)std::max<int64_t>(nnz, 1), 256);
    if (p.hot) {
        p.off_cnt = o;
        o = align_up(o + sizeof(int) * (size_t)M, 256);
        p.off_hot_idx = o;
        o = align_up(o + sizeof(int) * (size_t)M, 256);
        p.off_hist = o;
        o = align_up(o + sizeof(int) * (size_t)kHotBins, 256);
        p.off_meta = o;
        o = align_up(o + 256, 256);
        p.off_hblk = o;
        o = align_up(o + sizeof(int) * (size_t)p.n_hblk, 256);
        p.off_hot_ids = o;
        o = align_up(o + sizeof(int) * (size_t)p.t_max, 256);
        p.off_ehot = o;
        o = align_up(o + 2 * (size_t)p.t_max * (size_t)D, 256);
        p.off_shot = o;
        o = align_up(o + sizeof(float) * (size_t)B * (size_t)p.t_max, 256);
    }
    p.total = o;
    return p;
}

// Batched top-K of dense rows: rows longer than one block handles well are
// split into chunks whose top-K keys a second pass merges; the chunk count is
// kept so that the merged keys (chunks x K) fit the merge's LDS gather.
constexpr int64_t kTopkChunkMin = 4096;
constexpr int64_t kTopkGather = 6144;  // the merge kernel's LDS gather capacity (keys)

// Register-resident selection: a block holds a row segment of kTopkSeg
// scores and keeps its top K; a second block per row merges the segments'
// keys (at most kTopkMergeKeys).  Measured on MI355X it beats the histogram
// narrowing on long rows with many segments (64 rows x 262,144, K 512: 0.18
// against 0.22 ms) but not on one segment per row (256 x 16,384, K 128: 65
// against 42 us), so it is used only with at least kTopkRegMinBlocks segment
// blocks; other shapes take the histogram-narrowing kernels.
constexpr int64_t kTopkSeg = 16384;
constexpr int64_t kTopkMergeKeys = 8192;
constexpr int64_t kTopkRegMinBlocks = 2 * kNumCU;

struct TopkPlan {
    bool reg = false;  // register-resident selection (else histogram narrowing)
    int64_t C = 0;     // columns per chunk (segment)
    int nchunk = 1;
    size_t workspace = 0;
};

inline TopkPlan plan_topk(int R, int64_t N, int K) {
    TopkPlan p;
    const int64_t nseg = ceil_div(N, kTopkSeg);
    if (nseg > 1 && nseg * K <= kTopkMergeKeys && (int64_t)R * nseg >= kTopkRegMinBlocks) {
        p.reg = true;
        p.C = kTopkSeg;
        p.nchunk = (int)nseg;
        p.workspace = sizeof(uint64_t) * (size_t)R * (size_t)nseg * (size_t)K;
        return p;
    }
    const int64_t max_chunks = std::max<int64_t>(1, kTopkGather / std::max(1, K));
    int64_t C = std::max(kTopkChunkMin, ceil_div(N, max_chunks));
    C = ceil_div(C, 4096) * 4096;
    p.C = C;
    p.nchunk = (int)ceil_div(N, C);
    if (p.nchunk > 1) p.workspace = sizeof(uint64_t) * (size_t)R * (size_t)p.nchunk * (size_t)K;
    return p;
}

// ---------------------------------------------------------------------------
// Cross-entropy over the catalog (bf16 only)
// ---------------------------------------------------------------------------
constexpr int64_t kCeChunk = 65536;  // catalog rows per backward chunk at most (G held for one chunk)
// The k-blocked operands of the dH product are addressed through buffer
// resources (32-bit record counts and offsets): each stays under 1 GiB, which
// shrinks the chunk for D or B beyond 8,192, and bounds both by 2^21.
constexpr int64_t kCeBlockedMaxBytes = (int64_t)1 << 30;
constexpr int kCeMaxSplits = 8;      // reduction splits of the dH product (powers of two)

struct CePlan {
    bool ok = true;  // false: a blocked operand cannot fit 256 catalog rows (B or D > 2^21)
    Chunking main;  // forward logsumexp pass over the catalog
    int64_t n_pieces = 0;
    int64_t Bp = 0;        // users padded to 32 (reduction of the dE product)
    int64_t chunk = 0;     // catalog rows per backward chunk
    int64_t Mcp = 0;       // chunk rounded up to 256 (reduction of the dH product)
    int64_t n_chunks = 0;
    int splits = 1;
    size_t off_hdr = 0, off_w = 0, off_pm = 0, off_pl = 0, off_pcnt = 0, off_preg = 0, fwd_total = 0;
    size_t off_ht = 0, off_et = 0, off_grows = 0, off_gcols = 0, off_dhp = 0, bwd_total = 0;
};

inline CePlan plan_ce(int B, int D, int64_t M) {
    CePlan p;
    p.main = chunk_mfma(B, ceil_div(M, kMfmaTileItems));
    p.n_pieces = (int64_t)B * p.main.P * 4;
    p.Bp = ceil_div(B, 32) * 32;
    const int64_t wide = std::max<int64_t>(D, p.Bp);  // rows of the wider blocked operand
    const int64_t cap = kCeBlockedMaxBytes / 2 / wide / kMfmaTileItems * kMfmaTileItems;
    if (cap < kMfmaTileItems) p.ok = false;
    p.chunk = std::max<int64_t>(1, std::min<int64_t>({M, kCeChunk, cap}));
    p.Mcp = ceil_div(p.chunk, kMfmaTileItems) * kMfmaTileItems;
    p.n_chunks = ceil_div(M, p.chunk);
    const int64_t tiles = ceil_div(B, kMfmaTileUsers) * ceil_div(D, kMfmaTileItems);
    // two rounds of blocks measured faster than one round of twice the work
    while (p.splits < kCeMaxSplits && tiles * p.splits < 2 * kNumCU) p.splits *= 2;
    size_t o = 0;
    p.off_hdr = o;
    o += 256;
    p.off_w = o;
    o = align_up(o + sizeof(float) * (size_t)B, 256);
    const size_t common = o;
    p.off_pm = o;
    o = align_up(o + sizeof(float) * (size_t)p.n_pieces, 256);
    p.off_pl = o;
    o = align_up(o + sizeof(float) * (size_t)p.n_pieces, 256);
    p.off_pcnt = o;
    o = align_up(o + sizeof(int) * (size_t)p.n_pieces, 256);
    p.off_preg = o;
    o = align_up(o + sizeof(int64_t) * (size_t)p.n_pieces, 256);
    p.fwd_total = o;
    o = common;
    p.off_ht = o;
    o = align_up(o + 2 * (size_t)D * (size_t)p.Bp, 256);
    p.off_et = o;
    o = align_up(o + 2 * (size_t)D * (size_t)p.Mcp, 256);
    p.off_grows = o;  // k-blocked, Bp rows per block of 32 catalog rows
    o = align_up(o + 2 * (size_t)p.Bp * (size_t)p.Mcp, 256);
    p.off_gcols = o;
    o = align_up(o + 2 * (size_t)p.Mcp * (size_t)p.Bp, 256);
    p.off_dhp = o;
    o = align_up(o + sizeof(float) * (size_t)p.splits * (size_t)B * (size_t)D, 256);
    p.bwd_total = o;
    return p;
}

}  // namespace genrec
