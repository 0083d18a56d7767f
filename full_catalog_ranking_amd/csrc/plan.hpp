// Host-side planning for the ranking head: variant choice, work split and
// workspace layout.  Pure C++ (no HIP), so it can be unit-tested on any host.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <algorithm>
#include <cmath>

namespace genrec {

constexpr int kNumCU = 256;            // MI355X compute units
constexpr int kMfmaTileItems = 256;    // items per MFMA tile
constexpr int kMfmaTileUsers = 256;    // users per MFMA tile
constexpr int kMfmaBlockK = 32;        // reduction elements per k-step (and per k-block of a blocked operand)
constexpr int kStreamMaxB = 1;         // bf16 batches up to this size use the VALU path (a half-empty MFMA tile still beats re-reading E per user)
constexpr int64_t kSampleMinM = 65536; // smaller catalogs skip the threshold pre-pass
constexpr int64_t kSampleMinStride = 32; // sample one catalog tile of every G, G >= 32
constexpr int64_t kSampleMaxTiles = 128; // sampled items per user at most 128 * 256
constexpr int64_t kSampleMaxItems = 32768;  // = kSampleMaxTiles * 256: one user's sample fits the threshold kernel
constexpr int kFastOversample = 4;     // fast threshold: expected candidates ~ 4 K
constexpr int kSampleMaxSplits = 16;   // reduction splits of an MFMA sample pass that fills few CUs
constexpr int64_t kSampleMinSteps = 8; // k-steps each of those splits keeps at least
// MFMA path: the sample only has to place the fast threshold at rank >= 32 of
// the sampled scores.  The number of catalog items above the r-th largest of
// n sampled scores is about M r / n with a Gamma(r)-shaped spread, so at
// r = 32 and 4 K expected the chance of fewer than K (a rescue) is ~1e-9 per
// user.  A larger sample buys nothing there and costs a pass over more tiles.
constexpr int64_t kFastMinRank = 32;
constexpr int64_t kStreamPieces = 2048;  // target work pieces of the VALU path
constexpr int64_t kStreamChunkAlign = 32;
constexpr int kCandPiece = 256;        // candidate entries per piece (matches the kernels)
// Fused small-catalog path: on the VALU path without a sample, catalogs of up
// to this many items run as one launch (the last block of each user selects
// its top-K from the user's dense score row held in registers, 32 keys per
// thread of a 256-thread block; 64 would spill).
constexpr int64_t kFusedMaxM = 256 * 32;

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Workspace layouts: regions at 256-byte-aligned offsets, sizes checked so
// that a huge shape makes the plan unsupported instead of wrapping a size_t
// around to a small workspace.
constexpr uint64_t kMaxWorkspace = (uint64_t)1 << 56;
constexpr int64_t kMaxGrid = 2147483647;  // blocks per launch dimension

struct Layout {
    size_t o = 0;
    bool ok = true;
    // Reserves count elements of elem bytes; returns the region's offset.
    size_t take(uint64_t elem, uint64_t count) {
        const size_t at = o;
        uint64_t bytes = 0;
        if (__builtin_mul_overflow(elem, count, &bytes) || bytes > kMaxWorkspace || o > kMaxWorkspace - bytes) {
            ok = false;
            o = kMaxWorkspace;
            return at;
        }
        o = align_up(o + bytes, 256);
        return at;
    }
};

struct Chunking {
    int UT = 1, P = 1, base = 0, rem = 0;  // MFMA: P chunks of base(+1) tiles over UT user tiles
    int64_t CH = 0;                        // VALU: items per chunk (P chunks)
};

// Bounded candidate regions.  With a sampled threshold the main pass keeps,
// per piece (user, chunk, lane group), at most `cap` keys -- kCapFactor times
// the count the threshold is expected to let through there, at least
// kCapMin -- and sends a full piece's further keys to the user's overflow
// region.  A user whose overflow region fills too (or who was left short of
// K) is finished exactly by the rescue: its row is gathered with the other
// rescued users', and counting passes over the gathered rows narrow a
// 4,096-bin histogram of its ranking keys (12 bits a pass, kNarrowPasses
// passes cover 64-bit keys) until the keys at or above the bound fit its
// collect region of `ccol` keys, which one more pass fills.  Regions of every
// item (8 bytes per user and item) are kept while they take at most the key
// budget: they need no rescue for overflow.
constexpr size_t kDefaultKeyBudget = (size_t)256 << 20;
constexpr int kCapFactor = 8;
constexpr int kCapMin = 64;
constexpr int kNarrowPasses = 6;
constexpr int kNarrowBinsPlan = 4096;  // = the kernels' kNarrowBins
constexpr int kCollectSlack = 1024;    // collect region: kCapFactor K + this many keys
// Keys past a full piece go to the user's overflow region (an atomic slot):
// max(kOvfMin, 2 ccol) keys per user.  A user is rescued only when that fills
// too (a catalog stored in clusters concentrates a user's candidates in a
// few pieces; exchangeable catalogs never reach it).
constexpr int kOvfMin = 16384;

// The merge's smaller build (LDS gather of 2,048 keys, 512-piece batches)
// serves users expected to hold at most that many candidates and pieces.
constexpr int kMergeSmallGather = 2048;
constexpr int kMergeSmallPieces = 512;

struct DensePlan {
    bool ok = true;  // false: the workspace or a grid would be too large (unsupported)
    bool mfma = false;
    bool sample = false;
    int64_t stride = 1;        // G: the sample holds one full catalog tile of every G (mf_sample_tile)
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
    bool fused = false;        // one launch: dense rows [B][M] f32 and per-user arrival words
    // MFMA sample pass: its reduction split over `sample_splits` grid rows when
    // it would otherwise fill few CUs (one sampled tile per block is one tile's
    // latency); the sampled scores are then sums of partials, not bit-identical
    // to the main pass, so the K-th sampled score is no safe threshold: the
    // rescue pass then keeps every score of a flagged user
    int sample_splits = 1;
    bool safe_exact = true;
    bool bounded = false;      // candidate regions of `cap` keys per piece (else of every item)
    int cap = 0;
    int ccol = 0;              // bounded: keys of a flagged user's collect region
    int ovf_cap = 0;           // bounded: keys of a user's overflow region
    int64_t rec_stride = 0;    // piece records per user: 4 P (+ 1: the overflow region's, bounded)
    size_t off_hdr = 0, off_theta = 0, off_theta_safe = 0, off_uflag = 0, off_tflag = 0, off_sample = 0,
           off_pm = 0, off_pl = 0, off_pcnt = 0, off_preg = 0, off_keys = 0, off_arrive = 0, off_elect = 0, off_rows = 0,
           off_nst = 0, off_hist = 0, off_coll = 0, off_ccnt = 0, off_cbase = 0, off_rc = 0, off_hgat = 0, off_map = 0, total = 0;
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

// dtype: 0 = bf16, 1 = f32.  Matrix cores for bf16 batches of two users or
// more, and for fp32 ones as well unless the catalog is small enough for the
// one-launch VALU path (fp32 MFMA: 16 times fewer flops per cycle than bf16,
// still twice the non-packed VALU rate, and E read once rather than per user).
// ovf_keys: keys of each user's overflow region (bounded regions), -1: the
// default max(kOvfMin, 2 ccol); 0: none (a full piece sends its user to the
// rescue).
inline DensePlan plan_dense(int B, int D, int64_t M, int K, int dtype, size_t key_budget = kDefaultKeyBudget,
                            int64_t ovf_keys = -1) {
    DensePlan p;
    p.mfma = B > kStreamMaxB && (dtype == 0 || M > kFusedMaxM);
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
    if (p.mfma && p.sample) {
        const int64_t ke = dtype == 0 ? kMfmaBlockK : kMfmaBlockK / 2;  // reduction elements per k-step
        const int64_t blocks = (int64_t)p.pre.UT * p.pre.P;
        // a split writes (and the threshold pass reads back) a full partial
        // score row per sampled item: splits too short to pay for that traffic
        // are not made (the 256-user bf16 batch at D = 2,048: 8 splits of 8
        // k-steps beat 16 of 4 by 4 us; its fp32 twin keeps 16 of 8)
        while (p.sample_splits < kSampleMaxSplits && blocks * p.sample_splits * 2 <= kNumCU &&
               D % (ke * p.sample_splits * 2) == 0 && D / (ke * p.sample_splits * 2) >= kSampleMinSteps)
            p.sample_splits *= 2;
        p.safe_exact = p.sample_splits == 1;
    }
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
    p.fused = !p.mfma && !p.sample && M <= kFusedMaxM;
    if (p.mfma && p.fast && K > 0) {
        // full regions cost 8 bytes per (user, item); past the budget, pieces
        // of cap keys sized from the expected count (about 4 K per user over
        // 4 P pieces)
        const uint64_t full = 8ull * (uint64_t)B * (uint64_t)p.key_stride;
        const int64_t per_piece = ceil_div((int64_t)kFastOversample * K, (int64_t)p.main.P * 4);
        const int64_t piece_max = (int64_t)64 * (p.main.base + (p.main.rem > 0 ? 1 : 0));  // items of a piece
        int64_t cap = std::max<int64_t>(kCapMin, ceil_div(kCapFactor * per_piece, 16) * 16);
        cap = std::min<int64_t>(cap, piece_max);
        if (full > (uint64_t)key_budget && cap < piece_max) {
            p.bounded = true;
            p.cap = (int)cap;
            p.ccol = (int)(ceil_div((int64_t)kCapFactor * K + kCollectSlack, 256) * 256);
            p.ovf_cap = ovf_keys < 0 ? std::max(kOvfMin, 2 * p.ccol) : (int)std::min<int64_t>(ovf_keys, 1 << 30);
        }
    }
    p.rec_stride = (int64_t)p.main.P * p.pieces_per_chunk + (p.bounded ? 1 : 0);
    const int64_t n_rec = (int64_t)B * p.rec_stride;
    // launch grids: MFMA passes UT x P blocks, VALU passes B x P, merge B
    const int64_t grid = p.mfma ? (int64_t)p.main.UT * p.main.P : p.n_pieces;
    const int64_t pre_grid = p.sample ? (p.mfma ? (int64_t)p.pre.UT * p.pre.P : (int64_t)B * p.pre.P) : 0;
    p.ok = grid <= kMaxGrid && pre_grid <= kMaxGrid;
    Layout L;
    p.off_hdr = L.take(1, 256);
    if (p.fused) {
        p.off_arrive = L.take(sizeof(uint64_t), (uint64_t)p.n_pieces);  // a flag per block: B x P
        p.off_elect = L.take(sizeof(uint64_t), (uint64_t)B);
        p.off_pm = L.take(sizeof(float), (uint64_t)p.n_pieces);
        p.off_pl = L.take(sizeof(float), (uint64_t)p.n_pieces);
        p.off_rows = L.take(sizeof(float), (uint64_t)B * (uint64_t)M);
    } else {
        p.off_theta = L.take(sizeof(float), (uint64_t)B);
        p.off_theta_safe = L.take(sizeof(float), (uint64_t)B);
        p.off_uflag = L.take(sizeof(int), (uint64_t)B);
        p.off_tflag = L.take(sizeof(int), (uint64_t)ceil_div(B, kMfmaTileUsers));
        p.off_sample = L.take(sizeof(float), p.sample ? (uint64_t)p.sample_splits * B * (uint64_t)p.n_sample : 0);
        p.off_pm = L.take(sizeof(float), (uint64_t)n_rec);
        p.off_pl = L.take(sizeof(float), (uint64_t)n_rec);
        p.off_pcnt = L.take(sizeof(int), (uint64_t)n_rec);
        p.off_preg = L.take(sizeof(int64_t), (uint64_t)n_rec);
        if (p.bounded) {
            // the pieces' regions, then each user's overflow region
            p.off_keys = L.take(sizeof(uint64_t),
                                (uint64_t)p.n_pieces * (uint64_t)p.cap + (uint64_t)B * (uint64_t)p.ovf_cap);
            p.off_nst = L.take(32, (uint64_t)B);
            p.off_hist = L.take(sizeof(uint32_t) * (uint64_t)kNarrowBinsPlan, (uint64_t)B);
            p.off_coll = L.take(sizeof(uint64_t) * (uint64_t)p.ccol, (uint64_t)B);
            p.off_ccnt = L.take(sizeof(int), (uint64_t)B);
            p.off_cbase = L.take(sizeof(int64_t), (uint64_t)B);
            p.off_rc = L.take(1, 256);                                                // the rescue's two counts
            p.off_hgat = L.take((uint64_t)(dtype == 0 ? 2 : 4) * (uint64_t)D, (uint64_t)B);  // flagged users' rows
            p.off_map = L.take(sizeof(int), (uint64_t)B);
        } else {
            p.off_keys = L.take(sizeof(uint64_t), (uint64_t)B * (uint64_t)p.key_stride);
        }
    }
    p.ok = p.ok && L.ok;
    p.total = p.ok ? L.o : 0;
    return p;
}

struct CandPlan {
    bool ok = true;  // false: the workspace or a grid would be too large (unsupported)
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
    // the list pass runs one block per piece; the piece table is int-indexed
    p.ok = p.n_pieces_max <= kMaxGrid && nnz <= ((int64_t)1 << 40);
    Layout L;
    p.off_hdr = L.take(1, 256);
    p.off_begin = L.take(sizeof(int), (uint64_t)B + 1);
    p.off_table = L.take(16, (uint64_t)p.n_pieces_max);
    p.off_pm = L.take(sizeof(float), (uint64_t)p.n_pieces_max);
    p.off_pl = L.take(sizeof(float), (uint64_t)p.n_pieces_max);
    p.off_pcnt = L.take(sizeof(int), (uint64_t)p.n_pieces_max);
    p.off_preg = L.take(sizeof(int64_t), (uint64_t)p.n_pieces_max);
    p.off_keys = L.take(sizeof(uint64_t), (uint64_t)std::max<int64_t>(nnz, 1));
    if (p.hot) {
        p.off_cnt = L.take(sizeof(int), (uint64_t)M);
        p.off_hot_idx = L.take(sizeof(int), (uint64_t)M);
        p.off_hist = L.take(sizeof(int), (uint64_t)kHotBins);
        p.off_meta = L.take(1, 256);
        p.off_hblk = L.take(sizeof(int), (uint64_t)p.n_hblk);
        p.off_hot_ids = L.take(sizeof(int), (uint64_t)p.t_max);
        p.off_ehot = L.take(2, (uint64_t)p.t_max * (uint64_t)D);
        p.off_shot = L.take(sizeof(float), (uint64_t)B * (uint64_t)p.t_max);
    }
    p.ok = p.ok && L.ok;
    p.total = p.ok ? L.o : 0;
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
// Rows of at most one segment with K <= kTopkRowMaxK: one block per row, the
// top K found among the keys at or above the K-th largest of the threads'
// maxima (K <= 256) or of 1,024 group maxima (K <= 512) -- a few times K keys
// for unordered scores -- no second pass.
constexpr int kTopkRowMaxK = 512;
constexpr int kTopkBoundMaxK = 512;  // the row kernel's bound from 1,024 group maxima serves K up to this

// Long rows (more than one segment), K <= kTopkBoundMaxK: the filter route
// (xGR explainer page, xBeam: candidates filtered before they are sorted).
// A first block per row reads a sample of the row -- 256 runs of 64 columns
// spread evenly over it, 64 samples a thread -- and takes as the row's bound
// T the sj-th largest of the 256 threads' sample maxima; blocks of
// kTopkFiltCols columns then keep every key at or above T in a list of
// kTopkFiltCap keys per row, and a block per row ranks the list.  For
// unordered scores a thread's maximum reaches the sj-th largest with
// probability sj / 256, so one score does with q = 1 - (1 - sj/256)^(1/64),
// and N q keys reach T; sj is the smallest rank >= kTopkFiltMinRank that
// makes this 3 K, and the route is taken when that is at most half the list.
// A row whose list holds fewer than K keys or overflows (a sample that
// misses the row's top, exact ties at T) is ranked from the whole row by the
// histogram narrowing instead: exact either way, only slower.
constexpr int kTopkFiltCap = 8192;
constexpr int kTopkFiltParts = 64;  // the list's parts, each with its own count (columns = s mod 64 in part s)
constexpr int64_t kTopkFiltCols = 4096;
constexpr int kTopkFiltMinRank = 16;

inline double topk_filt_expect(int64_t N, int sj) {
    return (double)N * (1.0 - std::pow(1.0 - sj / 256.0, 1.0 / 64.0));
}

// The bound's rank sj for a row of N > kTopkSeg scores and K <= kTopkBoundMaxK,
// or 0 when the route does not apply.
inline int topk_filt_rank(int64_t N, int K) {
    if (N <= kTopkSeg || K > kTopkBoundMaxK) return 0;
    for (int sj = kTopkFiltMinRank; sj < 256; ++sj) {
        const double e = topk_filt_expect(N, sj);
        if (e >= 3.0 * K) return e <= kTopkFiltCap / 2 ? sj : 0;
    }
    return 0;
}

struct TopkPlan {
    bool ok = true;    // false: the workspace or the grid would be too large (unsupported)
    bool reg = false;  // register-resident selection (else histogram narrowing)
    bool row = false;  // ... of a whole row per block (rows of at most kTopkSeg, K <= 256)
    int filt = 0;      // the filter route: the bound's rank sj (0: another route)
    int64_t C = 0;     // columns per chunk (segment; filter block)
    int nchunk = 1;
    size_t off_thr = 0, off_cnt = 0;  // filter route: per-row bound and list part counts (the lists at 0)
    size_t workspace = 0;
};

inline TopkPlan plan_topk(int R, int64_t N, int K) {
    TopkPlan p;
    const int64_t nseg = ceil_div(N, kTopkSeg);
    if (nseg == 1 && K <= kTopkRowMaxK) {
        p.reg = p.row = true;
        p.C = N;
        p.nchunk = 1;
    } else if ((p.filt = topk_filt_rank(N, K)) > 0) {
        p.C = kTopkFiltCols;
        p.nchunk = (int)ceil_div(N, kTopkFiltCols);
        Layout L;
        L.take(sizeof(uint64_t) * (uint64_t)kTopkFiltCap, (uint64_t)R);
        p.off_thr = L.take(sizeof(uint32_t), (uint64_t)R);
        p.off_cnt = L.take(sizeof(int) * (uint64_t)kTopkFiltParts, (uint64_t)R);
        p.ok = (int64_t)R * p.nchunk <= kMaxGrid && L.ok;
        p.workspace = p.ok ? L.o : 0;
        return p;
    } else if (nseg > 1 && nseg * K <= kTopkMergeKeys && (int64_t)R * nseg >= kTopkRegMinBlocks) {
        p.reg = true;
        p.C = kTopkSeg;
        p.nchunk = (int)nseg;
    } else {
        const int64_t max_chunks = std::max<int64_t>(1, kTopkGather / std::max(1, K));
        int64_t C = std::max(kTopkChunkMin, ceil_div(N, max_chunks));
        C = ceil_div(C, 4096) * 4096;
        p.C = C;
        p.nchunk = (int)ceil_div(N, C);
    }
    p.ok = (int64_t)R * p.nchunk <= kMaxGrid;  // one block per (row, chunk)
    if (p.nchunk > 1) {
        Layout L;
        L.take(sizeof(uint64_t) * (uint64_t)p.nchunk, (uint64_t)R * (uint64_t)K);
        p.ok = p.ok && L.ok;
        p.workspace = p.ok ? sizeof(uint64_t) * (size_t)R * (size_t)p.nchunk * (size_t)K : 0;
    }
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
    bool ok = true;  // backward: false when a blocked operand cannot fit 256 catalog rows (B or D > 2^21)
                     // or the workspace would be too large
    bool fwd_ok = true;  // forward: false when its workspace would be too large
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
    Layout L;
    p.off_hdr = L.take(1, 256);
    p.off_w = L.take(sizeof(float), (uint64_t)B);
    Layout F = L;  // forward: the logsumexp pieces after the common part
    p.off_pm = F.take(sizeof(float), (uint64_t)p.n_pieces);
    p.off_pl = F.take(sizeof(float), (uint64_t)p.n_pieces);
    p.off_pcnt = F.take(sizeof(int), (uint64_t)p.n_pieces);
    p.off_preg = F.take(sizeof(int64_t), (uint64_t)p.n_pieces);
    p.off_ht = L.take(2, (uint64_t)D * (uint64_t)p.Bp);
    p.off_et = L.take(2, (uint64_t)D * (uint64_t)p.Mcp);
    p.off_grows = L.take(2, (uint64_t)p.Bp * (uint64_t)p.Mcp);  // k-blocked, Bp rows per block of 32 catalog rows
    p.off_gcols = L.take(2, (uint64_t)p.Mcp * (uint64_t)p.Bp);
    p.off_dhp = L.take(sizeof(float), (uint64_t)p.splits * (uint64_t)B * (uint64_t)D);
    // the forward's MFMA grid (UT x P) and the merge's (B) are small; the
    // dH product's is ceil(B/256) x P x splits
    const bool grids = (int64_t)p.main.UT * p.main.P <= kMaxGrid;
    p.fwd_ok = F.ok && grids;
    p.ok = p.ok && L.ok && grids;
    p.fwd_total = p.fwd_ok ? F.o : 0;
    p.bwd_total = p.ok ? L.o : 0;
    return p;
}

// Longest chains of fp32 additions into one output of the backward's two
// products: a dH entry sums Mcp / splits products within a split, is added
// into its partial once per chunk, and the partials are summed at the end; a
// dE entry sums the Bp (padded) users' products.
inline int64_t ce_depth_h(const CePlan& p) { return p.Mcp / p.splits + p.n_chunks + p.splits; }
inline int64_t ce_depth_e(const CePlan& p) { return p.Bp; }

}  // namespace genrec
