// Kernel argument blocks and launchers (internal to libgenrec.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/genrec.h"

namespace genrec {

constexpr int CAND_PIECE = 256;  // candidate-list entries per work piece

// Rescue of a user over bounded candidate regions: the keys at or above lo
// are narrowed by counting passes until they fit the user's collect region.
struct NarrowState {
    uint64_t lo;  // lower bound (inclusive) of the 64-bit ranking keys still considered
    int shift;    // counting pass: key k falls in bin (k - lo) >> shift of kNarrowBins
    int k_rem;    // keys of the top K in [lo, range end); the other K - k_rem lie above the range
    int status;   // 0: not flagged; 1: counting; 2: resolved (collect the keys >= lo)
    int pad;
};
constexpr int kNarrowBins = 4096;  // 12 bits of the key per counting pass
constexpr int kNarrowBits = 12;

struct MfmaArgs {
    const uint16_t* H;  // bf16 elements, or fp32 ones when f32 (modes 0 and 1)
    const uint16_t* E;
    int f32;
    int B, D;
    int64_t M;
    int n_tiles, tile_stride; // pass-tile t = catalog tile mf_sample_tile(t, G, M / 256), G = tile_stride
    int UT, P, base, rem;     // user tiles; P chunks of base(+1) pass-tiles
    float* sample_out;        // mode 0: [B][n_tiles * 256] scores (split z of grid y at + z * sample_split)
    int64_t sample_split;
    const float* theta;       // mode 1: [B] candidate thresholds (or null)
    uint64_t* keys;           // mode 1: candidate regions, [B][key_stride]
    int64_t key_stride;       // mode 1: >= 256 * ceil(M / 256)
    float* pm;                // per piece (user b, chunk c, lane group g) at (b*P + c)*4 + g
    float* pl;
    int* pcnt;
    int64_t* preg;
    // rescue pass (mode 1): only user tiles with tile_flag[ut] != 0 run, and
    // only users with user_flag[u] != 0 append candidates and write records
    const int* tile_flag;
    const int* user_flag;
    // mode 0: when set, only the first *live_rows catalog rows matter; chunks
    // that start past them exit at once
    const int* live_rows;
    // item mask (null: every item): item i takes part for user u only when bit
    // i % 32 of mask[u * mask_stride + i / 32] is set (stride 0: one mask)
    const uint32_t* mask;
    int64_t mask_stride;
    // Row stride, in elements, of both operands (0: D).  D is the reduction
    // length of this launch; grid y > 1 splits it: split z reads the operands
    // from element z * k_split of each row (D = k_split).
    int64_t ld;
    int64_t k_split;
    // mode 1: no candidate is kept at all (logsumexp pieces only)
    int no_cand;
    // mode 1: keys per candidate region when the regions are bounded (piece p
    // at keys + p * cap, p = (u P + c) 4 + g); a full piece's further keys go
    // to the user's overflow region at keys + ovf_base + u * ovf_cap, slot =
    // atomicAdd on the overflow record's count (record u * rec_stride + 4 P),
    // and its own count stops at cap; 0: region of every item (user u at
    // keys + u * key_stride)
    int cap;
    int ovf_cap;
    int64_t ovf_base;
    int64_t rec_stride;  // piece records per user (0: 4 P)
    // mode 6 -- exact rescue of flagged users over bounded regions, on their
    // gathered rows (H row r is user u = map[r]): only users whose
    // nst[u].status is 1 (counting, collect == 0) or 2 (collect == 1) take
    // part; every finite score's key k >= nst[u].lo is counted into
    // hist[u * kNarrowBins + ((k - lo) >> shift)] (keys past the last bin
    // skipped), or stored at coll[u * ccol + slot], slot = atomicAdd(&ccnt[u],
    // 1) (< ccol kept)
    NarrowState* nst;
    uint32_t* hist;
    uint64_t* coll;
    int* ccnt;
    int ccol;
    int collect;
    // mode 6: rc[0] = users still counting (0: the counting passes exit at
    // once), rc[1] = flagged users, whose rows the merge gathered into H (row
    // r is user map[r]; tiles past rc[1] exit at once)
    const int* rc;
    const int* map;
    // mode 3 -- softmax-minus-target tiles of the cross-entropy gradient:
    // rows are catalog items item0 + j (j < M valid), columns users;
    // g = w[u] (exp(s - lse[u]) - [item0 + j == labels[u]]) goes to
    // g_rows[u * ld_g + j] and g_cols[j * ld_gt + u] as bf16, with zeros in
    // invalid rows (j < n_tiles * 256) and in columns B .. gt_users - 1;
    // g_rows is k-blocked: G[u][j] at (j / 32) * ld_g + u * 32 + j % 32.
    const float* lse;
    const float* wgt;
    const int32_t* labels;
    int64_t item0;
    uint16_t* g_rows;
    uint16_t* g_cols;
    int64_t ld_g, ld_gt;
    int gt_users;
    // mode 4 -- plain product C[row][col] = sum_k A[row][k] B[col][k] (rows
    // from the E-side operand, M valid; columns from the H-side operand, B
    // valid) stored fp32 at c_out[row * ldc + col], or [col * ldc + row] when
    // c_trans, added to what is there when c_accum; split z writes from
    // c_out + z * c_split.
    float* c_out;
    int64_t ldc, c_split;
    int c_trans, c_accum;
    int c_bf16;  // stores bf16 (round to nearest even) at ((uint16_t*)c_out)[same index]; no c_accum
    // mode 5 -- mode 4 over k-blocked operands: element (r, k) of an operand
    // at (k / 32) * blk + r * 32 + k % 32 (blk_e / blk_h elements per block of
    // 32 reduction steps); e_elems / h_elems = the operands' sizes in elements
    // (reads past them give zeros; rows past the valid ones read neighbouring
    // data, which only reaches outputs that are not stored)
    int64_t blk_e, blk_h, e_elems, h_elems;
};

// Cross-entropy bookkeeping kernels.
struct CeArgs {
    const uint16_t* H;
    const uint16_t* E;
    int B, D;
    int64_t M;
    const int32_t* labels;
    const float* weights;  // null: 1
    float* w_eff;          // [B] weight, 0 for a label outside [0, M)
    int64_t* err;          // [0] += labels outside [0, M)
    const float* pm;       // forward: P pieces per user (logsumexp partials)
    const float* pl;
    int P;
    float* out_loss;
    float* out_lse;
};

struct TransposeArgs {
    const uint16_t* in;  // [R][ld_in]
    int64_t R, C, ld_in;
    uint16_t* out;       // [C][ld_out]: out[c][r] = in[r][c], zero for R <= r < ld_out
    int64_t ld_out;
    // blocked != 0: out[c][r] at (r / 32) * C * 32 + c * 32 + r % 32 instead
    int blocked;
};

struct CandPiece {
    int user;
    int len;
    int64_t e0;
};

struct StreamArgs {
    const void* H;
    const void* E;
    int B, D;
    int64_t M;
    int64_t n_items;          // dense modes: pass items j < n_items
    int tile_stride;          // dense modes: item j is catalog row 256 mf_sample_tile(j/256, G, M/256) + j%256
    int64_t CH;               // dense modes: items per chunk
    int P;                    // dense modes: chunks per user
    const int32_t* ids;       // candidate mode
    const int* n_pieces;
    const CandPiece* table;
    float* sample_out;
    const float* theta;
    uint64_t* keys;
    float* pm;
    float* pl;
    int* pcnt;
    int64_t* preg;
    int64_t* err;
    // candidate mode, hot head: hot_idx[id] >= 0 gives the entry's score as
    // s_hot[user * t_hot + hot_idx[id]] (no gather); null = every row gathered
    const int* hot_idx;
    const float* s_hot;
    int t_hot;
    // dense modes: item mask as in MfmaArgs (null: every item)
    const uint32_t* mask;
    int64_t mask_stride;
    // fused mode (one launch, rows of at most 8,192 items): dense score rows
    // [B][n_items], per-block arrival flags [B][P] (block of user b, chunk c
    // at b * P + c), per-user election words [B], this call's ticket (40 bits,
    // not 0 or all ones), K and the outputs; err = the workspace header (error
    // words and rescued count cleared by the call)
    float* rows;
    uint64_t* arrive;
    uint64_t* elect;
    uint64_t ticket;
    int K;
    int32_t* out_idx;
    float* out_scores;
    float* out_lse;
};

// Hot head of the candidate lists: per-item list counts, the count threshold,
// the deterministic compaction of hot ids and the gathered hot catalog rows.
struct HotArgs {
    const int32_t* ids;
    int64_t nnz;
    const uint16_t* E;
    int64_t M;
    int D;
    int c_min, t_max;  // c_min: minimum sampled count of a hot row
    int64_t n_hblk;
    int* cnt;        // [M] sampled list counts
    int* hot_idx;    // [M]
    int* hist;       // [4096]
    int* meta;       // [0] = c, [1] = number of hot rows
    int* hblk;       // [n_hblk] per-block counts, then their exclusive scan
    int* hot_ids;    // [t_max]
    uint16_t* e_hot; // [t_max][D]
};

struct MergeArgs {
    int B, K;
    int P;                   // dense: pieces of user b are [b*P, (b+1)*P)
    const int* piece_begin;  // candidates: [B+1]
    const uint64_t* keys;
    const float* pm;
    const float* pl;
    const int* pcnt;
    const int64_t* preg;
    int32_t* out_idx;
    float* out_scores;
    float* out_lse;
    int64_t* clear_err;  // zeroed by block 0 when non-null
    // mode 0: every user; 1: a user with fewer than K candidates is flagged
    // (user_flag, tile_flag of its 256-user tile, rescued count) and skipped;
    // 2: only flagged users
    int mode;
    int* user_flag;
    int* tile_flag;
    int64_t* rescued;
    // mode 1: a user is flagged only when the rescue threshold is lower than
    // the fast one (else the first pass already kept every item it would);
    // when the sampled scores were summed from reduction splits (safe_exact 0)
    // the sampled thresholds are estimates and any user short of K is flagged
    const float* theta_fast;
    const float* theta_safe;
    int safe_exact;
    // 1: the smaller merge build (users with at most ~512 pieces and ~2,048
    // candidates expected); any value gives the same result
    int small;
    // Bounded regions (cap > 0): each user's last piece record is its
    // overflow region's.  Mode 1 flags a user whose overflow region counted
    // more than ovf_cap keys as well, writes its lse, and starts its rescue
    // state (nst, a zeroed hist row, ccnt = 0, cbase = u * ccol, its row
    // gathered); mode 3 ranks flagged users from their collect region (coll +
    // cbase[u], min(ccnt[u], ccol) keys), lse left as mode 1 wrote it.
    int cap;
    NarrowState* nst;
    uint32_t* hist;
    const uint64_t* coll;
    int* ccnt;
    int64_t* cbase;
    int ccol;
    // rc[0]: users still counting (mode 1 adds them); rc[1]: flagged users,
    // each one's H row (D elements of es bytes) copied to hgat row rc[1]++ and
    // map[that row] = the user
    int* rc;
    int* map;
    const void* H;
    void* hgat;
    int D, es;
    int ovf_cap;    // the last record of each user is its overflow region's: full past this count
};

// One block per user: picks the bin of the counted histogram that holds the
// user's K-th key and narrows the state to it (or resolves it).
struct NarrowArgs {
    NarrowState* nst;
    uint32_t* hist;
    int* rc;        // rc[0]: users still counting; a resolved user leaves it
    int B, K, ccol;
};

struct ThresholdArgs {
    const float* sample;  // [B][n_sample] sampled scores: the sum of n_split partial rows split_stride apart
    int64_t n_sample;     // <= 32768, a multiple of 4
    int n_split;
    int64_t split_stride;
    int B, K, r_fast;
    float* theta_safe;    // [B] lower bound of the K-th largest sampled score
    float* theta_fast;    // [B] lower bound of the r_fast-th largest (may be null)
    int* user_flag;       // [B] cleared (may be null)
    int* tile_flag;       // [ceil(B/256)] cleared (may be null)
    int* rc;              // [2] cleared by block 0 (may be null): the bounded rescue's counts
    int64_t* rescued;     // cleared by block 0 (may be null)
    // bounded candidate regions (ovf_pm non-null): user b's overflow record,
    // at b * rec_stride + rec_off, starts empty (max -inf, sum 0, count 0)
    // and points at keys + ovf_base + b * ovf_cap
    float* ovf_pm;
    float* ovf_pl;
    int* ovf_pcnt;
    int64_t* ovf_preg;
    int64_t rec_stride, rec_off, ovf_base;
    int ovf_cap;
};

struct CandPlanArgs {
    const int64_t* offsets;
    int B;
    int64_t nnz;
    int* piece_begin;
    CandPiece* table;
    int* n_pieces;
    int64_t* err;
};

struct TopkRowsArgs {
    const float* scores;  // [R][ld], the first N of each row used
    int R;
    int64_t N, ld;
    int K;
    int32_t* out_idx;     // [R][K]
    float* out_scores;    // [R][K]
    int64_t C;            // columns per chunk
    int nchunk;           // chunks per row (1: no merge pass)
    uint64_t* part;       // nchunk > 1: [R][nchunk][K] chunk results
    int reg;              // 1: register-resident selection, chunks of kTopkSeg columns, nchunk >= 2, nchunk * K <= kTopkMergeKeys;
                          // 2: one block per row, the row (N <= kTopkSeg) in registers, nchunk = 1;
                          // 3: the filter route, blocks of kTopkFiltCols columns (part: [R][kTopkFiltCap] lists)
    uint32_t* tthr;       // filter route: [R] each row's bound (an order key)
    int* tcnt;            // filter route: [R][64] keys at or above it per list part (may exceed the part)
    int sj;               // filter route: the bound's rank among the 256 sample maxima
};

// modes 0 / 1; splits > 1 (mode 0): grid y splits the reduction (a.D per split, a.ld the row stride)
hipError_t launch_mfma(const MfmaArgs& a, int mode, hipStream_t s, int splits = 1);
hipError_t launch_topk_rows(const TopkRowsArgs& a, hipStream_t s);
hipError_t launch_stream(const StreamArgs& a, int mode, bool f32, int64_t grid, hipStream_t s);
// the whole call in one launch (fused mode): grid = B * P blocks
hipError_t launch_fused(const StreamArgs& a, bool f32, int64_t grid, hipStream_t s);
hipError_t launch_threshold(const ThresholdArgs& a, hipStream_t s);
hipError_t launch_merge(const MergeArgs& a, hipStream_t s);
hipError_t launch_narrow(const NarrowArgs& a, hipStream_t s);
hipError_t launch_cand_plan(const CandPlanArgs& a, hipStream_t s);
hipError_t launch_hot_select(const HotArgs& a, hipStream_t s);
// mode 3 / 4 of launch_mfma take grid y = splits of the reduction
hipError_t launch_mfma_split(const MfmaArgs& a, int mode, int splits, hipStream_t s);
hipError_t launch_ce_prep(const CeArgs& a, hipStream_t s);
hipError_t launch_ce_finish(const CeArgs& a, hipStream_t s);
hipError_t launch_transpose(const TransposeArgs& a, hipStream_t s);
// out[i] = sum_{z < n} in[z * stride + i], i < count
hipError_t launch_sum_splits(const float* in, int n, int64_t stride, int64_t count, float* out, hipStream_t s);

}  // namespace genrec
