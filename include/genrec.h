/*
 * genrec.h -- C ABI of the MI355X (gfx950) ranking-head library, libgenrec.so.
 *
 * The library scores a batch of pooled user vectors H (B x D) against an item
 * catalog E (M x D) and returns, per user, the softmax normaliser (logsumexp)
 * of the scores and the top-K items ranked by score.  The full B x M score
 * matrix is never written to device memory.
 *
 * Sources of the operation:
 *  - GenRec concept page (techistory.net scratchpad, page 13), scoring
 *    formula s = E^T h and its two PyTorch demos: the ranking head is a
 *    bias-free inner product of the user vector with every item embedding,
 *    computed for the whole catalog at once; the catalog is held as (M, D).
 *  - GenRec explainer page (koktn.github.io, "overall picture" section):
 *    s_i = phi(h, e_i); the scores are softmax-normalised over the catalog or
 *    over a candidate set and sorted in descending order to give the ranking;
 *    the paper targets full-catalog ranking or top-K ranking over a
 *    separately given candidate set.
 *  - HSTU explainer page (koktn.github.io, "ranking and retrieval" section):
 *    retrieval over the atomic-ID catalog by MIPS, i.e. exact maximum inner
 *    product top-K, which is the same computation.
 *
 * Conventions shared by all entry points
 *  - Every array argument is a DEVICE pointer owned by the caller.  The library
 *    allocates nothing and keeps no state between calls; scratch space is the
 *    caller's `workspace`, whose size the matching *_workspace() query returns.
 *    Two calls that may run concurrently need distinct workspaces.
 *  - Calls are asynchronous and stream-ordered on `stream` (a hipStream_t,
 *    NULL = the default stream).  Argument errors are detected on the host
 *    before anything is launched and returned synchronously; launch failures
 *    return GENREC_ERR_HIP; faults inside kernels surface at stream sync.
 *  - Layouts: H is [B][D], E is [M][D], both row-major and contiguous
 *    (D innermost).  dtype GENREC_BF16 means bfloat16 elements, GENREC_F32
 *    means float32.  Scores are accumulated in fp32.
 *  - Outputs: out_idx [B][K] int32 catalog ids, out_scores [B][K] float32 raw
 *    scores s (not log-probabilities; log-softmax = s - lse), sorted by score
 *    descending with ties broken by the lower catalog id; out_lse [B] float32,
 *    lse_b = ln sum_i exp(s_bi) over the catalog (or the user's list).
 *    When fewer than K items exist (K > M, or a list shorter than K) the tail
 *    is padded with id -1 and score -inf; an empty set gives lse = -inf.
 *  - Supported: 1 <= K <= GENREC_KMAX, B >= 1, 1 <= M < 2^31,
 *    1 <= D <= GENREC_DMAX with D % 8 == 0 (bf16) or D % 4 == 0 (f32), H and
 *    E 16-byte aligned.  Non-finite inputs are not supported.
 *  - Entry points never abort and no C++ exception crosses the ABI.
 */
#ifndef GENREC_H
#define GENREC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GENREC_OK = 0,
    GENREC_ERR_INVALID_ARG = -1, /* null pointer, non-positive size, bad alignment      */
    GENREC_ERR_UNSUPPORTED = -2, /* shape outside the supported set (K, D multiple, M)  */
    GENREC_ERR_WORKSPACE = -3,   /* workspace NULL or smaller than the query returned    */
    GENREC_ERR_HIP = -4,         /* a HIP runtime call or kernel launch failed           */
    GENREC_ERR_TOO_LARGE = -5    /* allocation-free entry point: the call needs more
                                    workspace than its fixed scratch holds              */
} genrec_status;

typedef enum { GENREC_BF16 = 0, GENREC_F32 = 1 } genrec_dtype;

#define GENREC_KMAX 1024
#define GENREC_DMAX 65536

/* Workspace bytes needed by genrec_score_lse_topk for these sizes (0 if the
 * arguments are unsupported).  The value depends only on the arguments and
 * on the key budget: candidate regions that hold a key for every (user, item)
 * (8 bytes each) are used while they take at most GENREC_KEY_BUDGET bytes
 * (an environment variable read at every call, default 256 MiB); larger
 * shapes with a sampled threshold take bounded regions (a fixed number of
 * keys per (user, catalog chunk, lane group), a per-user overflow region of
 * GENREC_OVERFLOW_KEYS keys, default max(16,384, 16 K + 2,048), a per-user
 * histogram, a collect region of 8 K + 1,024 keys and room for the rescued
 * users' rows): 0.41 GB for B = 1,024, M = 10^6, K = 500, D = 4,096, where
 * regions of every item take 8.2 GB.  Either layout gives the same results;
 * change the variables only between a query and calls that agree on them. */
size_t genrec_score_lse_topk_workspace(int B, int D, int64_t M, int K, int dtype);

/*
 * Full-catalog ranking head: for every user b < B,
 *   s_bi    = sum_d H[b][d] * E[i][d]            for all items i < M
 *   lse_b   = ln sum_i exp(s_bi)
 *   top-K   = the K items with the largest s_bi (ties: lower id first)
 * H: [B][D], E: [M][D] of `dtype`; out_idx, out_scores: [B][K]; out_lse: [B].
 * workspace: device memory of at least genrec_score_lse_topk_workspace(...)
 * bytes, 256-byte aligned; its contents on entry do not matter.
 */
int genrec_score_lse_topk(const void* H, const void* E, int dtype,
                          int B, int D, int64_t M, int K,
                          int32_t* out_idx, float* out_scores, float* out_lse,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * Allocation-free variant of genrec_score_lse_topk, for callers that cannot
 * allocate device memory around the call (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): the same
 * computation and outputs, with the workspace taken from a fixed scratch
 * array that the library holds on each GPU (GENREC_NOALLOC_SCRATCH_BYTES per
 * device, kept until the process ends).  The caller passes inputs and
 * outputs as for genrec_score_lse_topk; nothing is allocated or freed.
 * Shapes whose genrec_score_lse_topk_workspace() exceeds the scratch size
 * return GENREC_ERR_TOO_LARGE before anything is launched.  Every call on
 * one GPU shares that GPU's scratch: calls that may overlap on one GPU (two
 * streams, two host threads) race and must be serialised by the caller.
 * The first call on a device looks the scratch's address up on that device
 * (hipGetSymbolAddress); GENREC_ERR_HIP if that fails.
 */
#define GENREC_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int genrec_score_lse_topk_noalloc(const void* H, const void* E, int dtype,
                                  int B, int D, int64_t M, int K,
                                  int32_t* out_idx, float* out_scores, float* out_lse,
                                  void* stream);

/*
 * Masked full-catalog head: as genrec_score_lse_topk, over the items a
 * bitmask allows.  Item i takes part for user b only when bit (i % 32) of
 * item_mask[b * mask_stride_words + i / 32] is set (least significant bit
 * first); mask_stride_words == 0 means one mask of ceil(M/32) words for every
 * user, else each user's row has mask_stride_words >= ceil(M/32) words.
 * Items left out add nothing to lse and never rank; with fewer than K allowed
 * items the tail is padded (id -1, score -inf), with none lse = -inf.  Bits
 * past M are ignored.  item_mask: device memory, 4-byte aligned, caller-owned.
 * The workspace is the one genrec_score_lse_topk_workspace() gives.  Source:
 * the pages' item filtering -- the GenRec explainer page lists ignored
 * business constraints and out-of-catalog items among the failings of plain
 * LLM rankers; the xGR explainer page's xBeam filters invalid candidates with
 * masks.  Errors: GENREC_ERR_INVALID_ARG for a null or misaligned mask or a
 * stride below ceil(M/32); otherwise as genrec_score_lse_topk.
 */
int genrec_score_lse_topk_masked(const void* H, const void* E, int dtype,
                                 int B, int D, int64_t M, int K,
                                 const uint32_t* item_mask, int64_t mask_stride_words,
                                 int32_t* out_idx, float* out_scores, float* out_lse,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes needed by genrec_score_candidates_topk (0 if unsupported). */
size_t genrec_score_candidates_topk_workspace(int B, int D, int64_t M, int64_t nnz, int K,
                                              int dtype);

/*
 * Candidate-set ranking head: user b scores only its own list
 *   ids[cand_offsets[b] .. cand_offsets[b+1])      (CSR, catalog ids)
 * and returns lse over those entries and the top-K entries (as catalog ids,
 * ties broken by the lower id).  cand_offsets: [B+1] int64 with
 * cand_offsets[0] == 0, non-decreasing, cand_offsets[B] == nnz; cand_ids:
 * [nnz] int32.  Each entry is scored as given: a duplicated id counts twice.
 * Ids outside [0, M) are skipped and counted; malformed offsets make the
 * affected users empty and are counted too (see genrec_get_device_errors).
 * nnz may be 0 (then cand_ids may be NULL).
 */
int genrec_score_candidates_topk(const void* H, const void* E, int dtype,
                                 const int64_t* cand_offsets, const int32_t* cand_ids,
                                 int B, int D, int64_t M, int64_t nnz, int K,
                                 int32_t* out_idx, float* out_scores, float* out_lse,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * Reads the device error counters that the last candidate call on this
 * workspace wrote: *n_bad_ids = number of skipped out-of-range ids,
 * *n_bad_offsets = number of users whose offsets were malformed.  Either
 * output pointer may be NULL.  Synchronises `stream`.
 */
int genrec_get_device_errors(const void* workspace, void* stream, int64_t* n_bad_ids,
                             int64_t* n_bad_offsets);

/*
 * Number of users of the last genrec_score_lse_topk call on this workspace
 * that needed the rescue pass.  On the MFMA path with a sampled threshold the
 * main pass keeps only scores at or above a fast threshold (a high-ranked
 * sampled score); a user for whom fewer than K catalog items reach it is
 * scored again with the K-th largest sampled score, which at least K items
 * always reach.  Results are exact either way; the count reports the extra
 * work.  Synchronises `stream`.  GENREC_ERR_INVALID_ARG for null pointers.
 */
int genrec_get_rescued_users(const void* workspace, void* stream, int64_t* n_rescued);

/*
 * Batched top-K of dense score rows -- the selection step of a beam search
 * (xGR explainer page, xBeam: beam widths of 128 to 512, e.g. 128 beams x 128
 * continuations = 16,384 candidates ranked down to the best 128, without a
 * full sort).  For each row r < R of scores (fp32, row r at scores + r * ld,
 * its first N entries used, ld >= N), the K largest entries ranked by score
 * descending, ties by the lower column: out_idx [R][K] int32 column indices,
 * out_scores [R][K] the scores.  K > N pads with (-1, -inf).  Long rows are
 * either split into chunks merged by a second pass or, for K <= 512 and N
 * between about 36 K and 4e6, filtered (xBeam's filtering before the sort):
 * a sampled lower bound on each row's top K, one pass that lists the keys
 * at or above it (8,192 per row at most), and a ranking of the list -- a row
 * whose list falls short of K or overflows is ranked from the whole row, so
 * results are exact either way.  Both need `workspace` of
 * genrec_topk_rows_workspace(R, N, K) bytes (8-byte aligned; the filter
 * route about 64 KiB per row; 0 bytes -- workspace may be NULL -- when one
 * pass suffices); its contents on entry do not matter.  Asynchronous on
 * `stream`.  1 <= K <= GENREC_KMAX, 1 <= N < 2^31, R >= 1, 4-byte aligned
 * pointers; GENREC_ERR_INVALID_ARG / GENREC_ERR_UNSUPPORTED /
 * GENREC_ERR_WORKSPACE otherwise.  Non-finite scores are not supported.
 */
size_t genrec_topk_rows_workspace(int R, int64_t N, int K);
int genrec_topk_rows(const float* scores, int R, int64_t N, int64_t ld, int K,
                     int32_t* out_idx, float* out_scores,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * Cross-entropy over the whole catalog, forward and backward, without a
 * B x M score matrix in memory (GenRec explainer page, "two objectives and
 * reward-weighted ranking" section: the ranking objective is a cross-entropy
 * over the catalog, each example's loss multiplied by a scalar weight built
 * from reward signals; its "start from the ranking head" step: an
 * inner-product head trained with the full-catalog softmax).
 *
 * bf16 only.  H [B][D], E [M][D] as above (16-byte aligned, D % 8 == 0);
 * labels [B] int32 catalog ids; weights [B] float32, or NULL for all ones.
 * With s_bi = h_b . e_i and lse_b = ln sum_i exp(s_bi):
 *   forward:   out_loss[b] = w_b (lse_b - s_{b,y_b}),  out_lse[b] = lse_b;
 *   backward:  with G[b][i] = w_b (exp(s_bi - lse_b) - [i == y_b]),
 *              out_dH = G E  ([B][D] float32),  out_dE = G^T H  ([M][D], float32 when
 *              de_dtype is GENREC_F32, bfloat16 rounded to nearest even when it is
 *              GENREC_BF16 -- half the bytes of the largest output),
 *              the gradients of sum_b out_loss[b]; `lse` is the forward's out_lse.
 * An example whose label lies outside [0, M) is ignored (loss 0, no
 * gradient) and counted: genrec_get_device_errors on the same workspace
 * reports the count as *n_bad_ids (and 0 as *n_bad_offsets).
 * The backward recomputes the scores chunk by chunk (65,536 catalog rows at a
 * time, fewer when D or B exceeds 8,192 so that each chunk operand stays under
 * 1 GiB; B or D above 2^21 is GENREC_ERR_UNSUPPORTED for the backward),
 * holds G of one chunk in bf16 (rounded to nearest even) and computes
 * both products on the matrix cores with fp32 accumulation; only the
 * workspace of genrec_ce_backward_workspace() bytes is used.  Asynchronous on
 * `stream`; out_dH and out_dE are overwritten.  Outputs 4-byte aligned,
 * workspace 256-byte aligned.  GENREC_ERR_INVALID_ARG / _UNSUPPORTED /
 * _WORKSPACE as for the other entry points.
 */
size_t genrec_ce_forward_workspace(int B, int D, int64_t M);
int genrec_ce_forward(const void* H, const void* E, int B, int D, int64_t M,
                      const int32_t* labels, const float* weights,
                      float* out_loss, float* out_lse,
                      void* workspace, size_t workspace_bytes, void* stream);
size_t genrec_ce_backward_workspace(int B, int D, int64_t M);
int genrec_ce_backward(const void* H, const void* E, int B, int D, int64_t M,
                       const int32_t* labels, const float* weights, const float* lse,
                       float* out_dH, void* out_dE, int de_dtype,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Introspection: writes into buf (at most len bytes, NUL-terminated) a JSON
 * object describing how genrec_score_lse_topk would run these sizes: the
 * scoring path ("mfma" or "stream"), whether the sampled-threshold pre-pass
 * runs (its tile stride, sample size, fast-threshold rank, reduction splits,
 * whether the sampled scores are the main pass's bits -- "safe_exact" -- and
 * "first_sampled_tile", the catalog tile of 256 rows the sample takes from
 * the first window of "stride" tiles, or -1 without a sample), the work
 * split, which build of the top-K merge runs ("merge_small": the one with the
 * smaller LDS gather, for few expected candidates per user), whether the
 * candidate regions are bounded ("bounded", with "cap" keys per piece, an
 * overflow region of "ovf_cap" keys per user and a collect region of "ccol"
 * keys per rescued user) and the workspace size.
 * Host-only, touches no device.
 * Returns GENREC_OK or the status the compute call would return for the
 * shape. */
int genrec_describe_plan(int B, int D, int64_t M, int K, int dtype, char* buf, size_t len);

/* Introspection of the cross-entropy backward's plan for these sizes: writes
 * into buf (at most len bytes, NUL-terminated) a JSON object with the catalog
 * rows per backward chunk ("chunk", "Mcp" = the chunk rounded up to 256),
 * the number of chunks, the users padded to 32 ("Bp"), the reduction splits
 * of the dH product ("splits"), and the longest chains of fp32 additions into
 * one output of the two gradient products: "depth_h" = Mcp / splits (one
 * split's reduction) + n_chunks (accumulation over the chunks) + splits (the
 * final sum of the partials), "depth_e" = Bp (the reduction over the padded
 * users).  These bound the products' rounding (depth * 2^-24 relative).
 * Host-only.  Returns GENREC_OK, GENREC_ERR_INVALID_ARG for non-positive
 * sizes or a null / empty buf, GENREC_ERR_UNSUPPORTED where
 * genrec_ce_backward_workspace() returns 0. */
int genrec_describe_ce_plan(int B, int D, int64_t M, char* buf, size_t len);

/* Introspection of the candidate path's plan (genrec_score_candidates_topk)
 * for these sizes: writes into buf (at most len bytes, NUL-terminated) a
 * JSON object with "hot" (1: the most-listed rows are scored densely on the
 * matrix cores), "t_max" (hot rows at most), "c_min" (the smallest count that
 * makes a row hot), "sample_every" (the list counts come from every this-many
 * entries of the id array: entries 0, 16, 32, ...), "n_pieces_max" (work
 * pieces at most), the byte offsets in the workspace of the per-item counts
 * ("off_counts": int32[M], after a call the number of sampled entries naming
 * each id; -1 without a hot head) and of the hot-head result ("off_meta":
 * int32 count threshold c, then the number of hot rows; -1 without), and the
 * workspace size.  Host-only.  Returns GENREC_OK, the status the compute
 * call would return for the sizes, GENREC_ERR_INVALID_ARG for nnz < 0 or a
 * null / empty buf. */
int genrec_describe_cand_plan(int B, int D, int64_t M, int64_t nnz, int K, int dtype, char* buf, size_t len);

/*
 * Kernel-level timing with HIP events.  A profiler records an event pair
 * around every kernel that the *_profiled entry points launch, without
 * synchronising; genrec_profiler_summary() synchronises on the last event and
 * returns, per kernel kind, the number of launches and their summed duration
 * in milliseconds.  Kinds: 0 sampled-threshold scoring pass, 1 threshold
 * selection, 2 main scoring pass (MFMA or VALU), 3 top-K merge, 4 candidate
 * work-list plan, 5 rescue (the scoring pass and merge that recompute users
 * left short of K candidates; they exit at once when no user is), 6 hot-head
 * selection of a candidate call (per-item list counts, the count threshold,
 * the compaction and gather of the most-listed catalog rows), 7 dense scoring
 * of those rows for every user, 8 small cross-entropy kernels (label check,
 * loss, sum of the dH partials), 9 transposes (H, catalog chunks), 10 softmax-
 * minus-target tiles G, 11 dE product, 12 dH product.  One profiler holds up to `max_launches` launches; further
 * launches are not recorded.  A profiler may only be used by one stream at a
 * time.  create returns NULL on failure.
 */
#define GENREC_NUM_KERNEL_KINDS 13
typedef struct genrec_profiler genrec_profiler;
genrec_profiler* genrec_profiler_create(int max_launches);
void genrec_profiler_destroy(genrec_profiler* prof);
int genrec_profiler_reset(genrec_profiler* prof);
int genrec_profiler_summary(genrec_profiler* prof, int* counts, double* total_ms);

/* Same as genrec_score_lse_topk / genrec_score_lse_topk_masked /
 * genrec_score_candidates_topk / genrec_ce_forward / genrec_ce_backward,
 * recording every launch into `prof` (which may be NULL). */
int genrec_score_lse_topk_profiled(const void* H, const void* E, int dtype,
                                   int B, int D, int64_t M, int K,
                                   int32_t* out_idx, float* out_scores, float* out_lse,
                                   void* workspace, size_t workspace_bytes, void* stream,
                                   genrec_profiler* prof);
int genrec_score_lse_topk_masked_profiled(const void* H, const void* E, int dtype,
                                          int B, int D, int64_t M, int K,
                                          const uint32_t* item_mask, int64_t mask_stride_words,
                                          int32_t* out_idx, float* out_scores, float* out_lse,
                                          void* workspace, size_t workspace_bytes, void* stream,
                                          genrec_profiler* prof);
int genrec_score_candidates_topk_profiled(const void* H, const void* E, int dtype,
                                          const int64_t* cand_offsets, const int32_t* cand_ids,
                                          int B, int D, int64_t M, int64_t nnz, int K,
                                          int32_t* out_idx, float* out_scores, float* out_lse,
                                          void* workspace, size_t workspace_bytes, void* stream,
                                          genrec_profiler* prof);
int genrec_ce_forward_profiled(const void* H, const void* E, int B, int D, int64_t M,
                               const int32_t* labels, const float* weights,
                               float* out_loss, float* out_lse,
                               void* workspace, size_t workspace_bytes, void* stream,
                               genrec_profiler* prof);
int genrec_ce_backward_profiled(const void* H, const void* E, int B, int D, int64_t M,
                                const int32_t* labels, const float* weights, const float* lse,
                                float* out_dH, void* out_dE, int de_dtype,
                                void* workspace, size_t workspace_bytes, void* stream,
                                genrec_profiler* prof);

/* Human-readable name of a genrec_status value (static storage). */
const char* genrec_status_string(int status);

/* Library version as 10000*major + 100*minor + patch. */
int genrec_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GENREC_H */
