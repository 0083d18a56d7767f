/*
 * CPU oracle for the ranking head: a plain, slow, obviously correct reference.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or calls
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline
 * leg use it.  It shares no code with the GPU library.
 *
 * What it computes (plain definitions, fp64 throughout):
 *
 *  scores   s[b][i] = sum_{d=0}^{D-1} H[b][d] * E[i][d]
 *           The ranking head is the inner product of the pooled user vector
 *           with every item embedding, computed for all M items at once
 *           (GenRec concept page: s = E^T h and its PyTorch demos, a bias-free
 *           linear head and `user_vector @ candidate_embeddings.T`; GenRec
 *           explainer page, "overall picture": s_i = phi(h, e_i)).
 *           Inputs arrive as bf16 or fp32 bit patterns and are widened exactly
 *           to double; the products of two bf16 / two fp32 values are exact in
 *           double, the sum runs in index order d = 0..D-1.
 *
 *  lse      lse[b] = m + ln sum_i exp(s[b][i] - m), m = max_i s[b][i]
 *           The softmax normaliser over the catalog or over the candidate set
 *           (GenRec explainer page, "overall picture": softmax over the
 *           catalog or candidate set, then sort).  The sum is Neumaier-
 *           compensated.  An empty set gives -inf.
 *
 *  top-K    a full stable sort of the items by score, descending, then the
 *           first K (same passage: ranking = descending order).  Ties keep
 *           the lower catalog id first.  Fewer than K items: the tail is
 *           padded with (id -1, score -inf).
 *
 *  masked   the same three steps over the items a bitmask allows: item i
 *           takes part for user b only when bit i % 32 of word
 *           mask[b * stride + i / 32] is set (stride 0: one mask for every
 *           user).  Items left out add nothing to the normaliser and never
 *           rank; fewer than K allowed items pad as above.  (Reading of the
 *           pages' item filtering: the GenRec explainer page, on why plain
 *           LLM rankers fall short, lists ignored business constraints and
 *           items outside the catalog; the xGR explainer page, xBeam, filters
 *           invalid candidates with masks.)
 *
 *  candidates: the same three steps over user b's list
 *           ids[offsets[b] .. offsets[b+1]) only (GenRec explainer page, top-K
 *           ranking over a separately given candidate set).  Entries are
 *           ordered by (score desc, catalog id asc, list position asc).
 *           Ids outside [0, M) are skipped and counted.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC (no -ffast-math).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_BF16 = 0, ORACLE_F32 = 1 };

static double widen(const void* base, int dtype, int64_t k) {
    if (dtype == ORACLE_BF16) {
        uint32_t u = (uint32_t)((const uint16_t*)base)[k] << 16;
        float f;
        memcpy(&f, &u, 4);
        return (double)f;
    }
    return (double)((const float*)base)[k];
}

int oracle_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Inner product of user row b with item row i, summed in order d = 0..D-1. */
static double dot_row(const void* H, const void* E, int dtype, int64_t D, int64_t b, int64_t i) {
    double acc = 0.0;
    for (int64_t d = 0; d < D; ++d)
        acc += widen(H, dtype, b * D + d) * widen(E, dtype, i * D + d);
    return acc;
}

/* S[r][i] for the users listed in `users` (nu of them) against all M items. */
void oracle_scores(const void* H, const void* E, int dtype, int64_t D, int64_t M,
                   const int64_t* users, int64_t nu, double* S) {
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i)
        for (int64_t r = 0; r < nu; ++r)
            S[r * M + i] = dot_row(H, E, dtype, D, users[r], i);
}

/* Scores of explicit (user, item) pairs. */
void oracle_pair_scores(const void* H, const void* E, int dtype, int64_t D,
                        const int64_t* users, const int64_t* items, int64_t n, double* out) {
    #pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; ++j)
        out[j] = dot_row(H, E, dtype, D, users[j], items[j]);
}

double oracle_lse(const double* s, int64_t n) {
    if (n <= 0) return -INFINITY;
    double m = s[0];
    for (int64_t i = 1; i < n; ++i)
        if (s[i] > m) m = s[i];
    if (isinf(m)) return m;
    double sum = 0.0, comp = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        double t = exp(s[i] - m);
        double y = sum + t;
        if (fabs(sum) >= fabs(t)) comp += (sum - y) + t;
        else comp += (t - y) + sum;
        sum = y;
    }
    return m + log(sum + comp);
}

/* Ordering used by the ranking: higher score first, then lower catalog id,
 * then lower position.  Returns nonzero if entry a must precede entry b. */
static int before(const double* s, const int64_t* id, int64_t a, int64_t b) {
    if (s[a] != s[b]) return s[a] > s[b];
    if (id[a] != id[b]) return id[a] < id[b];
    return a < b;
}

/* Stable top-down merge sort of positions perm[0..n) under `before`. */
static void merge_sort(int64_t* perm, int64_t* tmp, int64_t n, const double* s, const int64_t* id) {
    if (n < 2) return;
    int64_t h = n / 2;
    merge_sort(perm, tmp, h, s, id);
    merge_sort(perm + h, tmp, n - h, s, id);
    int64_t i = 0, j = h, k = 0;
    while (i < h && j < n) {
        if (before(s, id, perm[j], perm[i])) tmp[k++] = perm[j++];
        else tmp[k++] = perm[i++];
    }
    while (i < h) tmp[k++] = perm[i++];
    while (j < n) tmp[k++] = perm[j++];
    memcpy(perm, tmp, (size_t)n * sizeof(int64_t));
}

/* Rank the n entries (scores s, catalog ids id) and keep the first K. */
static void rank_topk(const double* s, const int64_t* id, int64_t n, int64_t K,
                      int64_t* out_idx, double* out_score) {
    int64_t* perm = (int64_t*)malloc((size_t)(n > 0 ? n : 1) * sizeof(int64_t));
    int64_t* tmp = (int64_t*)malloc((size_t)(n > 0 ? n : 1) * sizeof(int64_t));
    for (int64_t i = 0; i < n; ++i) perm[i] = i;
    merge_sort(perm, tmp, n, s, id);
    for (int64_t j = 0; j < K; ++j) {
        if (j < n) {
            out_idx[j] = id[perm[j]];
            out_score[j] = s[perm[j]];
        } else {
            out_idx[j] = -1;
            out_score[j] = -INFINITY;
        }
    }
    free(perm);
    free(tmp);
}

/* Top-K of one dense row s[0..M) (ids are the positions). */
void oracle_topk_row(const double* s, int64_t M, int64_t K, int64_t* out_idx, double* out_score) {
    int64_t* id = (int64_t*)malloc((size_t)(M > 0 ? M : 1) * sizeof(int64_t));
    for (int64_t i = 0; i < M; ++i) id[i] = i;
    rank_topk(s, id, M, K, out_idx, out_score);
    free(id);
}

/* Full-catalog head for the listed users.  S (nu x M) receives the scores. */
void oracle_full(const void* H, const void* E, int dtype, int64_t D, int64_t M, int64_t K,
                 const int64_t* users, int64_t nu, double* S,
                 int64_t* out_idx, double* out_score, double* out_lse) {
    oracle_scores(H, E, dtype, D, M, users, nu, S);
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nu; ++r) {
        out_lse[r] = oracle_lse(S + r * M, M);
        oracle_topk_row(S + r * M, M, K, out_idx + r * K, out_score + r * K);
    }
}

/* Masked full-catalog head for the listed users: the items of user b are
 * those whose mask bit is set (see the header).  S (nu x M) receives every
 * score, allowed or not. */
void oracle_full_masked(const void* H, const void* E, int dtype, int64_t D, int64_t M, int64_t K,
                        const uint32_t* mask, int64_t stride, const int64_t* users, int64_t nu, double* S,
                        int64_t* out_idx, double* out_score, double* out_lse) {
    oracle_scores(H, E, dtype, D, M, users, nu, S);
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nu; ++r) {
        const uint32_t* mrow = mask + users[r] * stride;
        double* s = (double*)malloc((size_t)(M > 0 ? M : 1) * sizeof(double));
        int64_t* id = (int64_t*)malloc((size_t)(M > 0 ? M : 1) * sizeof(int64_t));
        int64_t kept = 0;
        for (int64_t i = 0; i < M; ++i) {
            if ((mrow[i / 32] >> (i % 32)) & 1u) {
                s[kept] = S[r * M + i];
                id[kept] = i;
                ++kept;
            }
        }
        out_lse[r] = oracle_lse(s, kept);
        rank_topk(s, id, kept, K, out_idx + r * K, out_score + r * K);
        free(s);
        free(id);
    }
}

/* Candidate-set head for the listed users.  `scores` receives, per entry of
 * the CSR list (nnz of them), h_b . E[id] for the entries of listed users
 * (NaN where the id is out of range).  Returns the number of skipped ids. */
int64_t oracle_cand(const void* H, const void* E, int dtype, int64_t D, int64_t M, int64_t K,
                    const int64_t* offsets, const int32_t* ids,
                    const int64_t* users, int64_t nu, double* scores,
                    int64_t* out_idx, double* out_score, double* out_lse) {
    int64_t bad = 0;
    #pragma omp parallel for schedule(dynamic, 1) reduction(+ : bad)
    for (int64_t r = 0; r < nu; ++r) {
        int64_t b = users[r];
        int64_t e0 = offsets[b], n = offsets[b + 1] - offsets[b];
        double* s = (double*)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
        int64_t* id = (int64_t*)malloc((size_t)(n > 0 ? n : 1) * sizeof(int64_t));
        int64_t kept = 0;
        for (int64_t j = 0; j < n; ++j) {
            int64_t c = ids[e0 + j];
            if (c < 0 || c >= M) {
                scores[e0 + j] = NAN;
                ++bad;
                continue;
            }
            s[kept] = dot_row(H, E, dtype, D, b, c);
            id[kept] = c;
            scores[e0 + j] = s[kept];
            ++kept;
        }
        out_lse[r] = oracle_lse(s, kept);
        rank_topk(s, id, kept, K, out_idx + r * K, out_score + r * K);
        free(s);
        free(id);
    }
    return bad;
}
