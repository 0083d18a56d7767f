// C ABI of libgenrec.so: argument validation, planning, and stream-ordered
// launches.  See include/genrec.h for the contract of each entry point.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <mutex>
#include <new>

#include "../../include/genrec.h"
#include "launch.hpp"
#include "mfma_layout.hpp"
#include "plan.hpp"
#include "validate.hpp"

using namespace genrec;

namespace {

inline int hip_status(hipError_t e) { return e == hipSuccess ? GENREC_OK : GENREC_ERR_HIP; }

// Per-call tickets of the fused path's arrival words: 40 bits, never 0 or all
// ones, unique within the process (a counter from a start that differs from
// run to run, so that a word another process or tensor left in reused memory
// is unlikely to hold a live ticket).
uint64_t next_ticket() {
    constexpr uint64_t kMask = (1ull << 40) - 1;
    static std::atomic<uint64_t> counter{[] {
        uint64_t x = (uint64_t)std::chrono::steady_clock::now().time_since_epoch().count();
        x ^= (uint64_t)(uintptr_t)&counter;
        x ^= x >> 31;
        x *= 0x9E3779B97F4A7C15ull;
        return x ^ (x >> 29);
    }()};
    for (;;) {
        const uint64_t t = counter.fetch_add(1, std::memory_order_relaxed) & kMask;
        if (t != 0 && t != kMask) return t;
    }
}

// Budget of the candidate regions that hold every item (8 bytes per user and
// item); larger shapes take bounded regions.  GENREC_KEY_BUDGET (bytes) sets
// it for the process, read at every plan, so that a workspace query and the
// call it sizes agree while the variable is unchanged.
// GENREC_OVERFLOW_KEYS sets the keys of each user's overflow region in the
// bounded layout the same way (0: none).  Unparsable values are ignored.
bool env_size(const char* name, unsigned long long& v) {
    const char* e = getenv(name);
    // digits only: strtoull would also take a sign (wrapping "-5" to 2^64 - 5) or leading blanks
    if (e == nullptr || *e < '0' || *e > '9') return false;
    char* end = nullptr;
    v = strtoull(e, &end, 10);
    return end != nullptr && *end == '\0';
}

size_t key_budget() {
    unsigned long long v = 0;
    return env_size("GENREC_KEY_BUDGET", v) ? (size_t)v : kDefaultKeyBudget;
}

DensePlan plan_dense_env(int B, int D, int64_t M, int K, int dtype) {
    unsigned long long o = 0;
    const int64_t ovf = env_size("GENREC_OVERFLOW_KEYS", o) ? (int64_t)std::min<unsigned long long>(o, 1ull << 30) : -1;
    return plan_dense(B, D, M, K, dtype, key_budget(), ovf);
}

template <class T>
inline T* at(void* ws, size_t off) {
    return (T*)((uint8_t*)ws + off);
}

}  // namespace

struct genrec_profiler {
    int cap = 0, n = 0;
    hipEvent_t* ev = nullptr;  // 2 per launch
    int* kind = nullptr;
};

namespace {

// Runs one launch, bracketed by profiler events when a profiler is given.
template <class F>
hipError_t timed(genrec_profiler* prof, int kind, hipStream_t s, F&& launch) {
    if (!prof || prof->n >= prof->cap) return launch();
    hipError_t e = hipEventRecord(prof->ev[2 * prof->n], s);
    if (e != hipSuccess) return e;
    e = launch();
    if (e != hipSuccess) return e;
    e = hipEventRecord(prof->ev[2 * prof->n + 1], s);
    if (e != hipSuccess) return e;
    prof->kind[prof->n++] = kind;
    return hipSuccess;
}

enum { KIND_SAMPLE = 0, KIND_THRESHOLD = 1, KIND_MAIN = 2, KIND_MERGE = 3, KIND_PLAN = 4, KIND_RESCUE = 5,
       KIND_HOT_SELECT = 6, KIND_HOT_SCORE = 7, KIND_CE_SMALL = 8, KIND_TRANSPOSE = 9, KIND_GRAD_TILES = 10,
       KIND_GRAD_E = 11, KIND_GRAD_H = 12 };

}  // namespace

extern "C" {

genrec_profiler* genrec_profiler_create(int max_launches) {
    if (max_launches <= 0) return nullptr;
    genrec_profiler* p = new (std::nothrow) genrec_profiler();
    if (!p) return nullptr;
    p->ev = new (std::nothrow) hipEvent_t[2 * (size_t)max_launches]();
    p->kind = new (std::nothrow) int[max_launches]();
    if (!p->ev || !p->kind) {
        delete[] p->ev;
        delete[] p->kind;
        delete p;
        return nullptr;
    }
    for (int i = 0; i < 2 * max_launches; ++i) {
        if (hipEventCreate(&p->ev[i]) != hipSuccess) {
            for (int j = 0; j < i; ++j) (void)hipEventDestroy(p->ev[j]);
            delete[] p->ev;
            delete[] p->kind;
            delete p;
            return nullptr;
        }
    }
    p->cap = max_launches;
    return p;
}

void genrec_profiler_destroy(genrec_profiler* p) {
    if (!p) return;
    for (int i = 0; i < 2 * p->cap; ++i) (void)hipEventDestroy(p->ev[i]);
    delete[] p->ev;
    delete[] p->kind;
    delete p;
}

int genrec_profiler_reset(genrec_profiler* p) {
    if (!p) return GENREC_ERR_INVALID_ARG;
    p->n = 0;
    return GENREC_OK;
}

int genrec_profiler_summary(genrec_profiler* p, int* counts, double* total_ms) {
    if (!p || !counts || !total_ms) return GENREC_ERR_INVALID_ARG;
    for (int k = 0; k < GENREC_NUM_KERNEL_KINDS; ++k) {
        counts[k] = 0;
        total_ms[k] = 0.0;
    }
    if (p->n == 0) return GENREC_OK;
    if (hipEventSynchronize(p->ev[2 * p->n - 1]) != hipSuccess) return GENREC_ERR_HIP;
    for (int i = 0; i < p->n; ++i) {
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, p->ev[2 * i], p->ev[2 * i + 1]) != hipSuccess) return GENREC_ERR_HIP;
        counts[p->kind[i]] += 1;
        total_ms[p->kind[i]] += ms;
    }
    return GENREC_OK;
}


int genrec_version(void) { return 10000; }

const char* genrec_status_string(int status) {
    switch (status) {
        case GENREC_OK: return "GENREC_OK";
        case GENREC_ERR_INVALID_ARG: return "GENREC_ERR_INVALID_ARG";
        case GENREC_ERR_UNSUPPORTED: return "GENREC_ERR_UNSUPPORTED";
        case GENREC_ERR_WORKSPACE: return "GENREC_ERR_WORKSPACE";
        case GENREC_ERR_HIP: return "GENREC_ERR_HIP";
        case GENREC_ERR_TOO_LARGE: return "GENREC_ERR_TOO_LARGE";
        default: return "GENREC_UNKNOWN_STATUS";
    }
}

size_t genrec_score_lse_topk_workspace(int B, int D, int64_t M, int K, int dtype) {
    static const float dummy[4] = {0, 0, 0, 0};
    if (check_common(dummy, dummy, dtype, B, D, M, K, (const int32_t*)dummy, dummy, dummy) != GENREC_OK)
        return 0;
    return plan_dense_env(B, D, M, K, dtype).total;  // 0 when the plan is unsupported
}

int genrec_describe_plan(int B, int D, int64_t M, int K, int dtype, char* buf, size_t len) {
    static const float dummy[4] = {0, 0, 0, 0};
    const int st = check_common(dummy, dummy, dtype, B, D, M, K, (const int32_t*)dummy, dummy, dummy);
    if (st != GENREC_OK) return st;
    if (!buf || len == 0) return GENREC_ERR_INVALID_ARG;
    const DensePlan p = plan_dense_env(B, D, M, K, dtype);
    if (!p.ok) return GENREC_ERR_UNSUPPORTED;
    snprintf(buf, len,
             "{\"path\":\"%s\",\"sample\":%d,\"stride\":%lld,\"n_sample\":%lld,\"fast\":%d,\"r_fast\":%d,"
             "\"UT\":%d,\"P\":%d,\"tiles_per_chunk\":%d,\"CH\":%lld,\"merge_small\":%d,\"fused\":%d,"
             "\"sample_splits\":%d,\"safe_exact\":%d,\"first_sampled_tile\":%lld,\"bounded\":%d,\"cap\":%d,"
             "\"ccol\":%d,\"ovf_cap\":%d,\"workspace\":%zu}",
             p.mfma ? "mfma" : "stream", p.sample ? 1 : 0, (long long)p.stride, (long long)p.n_sample,
             p.fast ? 1 : 0, p.r_fast, p.main.UT, p.main.P, p.main.base + (p.main.rem ? 1 : 0),
             (long long)p.main.CH, p.merge_small ? 1 : 0, p.fused ? 1 : 0, p.sample_splits, p.safe_exact ? 1 : 0,
             p.sample ? mf_sample_tile(0, p.stride, M / kMfmaTileItems) : -1LL, p.bounded ? 1 : 0, p.cap, p.ccol,
             p.ovf_cap, p.total);
    return GENREC_OK;
}

int genrec_score_lse_topk(const void* H, const void* E, int dtype, int B, int D, int64_t M, int K,
                          int32_t* out_idx, float* out_scores, float* out_lse, void* workspace,
                          size_t workspace_bytes, void* stream) {
    return genrec_score_lse_topk_profiled(H, E, dtype, B, D, M, K, out_idx, out_scores, out_lse, workspace,
                                          workspace_bytes, stream, nullptr);
}

}  // extern "C"

namespace {

// The full-catalog head, with an optional item mask (null: every item).
int score_dense(const void* H, const void* E, int dtype, int B, int D, int64_t M, int K, const uint32_t* mask,
                int64_t mask_stride, int32_t* out_idx, float* out_scores, float* out_lse, void* workspace,
                size_t workspace_bytes, void* stream, genrec_profiler* prof) {
    int st = check_common(H, E, dtype, B, D, M, K, out_idx, out_scores, out_lse);
    if (st != GENREC_OK) return st;
    const DensePlan p = plan_dense_env(B, D, M, K, dtype);
    if (!p.ok) return GENREC_ERR_UNSUPPORTED;
    if (!workspace || workspace_bytes < p.total) return GENREC_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return GENREC_ERR_INVALID_ARG;
    hipStream_t s = (hipStream_t)stream;

    if (p.fused) {
        // the whole call in one launch: scoring blocks, and per user the last
        // of its blocks computes lse and the top-K
        StreamArgs a{};
        a.H = H;
        a.E = E;
        a.B = B;
        a.D = D;
        a.M = M;
        a.mask = mask;
        a.mask_stride = mask_stride;
        a.n_items = M;
        a.tile_stride = 1;
        a.CH = p.main.CH;
        a.P = p.main.P;
        a.pm = at<float>(workspace, p.off_pm);
        a.pl = at<float>(workspace, p.off_pl);
        a.err = at<int64_t>(workspace, p.off_hdr);
        a.rows = at<float>(workspace, p.off_rows);
        a.arrive = at<uint64_t>(workspace, p.off_arrive);
        a.elect = at<uint64_t>(workspace, p.off_elect);
        a.ticket = next_ticket();
        a.K = K;
        a.out_idx = out_idx;
        a.out_scores = out_scores;
        a.out_lse = out_lse;
        return hip_status(timed(prof, KIND_MAIN, s, [&] {
            return launch_fused(a, dtype == GENREC_F32, (int64_t)B * p.main.P, s);
        }));
    }

    float* theta_fast = at<float>(workspace, p.off_theta);
    float* theta_safe = at<float>(workspace, p.off_theta_safe);
    int* uflag = at<int>(workspace, p.off_uflag);
    int* tflag = at<int>(workspace, p.off_tflag);
    int64_t* rescued = at<int64_t>(workspace, p.off_hdr + kHdrRescued);
    float* sample = at<float>(workspace, p.off_sample);
    float* pm = at<float>(workspace, p.off_pm);
    float* pl = at<float>(workspace, p.off_pl);
    int* pcnt = at<int>(workspace, p.off_pcnt);
    int64_t* preg = at<int64_t>(workspace, p.off_preg);
    uint64_t* keys = at<uint64_t>(workspace, p.off_keys);
    const bool f32 = dtype == GENREC_F32;

    ThresholdArgs th{};
    th.sample = sample;
    th.n_sample = p.n_sample;
    th.B = B;
    th.K = K;
    th.r_fast = p.r_fast;
    th.n_split = p.sample_splits;
    th.split_stride = (int64_t)B * p.n_sample;
    th.theta_safe = theta_safe;
    th.theta_fast = p.fast ? theta_fast : nullptr;
    th.user_flag = uflag;
    th.tile_flag = tflag;
    th.rc = p.bounded ? at<int>(workspace, p.off_rc) : nullptr;
    th.rescued = rescued;
    if (p.bounded) {
        th.ovf_pm = at<float>(workspace, p.off_pm);
        th.ovf_pl = at<float>(workspace, p.off_pl);
        th.ovf_pcnt = at<int>(workspace, p.off_pcnt);
        th.ovf_preg = at<int64_t>(workspace, p.off_preg);
        th.rec_stride = p.rec_stride;
        th.rec_off = p.rec_stride - 1;
        th.ovf_base = p.n_pieces * p.cap;
        th.ovf_cap = p.ovf_cap;
    }
    // The rescue counter is cleared by the threshold kernel when it runs,
    // else by the merge (see below).

    MfmaArgs a{};
    if (p.mfma) {
        a.H = (const uint16_t*)H;
        a.E = (const uint16_t*)E;
        a.f32 = f32 ? 1 : 0;
        a.B = B;
        a.D = D;
        a.M = M;
        a.mask = mask;
        a.mask_stride = mask_stride;
        if (p.sample) {
            a.n_tiles = (int)p.sample_tiles;
            a.tile_stride = (int)p.stride;
            a.UT = p.pre.UT;
            a.P = p.pre.P;
            a.base = p.pre.base;
            a.rem = p.pre.rem;
            a.sample_out = sample;
            // reduction split over grid y: each split's partial scores in a row
            // block of its own, summed by the threshold kernel
            a.ld = D;
            a.D = D / p.sample_splits;
            a.k_split = D / p.sample_splits;
            a.sample_split = (int64_t)B * p.n_sample;
            if ((st = hip_status(timed(prof, KIND_SAMPLE, s, [&] { return launch_mfma(a, 0, s, p.sample_splits); }))) !=
                GENREC_OK)
                return st;
            if ((st = hip_status(timed(prof, KIND_THRESHOLD, s, [&] { return launch_threshold(th, s); }))) != GENREC_OK) return st;
            a.ld = 0;
            a.D = D;
            a.k_split = 0;
            a.sample_split = 0;
        }
        a.n_tiles = (int)ceil_div(M, kMfmaTileItems);
        a.tile_stride = 1;
        a.UT = p.main.UT;
        a.P = p.main.P;
        a.base = p.main.base;
        a.rem = p.main.rem;
        a.sample_out = nullptr;
        a.theta = p.sample ? (p.fast ? theta_fast : theta_safe) : nullptr;
        a.keys = keys;
        a.key_stride = p.key_stride;
        a.pm = pm;
        a.pl = pl;
        a.pcnt = pcnt;
        a.preg = preg;
        a.cap = p.bounded ? p.cap : 0;
        if (p.bounded) {
            a.ovf_cap = p.ovf_cap;
            a.ovf_base = p.n_pieces * p.cap;
            a.rec_stride = p.rec_stride;
        }
        if ((st = hip_status(timed(prof, KIND_MAIN, s, [&] { return launch_mfma(a, 1, s); }))) != GENREC_OK) return st;
    } else {
        StreamArgs a{};
        a.H = H;
        a.E = E;
        a.B = B;
        a.D = D;
        a.M = M;
        a.mask = mask;
        a.mask_stride = mask_stride;
        if (p.sample) {
            a.n_items = p.n_sample;
            a.tile_stride = (int)p.stride;
            a.CH = p.pre.CH;
            a.P = p.pre.P;
            a.sample_out = sample;
            if ((st = hip_status(timed(prof, KIND_SAMPLE, s, [&] { return launch_stream(a, 0, f32, (int64_t)B * p.pre.P, s); }))) != GENREC_OK) return st;
            if ((st = hip_status(timed(prof, KIND_THRESHOLD, s, [&] { return launch_threshold(th, s); }))) != GENREC_OK) return st;
        }
        a.n_items = M;
        a.tile_stride = 1;
        a.CH = p.main.CH;
        a.P = p.main.P;
        a.sample_out = nullptr;
        a.theta = p.sample ? theta_safe : nullptr;
        a.keys = keys;
        a.pm = pm;
        a.pl = pl;
        a.pcnt = pcnt;
        a.preg = preg;
        if ((st = hip_status(timed(prof, KIND_MAIN, s, [&] { return launch_stream(a, 1, f32, (int64_t)B * p.main.P, s); }))) != GENREC_OK) return st;
    }
    MergeArgs m{};
    m.B = B;
    m.K = K;
    m.P = (int)p.rec_stride;
    m.piece_begin = nullptr;
    m.keys = keys;
    m.pm = pm;
    m.pl = pl;
    m.pcnt = pcnt;
    m.preg = preg;
    m.out_idx = out_idx;
    m.out_scores = out_scores;
    m.out_lse = out_lse;
    // clears the error words and, without a threshold pass, the rescue count
    m.clear_err = at<int64_t>(workspace, p.off_hdr);
    m.mode = p.fast ? 1 : 0;
    m.user_flag = uflag;
    m.tile_flag = tflag;
    m.rescued = rescued;
    m.theta_fast = theta_fast;
    m.theta_safe = theta_safe;
    m.safe_exact = p.safe_exact ? 1 : 0;
    m.small = p.merge_small ? 1 : 0;
    NarrowState* nst = nullptr;
    uint32_t* hist = nullptr;
    uint64_t* coll = nullptr;
    int* ccnt = nullptr;
    int* rc = nullptr;
    if (p.bounded) {
        nst = at<NarrowState>(workspace, p.off_nst);
        hist = at<uint32_t>(workspace, p.off_hist);
        coll = at<uint64_t>(workspace, p.off_coll);
        ccnt = at<int>(workspace, p.off_ccnt);
        rc = at<int>(workspace, p.off_rc);
        m.cap = p.cap;
        m.nst = nst;
        m.hist = hist;
        m.coll = coll;
        m.ccnt = ccnt;
        m.cbase = at<int64_t>(workspace, p.off_cbase);
        m.ccol = p.ccol;
        m.rc = rc;
        m.map = at<int>(workspace, p.off_map);
        m.H = H;
        m.hgat = at<uint8_t>(workspace, p.off_hgat);
        m.D = D;
        m.es = dtype == GENREC_F32 ? 4 : 2;
        m.ovf_cap = p.ovf_cap;
    }
    if ((st = hip_status(timed(prof, KIND_MERGE, s, [&] { return launch_merge(m, s); }))) != GENREC_OK) return st;
    if (!p.fast) return GENREC_OK;
    if (p.bounded) {
        // Rescue over bounded regions (users flagged by the merge for a full
        // overflow region or too few candidates): the merge gathered their
        // rows into the first user tiles; counting passes over those tiles
        // narrow each such user's bound on its ranking keys, a collect pass
        // stores the keys at or above it, and the merge ranks them.  With no
        // flagged user every launch exits at once.
        static_assert(kNarrowBinsPlan == kNarrowBins, "histogram bins of the plan and the kernels");
        a.cap = 0;
        a.rec_stride = 0;
        a.user_flag = nullptr;
        a.nst = nst;
        a.hist = hist;
        a.coll = coll;
        a.ccnt = ccnt;
        a.ccol = p.ccol;
        a.rc = rc;
        a.map = at<int>(workspace, p.off_map);
        a.H = at<uint16_t>(workspace, p.off_hgat);  // the flagged users' rows, gathered by the merge
        a.tile_flag = nullptr;
        NarrowArgs nr{};
        nr.nst = nst;
        nr.hist = hist;
        nr.rc = rc;
        nr.B = B;
        nr.K = K;
        nr.ccol = p.ccol;
        for (int pass = 0; pass < kNarrowPasses; ++pass) {
            a.collect = 0;
            if ((st = hip_status(timed(prof, KIND_RESCUE, s, [&] { return launch_mfma(a, 6, s); }))) != GENREC_OK)
                return st;
            if ((st = hip_status(timed(prof, KIND_RESCUE, s, [&] { return launch_narrow(nr, s); }))) != GENREC_OK)
                return st;
        }
        a.collect = 1;
        if ((st = hip_status(timed(prof, KIND_RESCUE, s, [&] { return launch_mfma(a, 6, s); }))) != GENREC_OK) return st;
        m.mode = 3;
        m.small = 0;
        m.clear_err = nullptr;
        return hip_status(timed(prof, KIND_RESCUE, s, [&] { return launch_merge(m, s); }));
    }
    // Rescue: users the fast threshold left short of K candidates are scored
    // again (their whole user tile) with the K-th sampled score -- or, when
    // the sampled scores came from a split reduction, with no threshold at all
    // (the regions hold every score) -- and merged; with no flagged user both
    // launches exit at once.
    a.theta = p.safe_exact ? theta_safe : nullptr;
    a.tile_flag = tflag;
    a.user_flag = uflag;
    if ((st = hip_status(timed(prof, KIND_RESCUE, s, [&] { return launch_mfma(a, 1, s); }))) != GENREC_OK) return st;
    m.mode = 2;
    m.small = 0;  // users past the K-th sampled score: many candidates
    m.clear_err = nullptr;
    return hip_status(timed(prof, KIND_RESCUE, s, [&] { return launch_merge(m, s); }));
}

}  // namespace

extern "C" {

int genrec_score_lse_topk_profiled(const void* H, const void* E, int dtype, int B, int D, int64_t M, int K,
                                   int32_t* out_idx, float* out_scores, float* out_lse, void* workspace,
                                   size_t workspace_bytes, void* stream, genrec_profiler* prof) {
    return score_dense(H, E, dtype, B, D, M, K, nullptr, 0, out_idx, out_scores, out_lse, workspace,
                       workspace_bytes, stream, prof);
}

}  // extern "C"

namespace {

// Workspace of the allocation-free entry point: one array per GPU (each
// device that loads the library holds its own copy until the process ends).
// In host code `scratch` is only a stand-in for the device symbol: kernels
// get the address hipGetSymbolAddress returns on each device, never this name.
static __device__ __align__(256) uint8_t scratch[GENREC_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The scratch's address on the current device, looked up once per device.
int scratch_on_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GENREC_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return GENREC_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return GENREC_OK;
}

}  // namespace

extern "C" {

int genrec_score_lse_topk_noalloc(const void* H, const void* E, int dtype, int B, int D, int64_t M, int K,
                                  int32_t* out_idx, float* out_scores, float* out_lse, void* stream) {
    int st = check_common(H, E, dtype, B, D, M, K, out_idx, out_scores, out_lse);
    if (st != GENREC_OK) return st;
    const DensePlan p = plan_dense_env(B, D, M, K, dtype);
    if (!p.ok) return GENREC_ERR_UNSUPPORTED;
    if (p.total > GENREC_NOALLOC_SCRATCH_BYTES) return GENREC_ERR_TOO_LARGE;
    void* ws = nullptr;
    if ((st = scratch_on_current_device(&ws)) != GENREC_OK) return st;
    return score_dense(H, E, dtype, B, D, M, K, nullptr, 0, out_idx, out_scores, out_lse, ws,
                       GENREC_NOALLOC_SCRATCH_BYTES, stream, nullptr);
}

int genrec_score_lse_topk_masked_profiled(const void* H, const void* E, int dtype, int B, int D, int64_t M, int K,
                                          const uint32_t* item_mask, int64_t mask_stride_words, int32_t* out_idx,
                                          float* out_scores, float* out_lse, void* workspace, size_t workspace_bytes,
                                          void* stream, genrec_profiler* prof) {
    if (!item_mask || !aligned(item_mask, 4)) return GENREC_ERR_INVALID_ARG;
    if (M > 0 && mask_stride_words != 0 && mask_stride_words < (M + 31) / 32) return GENREC_ERR_INVALID_ARG;
    if (mask_stride_words < 0) return GENREC_ERR_INVALID_ARG;
    return score_dense(H, E, dtype, B, D, M, K, item_mask, mask_stride_words, out_idx, out_scores, out_lse,
                       workspace, workspace_bytes, stream, prof);
}

int genrec_score_lse_topk_masked(const void* H, const void* E, int dtype, int B, int D, int64_t M, int K,
                                 const uint32_t* item_mask, int64_t mask_stride_words, int32_t* out_idx,
                                 float* out_scores, float* out_lse, void* workspace, size_t workspace_bytes,
                                 void* stream) {
    return genrec_score_lse_topk_masked_profiled(H, E, dtype, B, D, M, K, item_mask, mask_stride_words, out_idx,
                                                 out_scores, out_lse, workspace, workspace_bytes, stream, nullptr);
}

size_t genrec_score_candidates_topk_workspace(int B, int D, int64_t M, int64_t nnz, int K, int dtype) {
    static const float dummy[4] = {0, 0, 0, 0};
    if (check_common(dummy, dummy, dtype, B, D, M, K, (const int32_t*)dummy, dummy, dummy) != GENREC_OK)
        return 0;
    if (nnz < 0) return 0;
    return plan_cand(B, D, M, nnz, dtype).total;
}

int genrec_describe_cand_plan(int B, int D, int64_t M, int64_t nnz, int K, int dtype, char* buf, size_t len) {
    static const float dummy[4] = {0, 0, 0, 0};
    const int st = check_common(dummy, dummy, dtype, B, D, M, K, (const int32_t*)dummy, dummy, dummy);
    if (st != GENREC_OK) return st;
    if (nnz < 0 || !buf || len == 0) return GENREC_ERR_INVALID_ARG;
    const CandPlan p = plan_cand(B, D, M, nnz, dtype);
    if (!p.ok) return GENREC_ERR_UNSUPPORTED;
    snprintf(buf, len,
             "{\"hot\":%d,\"t_max\":%d,\"c_min\":%d,\"sample_every\":%d,\"n_pieces_max\":%lld,"
             "\"off_counts\":%lld,\"off_meta\":%lld,\"workspace\":%zu}",
             p.hot ? 1 : 0, p.t_max, p.c_min, kHotSample, (long long)p.n_pieces_max,
             p.hot ? (long long)p.off_cnt : -1LL, p.hot ? (long long)p.off_meta : -1LL, p.total);
    return GENREC_OK;
}

int genrec_score_candidates_topk(const void* H, const void* E, int dtype, const int64_t* cand_offsets,
                                 const int32_t* cand_ids, int B, int D, int64_t M, int64_t nnz, int K,
                                 int32_t* out_idx, float* out_scores, float* out_lse, void* workspace,
                                 size_t workspace_bytes, void* stream) {
    return genrec_score_candidates_topk_profiled(H, E, dtype, cand_offsets, cand_ids, B, D, M, nnz, K, out_idx,
                                                 out_scores, out_lse, workspace, workspace_bytes, stream, nullptr);
}

int genrec_score_candidates_topk_profiled(const void* H, const void* E, int dtype, const int64_t* cand_offsets,
                                          const int32_t* cand_ids, int B, int D, int64_t M, int64_t nnz, int K,
                                          int32_t* out_idx, float* out_scores, float* out_lse, void* workspace,
                                          size_t workspace_bytes, void* stream, genrec_profiler* prof) {
    int st = check_common(H, E, dtype, B, D, M, K, out_idx, out_scores, out_lse);
    if (st != GENREC_OK) return st;
    if (nnz < 0 || !cand_offsets || (nnz > 0 && !cand_ids)) return GENREC_ERR_INVALID_ARG;
    if (!aligned(cand_offsets, 8) || !aligned(cand_ids, 4)) return GENREC_ERR_INVALID_ARG;
    const CandPlan p = plan_cand(B, D, M, nnz, dtype);
    if (!p.ok) return GENREC_ERR_UNSUPPORTED;
    if (!workspace || workspace_bytes < p.total) return GENREC_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return GENREC_ERR_INVALID_ARG;
    hipStream_t s = (hipStream_t)stream;

    int64_t* err = at<int64_t>(workspace, p.off_hdr + kHdrErrIds);
    int* n_pieces = at<int>(workspace, p.off_hdr + kHdrPieces);
    int* piece_begin = at<int>(workspace, p.off_begin);
    CandPiece* table = at<CandPiece>(workspace, p.off_table);
    float* pm = at<float>(workspace, p.off_pm);
    float* pl = at<float>(workspace, p.off_pl);
    int* pcnt = at<int>(workspace, p.off_pcnt);
    int64_t* preg = at<int64_t>(workspace, p.off_preg);
    uint64_t* keys = at<uint64_t>(workspace, p.off_keys);

    CandPlanArgs c{};
    c.offsets = cand_offsets;
    c.B = B;
    c.nnz = nnz;
    c.piece_begin = piece_begin;
    c.table = table;
    c.n_pieces = n_pieces;
    c.err = err;
    if ((st = hip_status(timed(prof, KIND_PLAN, s, [&] { return launch_cand_plan(c, s); }))) != GENREC_OK) return st;

    if (p.hot) {
        // hot head: count, pick and gather the most-listed rows, then score
        // them densely for every user
        HotArgs h{};
        h.ids = cand_ids;
        h.nnz = nnz;
        h.E = (const uint16_t*)E;
        h.M = M;
        h.D = D;
        h.c_min = p.c_min;
        h.t_max = p.t_max;
        h.n_hblk = p.n_hblk;
        h.cnt = at<int>(workspace, p.off_cnt);
        h.hot_idx = at<int>(workspace, p.off_hot_idx);
        h.hist = at<int>(workspace, p.off_hist);
        h.meta = at<int>(workspace, p.off_meta);
        h.hblk = at<int>(workspace, p.off_hblk);
        h.hot_ids = at<int>(workspace, p.off_hot_ids);
        h.e_hot = at<uint16_t>(workspace, p.off_ehot);
        if ((st = hip_status(timed(prof, KIND_HOT_SELECT, s, [&] { return launch_hot_select(h, s); }))) != GENREC_OK)
            return st;
        MfmaArgs d{};
        d.H = (const uint16_t*)H;
        d.E = h.e_hot;
        d.B = B;
        d.D = D;
        d.M = p.t_max;
        d.n_tiles = p.t_max / kMfmaTileItems;
        d.tile_stride = 1;
        d.UT = p.hot_chunks.UT;
        d.P = p.hot_chunks.P;
        d.base = p.hot_chunks.base;
        d.rem = p.hot_chunks.rem;
        d.sample_out = at<float>(workspace, p.off_shot);
        d.live_rows = h.meta + 1;
        if ((st = hip_status(timed(prof, KIND_HOT_SCORE, s, [&] { return launch_mfma(d, 0, s); }))) != GENREC_OK) return st;
    }

    StreamArgs a{};
    a.H = H;
    a.E = E;
    a.B = B;
    a.D = D;
    a.M = M;
    a.hot_idx = p.hot ? at<int>(workspace, p.off_hot_idx) : nullptr;
    a.s_hot = p.hot ? at<float>(workspace, p.off_shot) : nullptr;
    a.t_hot = p.t_max;
    a.ids = cand_ids;
    a.n_pieces = n_pieces;
    a.table = table;
    a.theta = nullptr;
    a.keys = keys;
    a.pm = pm;
    a.pl = pl;
    a.pcnt = pcnt;
    a.preg = preg;
    a.err = err;
    if ((st = hip_status(timed(prof, KIND_MAIN, s, [&] { return launch_stream(a, 2, dtype == GENREC_F32, p.n_pieces_max, s); }))) != GENREC_OK)
        return st;

    MergeArgs m{};
    m.B = B;
    m.K = K;
    m.P = 0;
    m.piece_begin = piece_begin;
    m.keys = keys;
    m.pm = pm;
    m.pl = pl;
    m.pcnt = pcnt;
    m.preg = preg;
    m.out_idx = out_idx;
    m.out_scores = out_scores;
    m.out_lse = out_lse;
    m.clear_err = nullptr;
    m.mode = 0;
    m.small = nnz <= (int64_t)kMergeSmallGather * B ? 1 : 0;  // lists of up to ~2,048 entries on average
    return hip_status(timed(prof, KIND_MERGE, s, [&] { return launch_merge(m, s); }));
}

int genrec_get_device_errors(const void* workspace, void* stream, int64_t* n_bad_ids, int64_t* n_bad_offsets) {
    if (!workspace) return GENREC_ERR_INVALID_ARG;
    int64_t h[2] = {0, 0};
    hipStream_t s = (hipStream_t)stream;
    if (hipMemcpyAsync(h, workspace, sizeof(h), hipMemcpyDeviceToHost, s) != hipSuccess) return GENREC_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return GENREC_ERR_HIP;
    if (n_bad_ids) *n_bad_ids = h[0];
    if (n_bad_offsets) *n_bad_offsets = h[1];
    return GENREC_OK;
}

size_t genrec_topk_rows_workspace(int R, int64_t N, int K) {
    if (R <= 0 || N <= 0 || K <= 0 || K > GENREC_KMAX || N >= ((int64_t)1 << 31)) return 0;
    return plan_topk(R, N, K).workspace;
}

int genrec_topk_rows(const float* scores, int R, int64_t N, int64_t ld, int K, int32_t* out_idx,
                     float* out_scores, void* workspace, size_t workspace_bytes, void* stream) {
    if (R <= 0 || N <= 0 || K <= 0 || ld < N) return GENREC_ERR_INVALID_ARG;
    if (!scores || !out_idx || !out_scores) return GENREC_ERR_INVALID_ARG;
    if (!aligned(scores, 4) || !aligned(out_idx, 4) || !aligned(out_scores, 4)) return GENREC_ERR_INVALID_ARG;
    if (K > GENREC_KMAX) return GENREC_ERR_UNSUPPORTED;
    if (N >= ((int64_t)1 << 31)) return GENREC_ERR_UNSUPPORTED;
    const TopkPlan p = plan_topk(R, N, K);
    if (!p.ok) return GENREC_ERR_UNSUPPORTED;
    if (p.workspace > 0 && (!workspace || workspace_bytes < p.workspace)) return GENREC_ERR_WORKSPACE;
    if (p.workspace > 0 && !aligned(workspace, 8)) return GENREC_ERR_INVALID_ARG;
    TopkRowsArgs a{};
    a.scores = scores;
    a.R = R;
    a.N = N;
    a.ld = ld;
    a.K = K;
    a.out_idx = out_idx;
    a.out_scores = out_scores;
    a.C = p.C;
    a.nchunk = p.nchunk;
    a.part = (uint64_t*)workspace;
    a.reg = p.filt ? 3 : (p.row ? 2 : (p.reg ? 1 : 0));
    if (p.filt) {
        a.sj = p.filt;
        a.tthr = (uint32_t*)((char*)workspace + p.off_thr);
        a.tcnt = (int*)((char*)workspace + p.off_cnt);
    }
    return hip_status(launch_topk_rows(a, (hipStream_t)stream));
}

// ---------------------------------------------------------------------------
// Cross-entropy over the catalog
// ---------------------------------------------------------------------------
namespace {

CeArgs ce_args(const void* H, const void* E, int B, int D, int64_t M, const int32_t* labels, const float* weights,
               void* workspace, const CePlan& p) {
    CeArgs c{};
    c.H = (const uint16_t*)H;
    c.E = (const uint16_t*)E;
    c.B = B;
    c.D = D;
    c.M = M;
    c.labels = labels;
    c.weights = weights;
    c.w_eff = at<float>(workspace, p.off_w);
    c.err = at<int64_t>(workspace, p.off_hdr);
    return c;
}

}  // namespace

size_t genrec_ce_forward_workspace(int B, int D, int64_t M) {
    if (B <= 0 || D <= 0 || M <= 0 || M >= ((int64_t)1 << 31) || D > GENREC_DMAX) return 0;
    return plan_ce(B, D, M).fwd_total;  // 0 when unsupported
}

size_t genrec_ce_backward_workspace(int B, int D, int64_t M) {
    if (B <= 0 || D <= 0 || M <= 0 || M >= ((int64_t)1 << 31) || D > GENREC_DMAX) return 0;
    const CePlan p = plan_ce(B, D, M);
    return p.ok ? p.bwd_total : 0;
}

int genrec_describe_ce_plan(int B, int D, int64_t M, char* buf, size_t len) {
    if (B <= 0 || D <= 0 || M <= 0 || !buf || len == 0) return GENREC_ERR_INVALID_ARG;
    if (M >= ((int64_t)1 << 31) || D > GENREC_DMAX) return GENREC_ERR_UNSUPPORTED;
    const CePlan p = plan_ce(B, D, M);
    if (!p.ok) return GENREC_ERR_UNSUPPORTED;
    snprintf(buf, len,
             "{\"chunk\":%lld,\"Mcp\":%lld,\"n_chunks\":%lld,\"Bp\":%lld,\"splits\":%d,"
             "\"depth_h\":%lld,\"depth_e\":%lld,\"workspace\":%zu}",
             (long long)p.chunk, (long long)p.Mcp, (long long)p.n_chunks, (long long)p.Bp, p.splits,
             (long long)ce_depth_h(p), (long long)ce_depth_e(p), p.bwd_total);
    return GENREC_OK;
}

int genrec_ce_forward_profiled(const void* H, const void* E, int B, int D, int64_t M, const int32_t* labels,
                               const float* weights, float* out_loss, float* out_lse, void* workspace,
                               size_t workspace_bytes, void* stream, genrec_profiler* prof) {
    int st = check_ce(H, E, B, D, M, labels, weights);
    if (st != GENREC_OK) return st;
    if (!out_loss || !out_lse || !aligned(out_loss, 4) || !aligned(out_lse, 4)) return GENREC_ERR_INVALID_ARG;
    const CePlan p = plan_ce(B, D, M);
    if (!p.fwd_ok) return GENREC_ERR_UNSUPPORTED;
    if (!workspace || workspace_bytes < p.fwd_total) return GENREC_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return GENREC_ERR_INVALID_ARG;
    hipStream_t s = (hipStream_t)stream;
    CeArgs c = ce_args(H, E, B, D, M, labels, weights, workspace, p);
    if ((st = hip_status(timed(prof, KIND_CE_SMALL, s, [&] { return launch_ce_prep(c, s); }))) != GENREC_OK) return st;
    // logsumexp pieces of every (user, catalog chunk, lane group); no candidates
    MfmaArgs a{};
    a.H = (const uint16_t*)H;
    a.E = (const uint16_t*)E;
    a.B = B;
    a.D = D;
    a.M = M;
    a.n_tiles = (int)ceil_div(M, kMfmaTileItems);
    a.tile_stride = 1;
    a.UT = p.main.UT;
    a.P = p.main.P;
    a.base = p.main.base;
    a.rem = p.main.rem;
    a.no_cand = 1;
    a.pm = at<float>(workspace, p.off_pm);
    a.pl = at<float>(workspace, p.off_pl);
    a.pcnt = at<int>(workspace, p.off_pcnt);
    a.preg = at<int64_t>(workspace, p.off_preg);
    if ((st = hip_status(timed(prof, KIND_MAIN, s, [&] { return launch_mfma(a, 1, s); }))) != GENREC_OK) return st;
    c.pm = a.pm;
    c.pl = a.pl;
    c.P = p.main.P * 4;
    c.out_loss = out_loss;
    c.out_lse = out_lse;
    return hip_status(timed(prof, KIND_CE_SMALL, s, [&] { return launch_ce_finish(c, s); }));
}

int genrec_ce_forward(const void* H, const void* E, int B, int D, int64_t M, const int32_t* labels,
                      const float* weights, float* out_loss, float* out_lse, void* workspace, size_t workspace_bytes,
                      void* stream) {
    return genrec_ce_forward_profiled(H, E, B, D, M, labels, weights, out_loss, out_lse, workspace, workspace_bytes,
                                      stream, nullptr);
}

int genrec_ce_backward_profiled(const void* H, const void* E, int B, int D, int64_t M, const int32_t* labels,
                                const float* weights, const float* lse, float* out_dH, void* out_dE, int de_dtype,
                                void* workspace, size_t workspace_bytes, void* stream, genrec_profiler* prof) {
    int st = check_ce(H, E, B, D, M, labels, weights);
    if (st != GENREC_OK) return st;
    if (!lse || !out_dH || !out_dE || !aligned(lse, 4) || !aligned(out_dH, 4) || !aligned(out_dE, 4))
        return GENREC_ERR_INVALID_ARG;
    if (de_dtype != GENREC_F32 && de_dtype != GENREC_BF16) return GENREC_ERR_INVALID_ARG;
    const CePlan p = plan_ce(B, D, M);
    if (!p.ok) return GENREC_ERR_UNSUPPORTED;
    if (!workspace || workspace_bytes < p.bwd_total) return GENREC_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return GENREC_ERR_INVALID_ARG;
    hipStream_t s = (hipStream_t)stream;
    CeArgs c = ce_args(H, E, B, D, M, labels, weights, workspace, p);
    if ((st = hip_status(timed(prof, KIND_CE_SMALL, s, [&] { return launch_ce_prep(c, s); }))) != GENREC_OK) return st;
    uint16_t* ht = at<uint16_t>(workspace, p.off_ht);
    uint16_t* et = at<uint16_t>(workspace, p.off_et);
    uint16_t* grows = at<uint16_t>(workspace, p.off_grows);
    uint16_t* gcols = at<uint16_t>(workspace, p.off_gcols);
    float* dhp = at<float>(workspace, p.off_dhp);
    // H^T [D][Bp], users past B zero: the user side of the dE product
    TransposeArgs th{};
    th.in = (const uint16_t*)H;
    th.R = B;
    th.C = D;
    th.ld_in = D;
    th.out = ht;
    th.ld_out = p.Bp;
    if ((st = hip_status(timed(prof, KIND_TRANSPOSE, s, [&] { return launch_transpose(th, s); }))) != GENREC_OK)
        return st;
    for (int64_t ci = 0; ci < p.n_chunks; ++ci) {
        const int64_t r0 = ci * p.chunk;
        const int64_t rows = std::min<int64_t>(p.chunk, M - r0);
        const int64_t mcp = ceil_div(rows, kMfmaTileItems) * kMfmaTileItems;
        const int ntl = (int)(mcp / kMfmaTileItems);
        const uint16_t* Ec = (const uint16_t*)E + r0 * D;
        // E chunk^T [D][mcp] k-blocked, rows past the chunk zero: the item side of dH
        TransposeArgs te{};
        te.in = Ec;
        te.R = rows;
        te.C = D;
        te.ld_in = D;
        te.out = et;
        te.ld_out = mcp;
        te.blocked = 1;
        if ((st = hip_status(timed(prof, KIND_TRANSPOSE, s, [&] { return launch_transpose(te, s); }))) != GENREC_OK)
            return st;
        // G = w (softmax - target) of the chunk: [Bp][mcp] k-blocked and [mcp][Bp]
        MfmaArgs g{};
        g.H = (const uint16_t*)H;
        g.E = Ec;
        g.B = B;
        g.D = D;
        g.M = rows;
        g.n_tiles = ntl;
        g.tile_stride = 1;
        const Chunking cg = chunk_mfma(B, ntl);
        g.UT = cg.UT;
        g.P = cg.P;
        g.base = cg.base;
        g.rem = cg.rem;
        g.lse = lse;
        g.wgt = c.w_eff;
        g.labels = labels;
        g.item0 = r0;
        g.g_rows = grows;
        g.g_cols = gcols;
        g.ld_g = p.Bp * kMfmaBlockK;
        g.ld_gt = p.Bp;
        g.gt_users = (int)p.Bp;
        if ((st = hip_status(timed(prof, KIND_GRAD_TILES, s, [&] { return launch_mfma_split(g, 3, 1, s); }))) !=
            GENREC_OK)
            return st;
        // dE rows of the chunk = G^T H: rows = items, columns = D, reduction = Bp users
        MfmaArgs de{};
        de.E = gcols;
        de.H = ht;
        de.M = rows;
        de.B = D;
        de.D = (int)p.Bp;
        de.n_tiles = ntl;
        de.tile_stride = 1;
        const Chunking ce = chunk_mfma(D, ntl);
        de.UT = ce.UT;
        de.P = ce.P;
        de.base = ce.base;
        de.rem = ce.rem;
        de.c_bf16 = de_dtype == GENREC_BF16 ? 1 : 0;
        de.c_out = de.c_bf16 ? (float*)((uint16_t*)out_dE + r0 * D) : (float*)out_dE + r0 * D;
        de.ldc = D;
        if ((st = hip_status(timed(prof, KIND_GRAD_E, s, [&] { return launch_mfma_split(de, 4, 1, s); }))) !=
            GENREC_OK)
            return st;
        // dH += G E_chunk: rows = D, columns = users, reduction = the chunk's
        // items in `splits` parts, each into its own partial sum; both
        // operands k-blocked
        MfmaArgs dh{};
        dh.E = et;
        dh.H = grows;
        dh.M = D;
        dh.B = B;
        dh.D = (int)(mcp / p.splits);
        dh.k_split = mcp / p.splits;
        dh.blk_e = (int64_t)D * kMfmaBlockK;
        dh.blk_h = p.Bp * kMfmaBlockK;
        dh.e_elems = mcp * D;
        dh.h_elems = mcp * p.Bp;
        dh.n_tiles = (int)ceil_div(D, kMfmaTileItems);
        dh.tile_stride = 1;
        const Chunking chh = chunk_mfma(B, dh.n_tiles);
        dh.UT = chh.UT;
        dh.P = chh.P;
        dh.base = chh.base;
        dh.rem = chh.rem;
        dh.c_out = dhp;
        dh.ldc = D;
        dh.c_split = (int64_t)B * D;
        dh.c_trans = 1;
        dh.c_accum = ci > 0 ? 1 : 0;
        if ((st = hip_status(timed(prof, KIND_GRAD_H, s, [&] { return launch_mfma_split(dh, 5, p.splits, s); }))) !=
            GENREC_OK)
            return st;
    }
    return hip_status(timed(prof, KIND_CE_SMALL, s, [&] {
        return launch_sum_splits(dhp, p.splits, (int64_t)B * D, (int64_t)B * D, out_dH, s);
    }));
}

int genrec_ce_backward(const void* H, const void* E, int B, int D, int64_t M, const int32_t* labels,
                       const float* weights, const float* lse, float* out_dH, void* out_dE, int de_dtype,
                       void* workspace, size_t workspace_bytes, void* stream) {
    return genrec_ce_backward_profiled(H, E, B, D, M, labels, weights, lse, out_dH, out_dE, de_dtype, workspace,
                                       workspace_bytes, stream, nullptr);
}

int genrec_get_rescued_users(const void* workspace, void* stream, int64_t* n_rescued) {
    if (!workspace || !n_rescued) return GENREC_ERR_INVALID_ARG;
    int64_t h = 0;
    hipStream_t s = (hipStream_t)stream;
    if (hipMemcpyAsync(&h, (const uint8_t*)workspace + kHdrRescued, sizeof(h), hipMemcpyDeviceToHost, s) != hipSuccess)
        return GENREC_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return GENREC_ERR_HIP;
    *n_rescued = h;
    return GENREC_OK;
}

}  // extern "C"
