// Ranking-head kernels for gfx950 (CDNA4, MI355X).
//
// The operation (GenRec concept page, scoring formula s = E^T h; GenRec
// explainer page, "overall picture": softmax over the catalog or candidate set,
// then descending sort) is split into stream-ordered kernels:
//
//  mfma_score_kernel   S-tile = E-tile . H-tile^T on bf16 MFMA (32x32x16),
//                      E and H tiles staged through LDS; the epilogue keeps an
//                      online (max, sum-exp) per user and appends every score
//                      that reaches the user's threshold to a candidate region.
//                      The score matrix itself is never written out.
//  stream_score_kernel the same epilogue for few users or per-user candidate
//                      lists: VALU dot products (v_dot2_f32_bf16 / fp32 FMA)
//                      over gathered rows, one 16-byte load per lane per row
//                      step, eight rows in flight per wave.
//  threshold_kernel    per user, the K-th (and a smaller rank's) largest score
//                      of a sample of whole catalog tiles: lower bounds of the
//                      catalog's order statistics, the candidate thresholds of
//                      the main pass and of the rescue pass.
//  merge_kernel        per user, lse from the per-piece (max, sum-exp) pairs
//                      and the exact top-K of the candidates (range-narrowing
//                      histogram select, then rank placement or wave sorts and
//                      a rank merge), written sorted.
//  cand_plan_kernel    CSR offsets -> work list of fixed-size list pieces.
//  hot_*_kernel        candidate lists: the most-listed rows, scored densely.
//  topk_chunk_kernel,  batched top-K of dense score rows (a beam step) by
//  topk_merge_rows_kernel  histogram narrowing per chunk, then per row.
//  topk_seg_kernel,    the same for long rows with many segments: register-
//  topk_rowmerge_kernel  resident radix selection per segment, then per row.
//  mfma_score_kernel   modes 3-5 and ce_*, transpose, sum_splits kernels: the
//                      catalog cross-entropy (GenRec explainer page, "two
//                      objectives and reward-weighted ranking"): forward = the
//                      logsumexp pass plus the label's score; backward = per
//                      catalog chunk the softmax-minus-target tiles G and the
//                      products dE = G^T H and dH = G E.
#include <float.h>

#include "device_common.hpp"
#include "launch.hpp"
#include "mfma_layout.hpp"
#include "plan.hpp"

namespace genrec {

// ---------------------------------------------------------------------------
// Dense MFMA path
// ---------------------------------------------------------------------------

// s_waitcnt vmcnt(n) with expcnt / lgkmcnt left alone (gfx9 encoding), and
// the same with lgkmcnt(0) as well (every LDS read of the wave completed).
#define MF_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt((((n) >> 4) << 14) | 0x0F70 | ((n) & 15))
#define MF_WAIT_VMCNT_LDS(n) __builtin_amdgcn_s_waitcnt((((n) >> 4) << 14) | 0x0070 | ((n) & 15))

// F32: fp32 operands on the fp32 matrix cores (v_mfma_f32_32x32x2_f32).  The
// staged rows are 64 bytes either way -- 32 bf16 or 16 fp32 of the reduction
// per k-step -- so the DMA, the LDS layout and the fragment reads are the same;
// a 16-byte fragment holds 4 fp32 (not 8 bf16) and feeds four MFMAs of depth
// 2 instead of one of depth 16 (each lane half takes its own 4 k values, the
// same k for both operands: a fixed reordering of the reduction).  The
// accumulator layout, hence the epilogue, is the same.
template <int MODE, bool KTAIL, bool MASKED, bool F32 = false>
__global__ __launch_bounds__(MF_NT, 1) void mfma_score_kernel(MfmaArgs a) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[MF_NS][MF_STAGE];
    static_assert(!F32 || MODE <= 1 || MODE == 6, "fp32 operands: the dense sample, main and rescue passes only");
    constexpr int ES = F32 ? 4 : 2;         // bytes per element
    constexpr int KE = MF_ROWB / ES;        // reduction elements per k-step (32 bf16 / 16 fp32)
    constexpr int CE = 16 / ES;             // elements per 16-byte k-chunk

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wi = w & 1, wu = w >> 1;  // wave tile: items wi*128 .. +128, users wu*64 .. +64

    // Blocks are dealt round-robin to the 8 XCDs; renumber them so that the
    // user tiles sharing one catalog chunk sit on one XCD (one L2) together.
    const int nblk = gridDim.x;
    int L = blockIdx.x;
    if ((nblk & 7) == 0) L = (blockIdx.x & 7) * (nblk >> 3) + (blockIdx.x >> 3);
    // Bounded regions' rescue (mode 6): the flagged users' rows were gathered
    // into the first nut = ceil(rc[1] / 256) user tiles, and the grid's blocks
    // split the catalog into grid / nut chunks per tile (a handful of flagged
    // users keeps every CU busy); the counting passes stop once none counts.
    int nut = a.UT, Pd = a.P, base = a.base, rem = a.rem;
    if (MODE == 6) {
        const int nf = a.rc[1];
        if (nf == 0 || (!a.collect && a.rc[0] == 0)) return;
        nut = (nf + MF_TU - 1) / MF_TU;
        Pd = max(1, min(a.n_tiles, nblk / nut));
        base = a.n_tiles / Pd;
        rem = a.n_tiles - base * Pd;
    }
    const int c = L / nut, ut = L - c * nut;
    if (MODE == 6 && c >= Pd) return;
    // rescue pass: user tiles without a flagged user have nothing to redo
    if (MODE == 1 && a.tile_flag != nullptr && a.tile_flag[ut] == 0) return;
    const int tile0 = c * base + min(c, rem);  // first pass-tile of this chunk
    const int ntiles = base + (c < rem ? 1 : 0);
    // dense pass over a partly filled catalog: chunks past its live rows are idle
    if (MODE == 0 && a.live_rows != nullptr && (int64_t)tile0 * a.tile_stride * MF_TI >= *a.live_rows) return;
    const int u0 = ut * MF_TU;
    const int nk = (a.D + KE - 1) / KE;
    const int D = a.D;
    // row stride of both operands, and where this block's share of the
    // reduction starts in every row (grid y splits it)
    // mode 5: k-blocked operands, rows of 32 reduction elements
    constexpr bool BLKD = MODE == 5;
    const int64_t ldr = BLKD ? (int64_t)MF_BK : (a.ld != 0 ? a.ld : (int64_t)D);
    const int64_t kofs = (int64_t)blockIdx.y * a.k_split;
    const int64_t kofs_e = BLKD ? kofs / MF_BK * a.blk_e : kofs;  // element offsets of the split
    const int64_t kofs_h = BLKD ? kofs / MF_BK * a.blk_h : kofs;

    // Pass-tile t holds catalog rows [256 c, 256 c + 256) clipped to M, c = t
    // (G = 1) or, for the sample (G > 1), one full tile of the window [t G, t G + G).
    const int64_t full_tiles = a.M / MF_TI;
    auto tile_item0 = [&](int t) -> int64_t { return mf_sample_tile(t, a.tile_stride, full_tiles) * MF_TI; };
    auto tile_valid = [&](int t) -> int {
        const int64_t left = a.M - tile_item0(t);
        return left < MF_TI ? (int)left : MF_TI;
    };

    // ---- DMA (geometry in mfma_layout.hpp) --------------------------------
    // buffer_load ... lds through a buffer resource per operand (wave-uniform,
    // SGPRs); each op of a lane reads at a fixed 32-bit byte offset plus the
    // k-step's scalar offset.  The resource's record count ends at the last
    // valid row of the tile (or of the batch), so rows past the end of a
    // partial tile read as zeros without any clamping; k-chunks past D read
    // the next row or zeros, and the fragment reads replace them by zeros.
    const int wsu = __builtin_amdgcn_readfirstlane(w);  // wave index, provably uniform
    const int64_t row_bytes = ldr * ES;
    uint32_t voff[MF_DMA];
#pragma unroll
    for (int j = 0; j < MF_DMA; ++j) voff[j] = (uint32_t)mf_dma_voff_bytes(w, lane, j, row_bytes);
    // The user tile's resource is fixed; the catalog tile's is rebuilt when the
    // DMA moves to a new tile.  k0 rides in the scalar offset, so rows past the
    // end (and k-chunks past D on the last row) fall outside the record count.
    const int h_rows = a.B - u0 < MF_TU ? a.B - u0 : MF_TU;
    const int64_t h_off = (int64_t)u0 * (BLKD ? MF_BK : ldr) + kofs_h;  // elements
    const __amdgpu_buffer_rsrc_t hr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((const uint8_t*)a.H + h_off * ES), (short)0, (int)(BLKD ? (a.h_elems - h_off) * 2 : h_rows * row_bytes),
        0x00020000);
    __amdgpu_buffer_rsrc_t er;
    auto e_rsrc = [&](int t) {
        const int64_t e_off = tile_item0(t) * (BLKD ? MF_BK : ldr) + kofs_e;
        er = __builtin_amdgcn_make_buffer_rsrc((void*)((const uint8_t*)a.E + e_off * ES), (short)0,
                                               (int)(BLKD ? (a.e_elems - e_off) * 2 : tile_valid(t) * row_bytes),
                                               0x00020000);
    };

    // DMA op j of both operands for the stage at k0 (1 KiB per op per wave).
    auto dma_op = [&](int stg, int k0, int j) {
        uint8_t* sE = smem[stg] + mf_dma_lds_byte(wsu, 0, 0);
        uint8_t* sH = smem[stg] + MF_TI * MF_ROWB + mf_dma_lds_byte(wsu, 0, 0);
        const int soff_e = BLKD ? (int)(k0 / MF_BK * a.blk_e * 2) : k0 * ES;
        const int soff_h = BLKD ? (int)(k0 / MF_BK * a.blk_h * 2) : k0 * ES;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(er, (__attribute__((address_space(3))) void*)(sE + j * MF_NW * 1024),
                                                 16, (int)voff[j], soff_e, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(hr, (__attribute__((address_space(3))) void*)(sH + j * MF_NW * 1024),
                                                 16, (int)voff[j], soff_h, 0, 0);
    };

    f32x16_t acc[4][MF_UB];
    // MFMA operand fragments of one 16-deep k-slice: lane holds 8 consecutive
    // k of row (lane & 31) of each 32-row block, k-chunk (lane >> 5).
    struct Frag {
        bf16x8_t a[4], b[MF_UB];
    };
    auto load_frag = [&](Frag& f, int stg, int ks, int k0) {
        const uint8_t* sE = smem[stg];
        const uint8_t* sH = smem[stg] + MF_TI * MF_ROWB;
        const int chunk = ks * 2 + (lane >> 5);
        // k past D: both fragments zero.  The staged chunks there hold the next
        // row's first elements (or zeros), which need not be finite: the hot
        // rows of a candidate call are gathered into a workspace whose rows
        // past the live ones are stale, and NaN times zero is NaN.
        const bool kin = !KTAIL || k0 + chunk * CE < D;
#pragma unroll
        for (int ib = 0; ib < 4; ++ib) {
            f.a[ib] = *(const bf16x8_t*)(sE + mf_frag_lds_byte(wi * 128 + ib * 32 + (lane & 31), chunk));
            if (!kin) f.a[ib] = bf16x8_t{};
        }
#pragma unroll
        for (int ub = 0; ub < MF_UB; ++ub) {
            f.b[ub] = *(const bf16x8_t*)(sH + mf_frag_lds_byte(wu * MF_WU + ub * 32 + (lane & 31), chunk));
            if (!kin) f.b[ub] = bf16x8_t{};
        }
    };
    auto mma = [&](const Frag& f) {
#pragma unroll
        for (int ib = 0; ib < 4; ++ib)
#pragma unroll
            for (int ub = 0; ub < MF_UB; ++ub) {
                if constexpr (F32) {
                    const f32x4_t fa = __builtin_bit_cast(f32x4_t, f.a[ib]), fb = __builtin_bit_cast(f32x4_t, f.b[ub]);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        acc[ib][ub] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[e], fb[e], acc[ib][ub], 0, 0, 0);
                } else {
                    acc[ib][ub] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[ib], f.b[ub], acc[ib][ub], 0, 0, 0);
                }
            }
    };

    // ---- epilogue state ---------------------------------------------------
    // Lane owns user column (lane & 31) of each 32-wide user block ub; the
    // accumulator element r of block (ib, ub) is tile row
    //   wi*128 + ib*32 + (r/4)*8 + (lane/32)*4 + r%4.
    // Per (user, chunk) the four lane groups g = (wi, lane/32) that share a
    // user each own a quarter of the chunk's candidate region and a piece
    // record: no atomics, no cross-lane combine.
    const int g = wi * 2 + (lane >> 5);
    const int lrow0 = wi * 128 + (lane >> 5) * 4;
    const int64_t chunk_item0 = tile_item0(tile0);  // (mode 1: G = 1)
    const int64_t n_pass = (int64_t)a.n_tiles * MF_TI;  // mode 0: row length of sample_out
    float m_[MF_UB], l_[MF_UB], th_[MF_UB];
    int cnt_[MF_UB];
    uint64_t nlo_[MF_UB];  // mode 6: the user's key bound, bin shift and whether it takes part
    int nsh_[MF_UB];
    bool nin_[MF_UB];
    int mu_[MF_UB];  // mode 6: the user whose gathered row this column holds (B: none)
#pragma unroll
    for (int ub = 0; ub < MF_UB; ++ub) {
        const int u = u0 + wu * MF_WU + ub * 32 + (lane & 31);
        m_[ub] = -INFINITY;
        l_[ub] = 0.f;
        cnt_[ub] = 0;
        float t = -FLT_MAX;
        if (MODE == 1 && a.theta != nullptr && u < a.B) t = fmaxf(a.theta[u], -FLT_MAX);
        // users past B never append, nor, in the rescue pass, unflagged users
        const bool active = u < a.B && (a.user_flag == nullptr || a.user_flag[u] != 0);
        th_[ub] = active && !a.no_cand ? t : INFINITY;
        if (MODE == 6) {
            const int mu = u < a.rc[1] ? a.map[u] : a.B;
            const bool in = mu < a.B && a.nst[mu].status == (a.collect ? 2 : 1);
            nlo_[ub] = in ? a.nst[mu].lo : ~0ull;
            nsh_[ub] = in ? a.nst[mu].shift : 0;
            nin_[ub] = in;
            mu_[ub] = mu;
        }
    }

    auto epilogue = [&](int t) {
        const int lim = tile_valid(t);  // valid tile rows (mode 0 stores only these)
        const int64_t j0 = tile_item0(t);
        // Rows past the end of a partial tile hold -inf (set before the call):
        // they add nothing to the sum and never pass a threshold.  Each 32 x 32 block (16
        // scores per lane) is finished before the next is read, fenced by a
        // scheduling barrier, which keeps the live register set small.
#pragma unroll
        for (int ub = 0; ub < MF_UB; ++ub) {
            // (mode 6: the user of the gathered row in this column)
            const int u = MODE == 6 ? mu_[ub] : u0 + wu * MF_WU + ub * 32 + (lane & 31);
            // Item mask: the 32 rows of block ib that this lane group covers
            // (rows wi*128 + ib*32 + 4*(lane/32) + 8q + e) lie in one mask word;
            // masked items score -inf (nothing to the sum, never a candidate).
            auto mask_word = [&](int ib) -> uint32_t {
                if (!MASKED || u >= a.B) return 0xFFFFFFFFu;
                const int64_t w0 = j0 + wi * 128 + ib * 32;  // multiple of 32
                if (w0 >= a.M) return 0u;
                return a.mask[(int64_t)u * a.mask_stride + (w0 >> 5)];
            };
            const int mbit0 = (lane >> 5) * 4;
            if (MODE == 3) {
                // g = w (softmax - target) of the scores, rounded to bf16, into
                // both layouts; zeros past the valid rows and past the users.
                // The user index is made opaque so that the compiler rebuilds
                // the store addresses per tile instead of keeping 32 of them
                // live (and spilled) across the whole tile loop.
                int uo = u;
                asm volatile("" : "+v"(uo));
                const int u = uo;
                if (u < a.gt_users) {
                    const bool real = u < a.B;
                    const float lse_u = real ? a.lse[u] : 0.f;
                    const float w_u = real ? a.wgt[u] : 0.f;
                    // row of the user's label within this tile (outside [0, 256): none)
                    const int64_t y_row = real ? (int64_t)a.labels[u] - a.item0 - j0 : -1;
#pragma unroll
                    for (int ib = 0; ib < 4; ++ib)
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const int jq = lrow0 + ib * 32 + q * 8;
                            uint16_t gb[4];
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                const float p = fast_exp2((acc[ib][ub][4 * q + e] - lse_u) * kLog2e);
                                const float gv = w_u * (p - (jq + e == y_row ? 1.f : 0.f));
                                gb[e] = bf16_bits(real && jq + e < lim ? gv : 0.f);
                            }
                            const int64_t jl = j0 + jq;  // k-blocked: 32 items of 32 users' rows per 2 KiB
                            *(uint2*)(a.g_rows + (jl >> 5) * a.ld_g + (int64_t)u * MF_BK + (jl & 31)) =
                                make_uint2(gb[0] | ((uint32_t)gb[1] << 16), gb[2] | ((uint32_t)gb[3] << 16));
                            uint16_t* gc = a.g_cols + (j0 + jq) * a.ld_gt + u;
#pragma unroll
                            for (int e = 0; e < 4; ++e) gc[e * a.ld_gt] = gb[e];
                        }
                }
                continue;
            }
            if (MODE == 4 || MODE == 5) {
                // plain product: the tile's valid rows of column u, fp32
                if (u < a.B) {
                    float* cz = a.c_out + (int64_t)blockIdx.y * a.c_split;
#pragma unroll
                    for (int ib = 0; ib < 4; ++ib)
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const int jq = lrow0 + ib * 32 + q * 8;
                            const int64_t row = j0 + jq;
                            if (a.c_trans) {  // [u][row .. row + 3]: consecutive
                                float* o = cz + (int64_t)u * a.ldc + row;
                                if (jq + 3 < lim) {
                                    float4 v = make_float4(acc[ib][ub][4 * q], acc[ib][ub][4 * q + 1],
                                                           acc[ib][ub][4 * q + 2], acc[ib][ub][4 * q + 3]);
                                    if (a.c_accum) {
                                        const float4 o4 = *(const float4*)o;
                                        v.x += o4.x;
                                        v.y += o4.y;
                                        v.z += o4.z;
                                        v.w += o4.w;
                                    }
                                    *(float4*)o = v;
                                } else {
#pragma unroll
                                    for (int e = 0; e < 4; ++e)
                                        if (jq + e < lim) o[e] = acc[ib][ub][4 * q + e] + (a.c_accum ? o[e] : 0.f);
                                }
                            } else if (a.c_bf16) {  // [row + e][u], bf16
                                // an output written once and not read back by this
                                // call: non-temporal (streaming) stores, which keep
                                // the operands in the caches (the dE product: -12%)
#pragma unroll
                                for (int e = 0; e < 4; ++e)
                                    if (jq + e < lim)
                                        __builtin_nontemporal_store(bf16_bits(acc[ib][ub][4 * q + e]),
                                                                    (uint16_t*)a.c_out + (row + e) * a.ldc + u);
                            } else {  // [row + e][u]: a row segment across the lanes
#pragma unroll
                                for (int e = 0; e < 4; ++e)
                                    if (jq + e < lim) {
                                        float* o = cz + (row + e) * a.ldc + u;
                                        if (a.c_accum) *o = acc[ib][ub][4 * q + e] + *o;
                                        else __builtin_nontemporal_store(acc[ib][ub][4 * q + e], o);
                                    }
                            }
                        }
                }
                continue;
            }
            if (MODE == 0) {
                if (u < a.B) {  // rows jq .. jq+3 of the lane are consecutive items: one 16-byte store
                    float* orow = a.sample_out + (int64_t)blockIdx.y * a.sample_split + (int64_t)u * n_pass +
                                  (int64_t)t * MF_TI;
#pragma unroll
                    for (int ib = 0; ib < 4; ++ib) {
                        const uint32_t mw = mask_word(ib);
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const int jq = lrow0 + ib * 32 + q * 8;
                            float v4[4];
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                v4[e] = (!MASKED || ((mw >> (mbit0 + 8 * q + e)) & 1u)) ? acc[ib][ub][4 * q + e] : -INFINITY;
                            if (jq + 3 < lim)
                                *(float4*)(orow + jq) = make_float4(v4[0], v4[1], v4[2], v4[3]);
                            else
#pragma unroll
                                for (int e = 0; e < 4; ++e)
                                    if (jq + e < lim) orow[jq + e] = v4[e];
                        }
                    }
                }
                continue;
            }
            if (MODE == 6) {
                // rescue of a flagged user: count (or collect) every finite
                // score whose ranking key is at least the user's bound
                if (nin_[ub]) {
                    const uint64_t lo = nlo_[ub];
#pragma unroll
                    for (int ib = 0; ib < 4; ++ib) {
                        const uint32_t mw = mask_word(ib);
                        const uint32_t idb = (uint32_t)(j0 + lrow0 + ib * 32);
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const float v = acc[ib][ub][r];
                            if (MASKED && !((mw >> (mbit0 + (r >> 2) * 8 + (r & 3))) & 1u)) continue;
                            if (!(v >= -FLT_MAX)) continue;  // rows past the catalog's end (-inf)
                            const uint64_t key = rank_key(v, idb + (r >> 2) * 8 + (r & 3));
                            if (key < lo) continue;
                            if (a.collect) {
                                const int slot = atomicAdd(a.ccnt + u, 1);
                                if (slot < a.ccol) a.coll[(int64_t)u * a.ccol + slot] = key;
                            } else {
                                const uint64_t bin = (key - lo) >> nsh_[ub];
                                if (bin < (uint64_t)kNarrowBins) atomicAdd(a.hist + (int64_t)u * kNarrowBins + bin, 1u);
                            }
                        }
                    }
                }
                continue;
            }
            // exact running max per 32 x 32 block: the block's max, one rescale
            // of the running sum and one exp per score against it
            const float th = th_[ub];
#pragma unroll
            for (int ib = 0; ib < 4; ++ib) {
                const int jb = lrow0 + ib * 32;  // rows jb + 8q + e
                float v[16];
                const uint32_t mw = mask_word(ib);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    v[r] = acc[ib][ub][r];
                    if (MASKED && !((mw >> (mbit0 + (r >> 2) * 8 + (r & 3))) & 1u)) v[r] = -INFINITY;
                }
                float bmax = v[0];
#pragma unroll
                for (int r = 1; r < 16; ++r) bmax = fmaxf(bmax, v[r]);
                const float mnew = fmaxf(m_[ub], bmax);
                if (mnew != -INFINITY) {
                    const float mb = mnew * kLog2e;
                    float s0 = 0.f, s1 = 0.f;
#pragma unroll
                    for (int r = 0; r < 16; r += 2) {
                        s0 += fast_exp2(fmaf(v[r], kLog2e, -mb));
                        s1 += fast_exp2(fmaf(v[r + 1], kLog2e, -mb));
                    }
                    l_[ub] = l_[ub] * fast_exp2(fmaf(m_[ub], kLog2e, -mb)) + (s0 + s1);
                    m_[ub] = mnew;
                }
                if (bmax >= th) {
                    // bounded regions: past a full piece, keys go to the
                    // user's overflow region (an atomic slot; rare but for
                    // catalogs stored in clusters)
                    const int capr = a.cap > 0 ? a.cap : INT_MAX;
                    uint64_t* kreg = a.keys + (a.cap > 0 ? (((int64_t)u * a.P + c) * 4 + g) * a.cap
                                                         : (int64_t)u * a.key_stride + chunk_item0 + (int64_t)g * 64 * ntiles);
                    const uint32_t idb = (uint32_t)(j0 + jb);
                    uint32_t spill = 0;  // scores that found the piece full
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (v[r] >= th) {
                            if (cnt_[ub] < capr) {
                                kreg[cnt_[ub]] = rank_key(v[r], idb + (r >> 2) * 8 + (r & 3));
                                ++cnt_[ub];
                            } else {
                                spill |= 1u << r;
                            }
                        }
                    if (spill != 0u) {
                        // one slot reservation for the block's spilled keys
                        int slot = atomicAdd(a.pcnt + (int64_t)u * a.rec_stride + (int64_t)a.P * 4, __popc(spill));
                        uint64_t* ovr = a.keys + a.ovf_base + (int64_t)u * a.ovf_cap;
#pragma unroll
                        for (int r = 0; r < 16; ++r)
                            if ((spill >> r) & 1u) {
                                if (slot < a.ovf_cap) ovr[slot] = rank_key(v[r], idb + (r >> 2) * 8 + (r & 3));
                                ++slot;
                            }
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    // ---- pipeline ------------------------------------------------------------
    // Steps run over the flat sequence (tile, k-step).  Each step issues the
    // DMA of step + (NS - 1) -- op 0 of both operands among the MFMAs of its
    // first half, op 1 among those of its second half, so that the CU's
    // vector-memory path sees an even stream rather than a burst after every
    // barrier (past the end: the last tile again, into a stage nobody reads,
    // so every step issues the same number of ops).  It reads slice 1 of its
    // stage while slice 0 runs on the matrix cores, waits until the DMA of
    // step+1 has landed (loads retire in order, so "at most the ops of the
    // later steps and the first half of the newest outstanding" suffices;
    // epilogue stores in between only make the wait stricter) and until its
    // own LDS reads have completed, then meets the other waves at the
    // barrier: past it every read of this step's stage is done, and that
    // stage is the one the next step's DMA overwrites.  It reads slice 0 of
    // the next stage while slice 1 runs.  The DMA ring moves on after both
    // halves.
    static_assert(MF_DMA == 2, "one op per operand in each half of a step");
    constexpr int kOpsPerStep = 2 * MF_DMA;
    constexpr int kWaitOps = (MF_NS - 3) * kOpsPerStep + 2;
    int ls = 0, lt = 0, lk = 0;  // next DMA: stage, tile (chunk-relative), k-step
    e_rsrc(tile0);
    auto advance = [&]() {
        ls = ls + 1 == MF_NS ? 0 : ls + 1;
        if (++lk == nk) {
            lk = 0;
            if (++lt < ntiles) e_rsrc(tile0 + lt);  // past the end: keep re-reading the last tile
        }
    };
#pragma unroll
    for (int q = 0; q < MF_NS - 1; ++q) {
        dma_op(ls, lk * KE, 0);
        dma_op(ls, lk * KE, 1);
        advance();
    }
    MF_WAIT_VMCNT((MF_NS - 2) * kOpsPerStep);
    __builtin_amdgcn_s_barrier();

    Frag f0, f1;
    load_frag(f0, 0, 0, 0);
    int cs = 0;  // stage being computed
    for (int t = 0; t < ntiles; ++t) {
#pragma unroll
        for (int ib = 0; ib < 4; ++ib)
#pragma unroll
            for (int ub = 0; ub < MF_UB; ++ub) acc[ib][ub] = f32x16_t{};
        // MFMAs per half step, and the spacing R of the schedule's reads and DMA
        // ops among them (one MFMA apart for bf16, four for fp32)
        constexpr int NMF = 4 * MF_UB * (F32 ? 4 : 1), R = NMF / (4 * MF_UB);
        for (int k = 0; k < nk; ++k) {
            dma_op(ls, lk * KE, 0);
            load_frag(f1, cs, 1, k * KE);
            mma(f0);
            // schedule: slice-1 reads between the MFMAs, the two DMA ops after MFMA groups 3 and 6
#pragma unroll
            for (int i = 0; i < NMF; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                if (i % R == 0 && i / R < 4 + MF_UB) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
                if (i == 2 * R || i == 5 * R) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM (DMA)
            }
            MF_WAIT_VMCNT_LDS(kWaitOps);
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
            cs = cs + 1 == MF_NS ? 0 : cs + 1;
            dma_op(ls, lk * KE, 1);
            // (on the very last step this reads a stage whose data is never used)
            load_frag(f0, cs, 0, (k + 1 < nk ? k + 1 : 0) * KE);
            mma(f1);
#pragma unroll
            for (int i = 0; i < NMF; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
                if (i % R == 0 && i / R < 4 + MF_UB) __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
                if (i == 2 * R || i == 5 * R) __builtin_amdgcn_sched_group_barrier(0x020, 1, 1);
            }
            __builtin_amdgcn_sched_barrier(0);
            advance();
        }
        // Partial tile (the catalog's last): rows past the end score -inf,
        // set once here under a uniform branch.  Folding this test into every
        // block's epilogue made the compiler keep 16 row masks per block in
        // scalar registers and spill them on every tile.
        if ((MODE == 1 || MODE == 6) && tile_valid(tile0 + t) < MF_TI) {
            const int lim = tile_valid(tile0 + t);
#pragma unroll
            for (int ib = 0; ib < 4; ++ib)
#pragma unroll
                for (int ub = 0; ub < MF_UB; ++ub)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (lrow0 + ib * 32 + (r >> 2) * 8 + (r & 3) >= lim) acc[ib][ub][r] = -INFINITY;
        }
        epilogue(tile0 + t);
    }
    MF_WAIT_VMCNT(0);

    if (MODE == 1) {
#pragma unroll
        for (int ub = 0; ub < MF_UB; ++ub) {
            const int u = u0 + wu * MF_WU + ub * 32 + (lane & 31);
            if (u < a.B && (a.user_flag == nullptr || a.user_flag[u] != 0)) {
                const int64_t piece = ((int64_t)u * a.P + c) * 4 + g;
                const int64_t rec = a.rec_stride > 0 ? (int64_t)u * a.rec_stride + c * 4 + g : piece;
                a.pm[rec] = m_[ub];
                a.pl[rec] = l_[ub];
                a.pcnt[rec] = cnt_[ub];
                a.preg[rec] = a.cap > 0 ? piece * a.cap : (int64_t)u * a.key_stride + chunk_item0 + (int64_t)g * 64 * ntiles;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Block-level selection of the k-th largest 64-bit key
// ---------------------------------------------------------------------------
constexpr int SEL_NT = 256;
constexpr int SEL_NB = 256;     // histogram bins per narrowing pass
constexpr int SEL_GCAP = 6144;  // range gathered into LDS once it holds at most this many keys
constexpr int SEL_SMALL = 256;  // range ranked once it holds at most this many keys
constexpr int SEL_UNR = 8;      // independent loads in flight per thread

// Block-shared state of a selection; GCAP = keys the LDS gather holds (the
// merge also uses a smaller build, which fits twice the blocks on a CU).
template <int GCAP>
struct SelSharedT {
    static_assert(GCAP >= GENREC_KMAX, "the merge places the final K keys in the gather buffer");
    static constexpr int kGcap = GCAP;
    unsigned long long red_lo[SEL_NT / kWave], red_hi[SEL_NT / kWave];
    int hist[SEL_NT / kWave][SEL_NB];  // one histogram per wave: less atomic contention
    int cnt_a, cnt_b, bin, above;
    uint64_t gbuf[GCAP];
    uint64_t sbuf[SEL_SMALL];
    uint64_t out[GENREC_KMAX];
};
using SelShared = SelSharedT<SEL_GCAP>;

__device__ __forceinline__ unsigned long long wave_min_u64(unsigned long long v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const unsigned long long t = __shfl_xor(v, o);
        v = t < v ? t : v;
    }
    return v;
}
__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const unsigned long long t = __shfl_xor(v, o);
        v = t > v ? t : v;
    }
    return v;
}

// Bitonic sort, descending, of one wave's 64 * C keys held in registers:
// element t * 64 + lane is v[t]; partners in other lanes are exchanged with
// shuffles, partners in the same lane directly.  No barrier.
template <int C>
__device__ void wave_sort_desc(uint64_t (&v)[C]) {
    const int lane = threadIdx.x & 63;
    constexpr int N = 64 * C;
#pragma unroll
    for (int k = 2; k <= N; k <<= 1) {
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1) {
            if (j >= 64) {
#pragma unroll
                for (int t = 0; t < C; ++t) {
                    const int tp = t ^ (j >> 6);
                    if (tp > t) {
                        const bool desc = ((t * 64 + lane) & k) == 0;
                        const uint64_t x = v[t], y = v[tp];
                        if (desc ? (x < y) : (x > y)) {
                            v[t] = y;
                            v[tp] = x;
                        }
                    }
                }
            } else {
#pragma unroll
                for (int t = 0; t < C; ++t) {
                    const uint64_t x = v[t];
                    const uint64_t y = __shfl_xor(x, j);
                    const bool desc = ((t * 64 + lane) & k) == 0;
                    const bool lower = (lane & j) == 0;  // the smaller index of the pair
                    const bool take_max = desc == lower;
                    v[t] = take_max ? (x > y ? x : y) : (x < y ? x : y);
                }
            }
        }
    }
}

template <int C>
__device__ void block_sort_runs(uint64_t* in, int n, uint64_t* out, int R) {  // R = 64 C
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    uint64_t v[C];
#pragma unroll
    for (int t = 0; t < C; ++t) {
        const int e = w * R + t * 64 + lane;
        v[t] = e < n ? in[e] : 0ull;  // 0: below every key
    }
    wave_sort_desc<C>(v);
    __syncthreads();  // every key of `in` is read before the runs overwrite it
#pragma unroll
    for (int t = 0; t < C; ++t) in[w * R + t * 64 + lane] = v[t];
    __syncthreads();
    // Each key's rank: its place in its run plus, in each other run, the keys
    // above it (earlier runs first among equal keys) -- binary searches, all
    // C x 3 of a thread advanced in lock step so that their LDS reads are in
    // flight together rather than one dependent chain after another.
    constexpr int NQ = SEL_NT / kWave - 1;  // the other runs
    constexpr int STEPS = C == 1 ? 7 : (C == 2 ? 8 : 9);  // halvings of [0, R], R = 64 C
    static_assert(C == 1 || C == 2 || C == 4, "runs of 64, 128 or 256 keys");
    int lo[C][NQ], hi[C][NQ];
#pragma unroll
    for (int t = 0; t < C; ++t)
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            lo[t][i] = 0;
            hi[t][i] = R;
        }
#pragma unroll
    for (int step = 0; step < STEPS; ++step)
#pragma unroll
        for (int t = 0; t < C; ++t)
#pragma unroll
            for (int i = 0; i < NQ; ++i) {
                const int q = i + (i >= w ? 1 : 0);  // wave-uniform
                const int mid = min((lo[t][i] + hi[t][i]) >> 1, R - 1);  // (read only while lo < hi)
                const uint64_t y = in[q * R + mid];
                const bool above = q < w ? (y >= v[t]) : (y > v[t]);
                if (lo[t][i] < hi[t][i]) {
                    if (above) lo[t][i] = mid + 1;
                    else hi[t][i] = mid;
                }
            }
#pragma unroll
    for (int t = 0; t < C; ++t) {
        if (v[t] == 0ull) continue;
        int r = t * 64 + lane;
#pragma unroll
        for (int i = 0; i < NQ; ++i) r += lo[t][i];
        out[r] = v[t];
    }
}

// Sort, descending, of in[0..n) into out[0..n), n <= 4 * 256 (`in` needs room
// for 4 runs of R keys and is overwritten): each wave sorts a run of R keys
// (a power of two >= n / 4) in registers, then every key's rank is its place
// in its run plus the larger keys of the other three runs (binary searches);
// equal keys keep their run order.  Two barriers instead of a bitonic
// network's one per stage.
__device__ void block_sort_into(uint64_t* in, int n, uint64_t* out) {
    static_assert(SEL_NT == 4 * kWave, "four runs, one per wave");
    static_assert(GENREC_KMAX <= 4 * 256, "runs of at most 256 keys fill the 1,024-key output buffer");
    int R = 64;
    while (R * (SEL_NT / kWave) < n) R <<= 1;
    if (R == 64) block_sort_runs<1>(in, n, out, R);
    else if (R == 128) block_sort_runs<2>(in, n, out, R);
    else block_sort_runs<4>(in, n, out, R);
}

// Rank placement: key i of in[0..n) goes to out[r], r = the number of keys
// that rank before it (larger, or equal with a lower index), i.e. out holds
// the keys in descending order, a stable sort.  O(n^2 / threads) compares but
// no barrier inside; used for the few hundred keys at the end of a selection.
// With limit < n only the keys of rank < limit are written.
__device__ void block_rank_place(const uint64_t* in, int n, uint64_t* out, int limit) {
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
        const uint64_t x = in[i];
        int r = 0;
#pragma unroll 8
        for (int j = 0; j < n; ++j) {  // (unrolled: several LDS reads in flight)
            const uint64_t y = in[j];
            r += (y > x) | ((y == x) & (j < i));
        }
        if (r < limit) out[r] = x;
    }
}

// Keys of an LDS array, for the narrowing passes after the gather.
struct LdsSrc {
    const uint64_t* buf;
    int n;
    template <class F>
    __device__ void for_each(F&& f) const {
        for (int i = threadIdx.x; i < n; i += SEL_NT) f(buf[i]);
    }
};

// One narrowing pass: histogram the keys of [lo, hi] into 256 power-of-two-
// wide bins and move [lo, hi] to the bin holding the k_rem-th largest key.
// k_rem drops by the keys of the bins above it; returns the keys in the bin.
template <class Src, class Sh>
__device__ int64_t narrow(const Src& src, unsigned long long& lo, unsigned long long& hi, int& k_rem, Sh& sh) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const unsigned long long span = hi - lo;
    const int shift = max(0, 64 - __clzll(span) - 8);  // (hi - lo) >> shift < 256
    for (int i = tid; i < SEL_NB * (SEL_NT / kWave); i += SEL_NT) (&sh.hist[0][0])[i] = 0;
    __syncthreads();
    const unsigned long long clo = lo, chi = hi;
    int* whist = sh.hist[w];
    src.for_each([&](uint64_t key) {
        if (key >= clo && key <= chi) atomicAdd(&whist[(int)((key - clo) >> shift)], 1);
    });
    __syncthreads();
    for (int i = tid; i < SEL_NB; i += SEL_NT) {
        int t = 0;
#pragma unroll
        for (int q = 0; q < SEL_NT / kWave; ++q) t += sh.hist[q][i];
        sh.hist[0][i] = t;
    }
    __syncthreads();
    // wave 0 finds bin d with above(d) < k_rem <= above(d) + hist[d]
    if (w == 0) {
        int v[SEL_NB / kWave];
        int tsum = 0;
#pragma unroll
        for (int i = 0; i < SEL_NB / kWave; ++i) {  // lane owns 4 bins, highest bins first
            v[i] = sh.hist[0][SEL_NB - 1 - (lane * (SEL_NB / kWave) + i)];
            tsum += v[i];
        }
        int incl = tsum;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int t = __shfl_up(incl, o);
            if (lane >= o) incl += t;
        }
        int run = incl - tsum;
#pragma unroll
        for (int i = 0; i < SEL_NB / kWave; ++i) {
            if (run < k_rem && k_rem <= run + v[i]) {
                sh.bin = SEL_NB - 1 - (lane * (SEL_NB / kWave) + i);
                sh.above = run;
            }
            run += v[i];
        }
    }
    __syncthreads();
    const int d = sh.bin;
    k_rem -= sh.above;
    const int64_t n_bin = sh.hist[0][d];
    lo = clo + ((unsigned long long)d << shift);
    const unsigned long long top = lo + ((1ull << shift) - 1);
    hi = top < chi ? top : chi;
    __syncthreads();
    return n_bin;
}

// Finds the k-th largest key (1 <= k <= n) among the keys the source yields
// and, with COLLECT, leaves the k largest keys in sh.out[0..k) (unsorted).
// Returns the k-th largest key.  At most GCAP keys (the shared state's gather
// capacity): one pass copies them into LDS.  More: passes over the source --
//   1. min / max of all keys;
//   2. while the candidate range [lo, hi] holds more than GCAP keys, a
//      narrowing pass (histogram of the range, keep the bin of the k-th);
//   3. gather: the range into LDS and (COLLECT) every key above it into out.
// Then, in LDS, narrowing continues until at most SEL_SMALL keys remain in
// the range, which are sorted; keys above the final range join out.
// Block-wide min and max of the keys a source yields (every thread gets both).
template <class Src, class Sh>
__device__ void block_minmax(const Src& src, unsigned long long& lo, unsigned long long& hi, Sh& sh) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    lo = ~0ull;
    hi = 0;
    src.for_each([&](uint64_t key) {
        lo = key < lo ? key : lo;
        hi = key > hi ? key : hi;
    });
    lo = wave_min_u64(lo);
    hi = wave_max_u64(hi);
    if (lane == 0) { sh.red_lo[w] = lo; sh.red_hi[w] = hi; }
    __syncthreads();
    lo = sh.red_lo[0];
    hi = sh.red_hi[0];
    for (int q = 1; q < SEL_NT / kWave; ++q) {
        lo = sh.red_lo[q] < lo ? sh.red_lo[q] : lo;
        hi = sh.red_hi[q] > hi ? sh.red_hi[q] : hi;
    }
    __syncthreads();
}

template <bool COLLECT, class Src, class Sh>
__device__ uint64_t block_select(const Src& src, int k, Sh& sh) {
    constexpr int GCAP = Sh::kGcap;
    const int tid = threadIdx.x;
    unsigned long long lo, hi;
    int64_t n_range = src.total();
    int k_rem = k;
    int ng;
    if (n_range <= GCAP) {
        // few keys: one pass copies them all into LDS (each to its position in
        // the source's order), and everything else happens there
        src.gather(sh.gbuf);
        if (tid == 0) sh.cnt_a = 0;
        __syncthreads();
        ng = (int)n_range;
        block_minmax(LdsSrc{sh.gbuf, ng}, lo, hi, sh);
    } else {
        block_minmax(src, lo, hi, sh);
        while (lo != hi && n_range > GCAP) n_range = narrow(src, lo, hi, k_rem, sh);
        // gather the range into LDS; keys above it are in the result for sure
        if (tid == 0) { sh.cnt_a = 0; sh.cnt_b = 0; }
        __syncthreads();
        {
            const unsigned long long flo = lo, fhi = hi;
            const bool single = flo == fhi;
            src.for_each([&](uint64_t key) {
                if (key > fhi) {
                    if (COLLECT) sh.out[atomicAdd(&sh.cnt_a, 1)] = key;
                } else if (key >= flo && !single) {
                    sh.gbuf[atomicAdd(&sh.cnt_b, 1)] = key;
                }
            });
        }
        __syncthreads();
        ng = sh.cnt_b;
        // every thread holds its copy before thread 0 clears the count for the
        // last pass below (with no LDS narrowing pass in between, nothing else
        // separates that read from the clear)
        __syncthreads();
    }
    uint64_t kth;
    if (lo == hi) {  // every key left in the range is the k-th (equal keys)
        kth = lo;
        if (COLLECT) {
            const int n_above = sh.cnt_a;
            for (int i = tid; i < k_rem; i += SEL_NT) sh.out[n_above + i] = lo;
        }
        __syncthreads();
        return kth;
    }
    LdsSrc lsrc{sh.gbuf, ng};
    while (lo != hi && n_range > SEL_SMALL) n_range = narrow(lsrc, lo, hi, k_rem, sh);
    // keys of the gathered set above the final range join out; the range is sorted
    if (tid == 0) sh.cnt_b = 0;
    __syncthreads();
    {
        const unsigned long long flo = lo, fhi = hi;
        const bool single = flo == fhi;
        for (int i = tid; i < ng; i += SEL_NT) {
            const uint64_t key = sh.gbuf[i];
            if (key > fhi) {
                if (COLLECT) sh.out[atomicAdd(&sh.cnt_a, 1)] = key;
            } else if (key >= flo && !single) {
                sh.sbuf[atomicAdd(&sh.cnt_b, 1)] = key;
            }
        }
    }
    __syncthreads();
    const int n_above = sh.cnt_a;  // == k - k_rem when COLLECT
    if (lo == hi) {
        kth = lo;
        if (COLLECT)
            for (int i = tid; i < k_rem; i += SEL_NT) sh.out[n_above + i] = lo;
    } else {
        // the k_rem largest keys of the range, in descending order, after the
        // keys above it
        block_rank_place(sh.sbuf, (int)n_range, sh.out + n_above, k_rem);
        __syncthreads();
        kth = sh.out[n_above + k_rem - 1];
    }
    __syncthreads();
    return kth;
}

// ---------------------------------------------------------------------------
// Sampled thresholds: per user, the K-th (and the r_fast-th) largest score of
// the catalog sample.  One block per user holds the whole sample in
// registers as 32-bit order keys (128 per thread), so the row is read once;
// selection narrows a key range with 256-bin histograms, after a subsample
// histogram and an exact count have cut the range to a few k keys.
// ---------------------------------------------------------------------------
constexpr int TH_KEYS = 32768;  // one user's sample at most (a 16,384-key build serves smaller samples)

constexpr int TH_GROUPS = 256;  // thread groups whose maxima bound the fast route
constexpr int TH_FAST = 1024;   // keys the fast route ranks at most

template <int NW>
struct ThShared {
    int hist[2][NW][256];  // per rank, per wave
    unsigned red_lo[NW], red_hi[NW];
    int cnt[2][NW];
    int bin[2], above[2];
    // fast route
    uint32_t gmax[TH_GROUPS];
    uint32_t tred[NW];
    int wcnt[NW];
    uint32_t cand[TH_FAST + 4];
    uint32_t res[2];
};

__device__ __forceinline__ int th_shift(unsigned span) { return max(0, 32 - __clz(span) - 8); }

// Wave 0: the bin d of hist holding the k-th largest key (above(d) < k <=
// above(d) + hist[d], bins scanned from the top); result in sh.bin[q], sh.above[q].
template <class Sh>
__device__ void th_find(const int* hist, int k, int q, Sh& sh) {
    const int lane = threadIdx.x & 63;
    int v[4], tsum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {  // lane owns 4 bins, highest bins first
        v[i] = hist[255 - (lane * 4 + i)];
        tsum += v[i];
    }
    int incl = tsum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(incl, o);
        if (lane >= o) incl += t;
    }
    int run = incl - tsum;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (run < k && k <= run + v[i]) {
            sh.bin[q] = 255 - (lane * 4 + i);
            sh.above[q] = run;
        }
        run += v[i];
    }
}

// A hair below the sampled score: still a lower bound of the catalog's
// order statistic, robust to any rounding difference between passes.
__device__ __forceinline__ float th_lower(float t) { return t - fabsf(t) * 0x1p-20f - FLT_MIN; }

// TH_NT threads of TH_CAP / TH_NT keys each (TH_CAP >= the sample size):
// many threads for few users (latency), fewer for many (throughput).
template <int TH_NT, int TH_CAP>
__global__ __launch_bounds__(TH_NT) void threshold_kernel(ThresholdArgs a) {
    constexpr int TH_PER = TH_CAP / TH_NT;
    constexpr int TH_NW = TH_NT / kWave;
    static_assert(TH_PER % 8 == 0 && TH_NT >= 256, "thread layout");
    __shared__ ThShared<TH_NW> sh;
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    if (tid == 0) {
        if (a.user_flag != nullptr) a.user_flag[b] = 0;
        if (a.tile_flag != nullptr && b % MF_TU == 0) a.tile_flag[b / MF_TU] = 0;
        if (a.rc != nullptr && b == 0) {
            a.rc[0] = 0;
            a.rc[1] = 0;
        }
        if (a.rescued != nullptr && b == 0) *a.rescued = 0;
        if (a.ovf_pm != nullptr) {  // the user's overflow record starts empty
            const int64_t rec = (int64_t)b * a.rec_stride + a.rec_off;
            a.ovf_pm[rec] = -INFINITY;
            a.ovf_pl[rec] = 0.f;
            a.ovf_pcnt[rec] = 0;
            a.ovf_preg[rec] = a.ovf_base + (int64_t)b * a.ovf_cap;
        }
    }
    const int n = (int)a.n_sample;
    if (n < a.K) {
        if (tid == 0) {
            a.theta_safe[b] = -INFINITY;
            if (a.theta_fast != nullptr) a.theta_fast[b] = -INFINITY;
        }
        return;
    }
    // key e of thread t: e = 4 TH_NT i + 4 t + j (j < 4): 16-byte loads,
    // contiguous across the block
    // (sampled scores of a split reduction: the partial rows summed in split order)
    const float* row = a.sample + (int64_t)b * a.n_sample;
    // 16-byte buffer loads (n is a multiple of 4), split after split, each
    // split's loads in flight together.  The record count ends at the row's
    // end, so a quad past it reads zeros (dropped below) with neither a branch
    // nor a 64-bit address per load; the split sums keep their order.
    typedef unsigned int th_u32x4 __attribute__((ext_vector_type(4)));
    auto quad = [&](const __amdgpu_buffer_rsrc_t& r, int i) {
        const th_u32x4 q = __builtin_amdgcn_raw_buffer_load_b128(r, tid * 16, i * TH_NT * 16, 0);
        return make_float4(__uint_as_float(q.x), __uint_as_float(q.y), __uint_as_float(q.z), __uint_as_float(q.w));
    };
    auto rsrc_of = [&](int z) {
        return __builtin_amdgcn_make_buffer_rsrc((void*)(row + (int64_t)z * a.split_stride), (short)0, n * 4,
                                                 0x00020000);
    };
    // Chunks of at most 16 quads: loaded (and summed over the splits), then
    // turned into keys, before the next chunk's loads start -- 64 loaded
    // floats live at a time beside the keys.  Within a split, four quads at a
    // time: the scheduling barriers keep the loads from all being hoisted
    // above the adds, which would hold twice the registers and cost the
    // many-user builds their occupancy.
    constexpr int QC = TH_PER / 4 < 16 ? TH_PER / 4 : 16;  // quads per chunk
    static_assert((TH_PER / 4) % QC == 0 && QC % 4 == 0, "chunk layout");
    uint32_t key[TH_PER];  // 0 = no key (every score's key is larger)
#pragma unroll
    for (int c0 = 0; c0 < TH_PER / 4; c0 += QC) {
        float4 v[QC];
        {
            const __amdgpu_buffer_rsrc_t r0 = rsrc_of(0);
#pragma unroll
            for (int i = 0; i < QC; ++i) v[i] = quad(r0, c0 + i);
        }
        for (int z = 1; z < a.n_split; ++z) {
            const __amdgpu_buffer_rsrc_t rz = rsrc_of(z);
#pragma unroll
            for (int i0 = 0; i0 < QC; i0 += 4) {
                float4 p[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) p[c] = quad(rz, c0 + i0 + c);
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    v[i0 + c].x += p[c].x;
                    v[i0 + c].y += p[c].y;
                    v[i0 + c].z += p[c].z;
                    v[i0 + c].w += p[c].w;
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
#pragma unroll
        for (int i = 0; i < QC; ++i) {
            const int e = (c0 + i) * (TH_NT * 4) + tid * 4;
            const float f[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) key[4 * (c0 + i) + j] = e + j < n ? order_key(f[j]) : 0u;
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    unsigned lo = ~0u, hi = 0u;
#pragma unroll
    for (int i = 0; i < TH_PER; ++i)
        if (key[i] != 0u) {
            lo = min(lo, key[i]);
            hi = max(hi, key[i]);
        }
    // ranks: q = 0 the K-th largest, q = 1 the r_fast-th largest
    const int nq = a.theta_fast != nullptr ? 2 : 1;
    int krem[2] = {a.K, max(1, min(a.r_fast, a.K))};
    // Fast route (K <= 256 groups): the block's threads form TH_GROUPS groups
    // of TH_NT / TH_GROUPS; T = the K-th largest of the groups' maxima.  K
    // groups hold a key >= T, so at least K keys reach T and both ranks (K
    // and r_fast <= K) are among the keys >= T: a few times K of them for
    // unordered scores, every key when fewer than K groups hold one (T = 0).
    // They are compacted and ranked exactly -- the same keys the narrowing
    // passes below end on.  More than TH_FAST of them (heavy ties): those
    // passes, which use none of the fast route's shared fields.  Built for
    // the few-user launches (at most 32 keys a thread): with 64 or 128 the
    // route's registers would cost those builds their occupancy.
    if constexpr (TH_PER <= 32)
    if (a.K <= TH_GROUPS) {  // block-uniform
        constexpr int GS = TH_NT / TH_GROUPS;     // threads per group
        constexpr int PER_T = TH_GROUPS / GS;     // group maxima each thread compares
        static_assert(GS >= 1 && (GS & (GS - 1)) == 0 && PER_T % 4 == 0, "group layout");
        uint32_t gm = 0u;
#pragma unroll
        for (int i = 0; i < TH_PER; ++i) gm = max(gm, key[i]);
#pragma unroll
        for (int o = 1; o < GS; o <<= 1) gm = max(gm, (uint32_t)__shfl_xor((int)gm, o));
        const int g = tid / GS, gl = tid - g * GS;
        if (gl == 0) sh.gmax[g] = gm;
        __syncthreads();
        // the group maximum's rank (maxima strictly above it), its GS threads
        // each comparing a slice of the maxima
        int rk = 0;
        const uint4* g4 = (const uint4*)(sh.gmax + gl * PER_T);
#pragma unroll 8
        for (int q = 0; q < PER_T / 4; ++q) {
            const uint4 m4 = g4[q];
            rk += (m4.x > gm) + (m4.y > gm) + (m4.z > gm) + (m4.w > gm);
        }
#pragma unroll
        for (int o = 1; o < GS; o <<= 1) rk += __shfl_xor(rk, o);
        uint32_t tc = rk < a.K ? gm : 0xFFFFFFFFu;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) tc = min(tc, (uint32_t)__shfl_xor((int)tc, o));
        if (lane == 0) sh.tred[w] = tc;
        __syncthreads();
        uint32_t T = sh.tred[0];
#pragma unroll
        for (int q = 1; q < TH_NW; ++q) T = min(T, sh.tred[q]);
        // keys >= T as bits of the thread's own words (not one scalar mask
        // per key held until the compaction)
        uint32_t pass[(TH_PER + 31) / 32] = {};
#pragma unroll
        for (int i = 0; i < TH_PER; ++i) pass[i >> 5] |= (key[i] != 0u && key[i] >= T) ? 1u << (i & 31) : 0u;
        int c = 0;
#pragma unroll
        for (int q = 0; q < (TH_PER + 31) / 32; ++q) c += __popc(pass[q]);
        int incl = c;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int t = __shfl_up(incl, o);
            if (lane >= o) incl += t;
        }
        if (lane == 63) sh.wcnt[w] = incl;
        __syncthreads();
        int base = incl - c, total = 0;
#pragma unroll
        for (int q = 0; q < TH_NW; ++q) {
            base += q < w ? sh.wcnt[q] : 0;
            total += sh.wcnt[q];
        }
        if (total <= TH_FAST) {  // block-uniform
#pragma unroll
            for (int i = 0; i < TH_PER; ++i)
                if ((pass[i >> 5] >> (i & 31)) & 1u) sh.cand[base++] = key[i];
            if (tid < 4) sh.cand[total + tid] = 0u;  // to whole uint4s (0 is below every key)
            __syncthreads();
            // the k-th largest value x: fewer than k keys above it, at least k at or above
            const uint4* c4 = (const uint4*)sh.cand;
            for (int i = tid; i < total; i += TH_NT) {
                const uint32_t x = sh.cand[i];
                int gt = 0, ge = 0;
                for (int q = 0; q < (total + 3) / 4; ++q) {
                    const uint4 y = c4[q];
                    gt += (y.x > x) + (y.y > x) + (y.z > x) + (y.w > x);
                    ge += (y.x >= x) + (y.y >= x) + (y.z >= x) + (y.w >= x);
                }
                // several keys may share the value: they write the same word
                if (gt < krem[0] && krem[0] <= ge) sh.res[0] = x;
                if (nq > 1 && gt < krem[1] && krem[1] <= ge) sh.res[1] = x;
            }
            __syncthreads();
            if (tid == 0) {
                a.theta_safe[b] = th_lower(key_to_score(sh.res[0]));
                if (a.theta_fast != nullptr) a.theta_fast[b] = th_lower(key_to_score(sh.res[1]));
            }
            return;
        }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        lo = min(lo, (unsigned)__shfl_xor((int)lo, o));
        hi = max(hi, (unsigned)__shfl_xor((int)hi, o));
    }
    if (lane == 0) { sh.red_lo[w] = lo; sh.red_hi[w] = hi; }
    __syncthreads();
    lo = sh.red_lo[0];
    hi = sh.red_hi[0];
#pragma unroll
    for (int q = 1; q < TH_NW; ++q) {
        lo = min(lo, sh.red_lo[q]);
        hi = max(hi, sh.red_hi[q]);
    }
    unsigned qlo[2] = {lo, lo}, qhi[2] = {hi, hi};
    if (lo < hi) {
        // Cut the range from below first: a histogram of every 8th key places
        // the (2k/8 + 8)-th largest of that subsample; the lower edge c of its
        // bin is checked exactly -- if at least k keys reach c, the k-th
        // largest lies in [c, hi], which holds a few k keys instead of all of
        // them.  Otherwise the full range.
        const int nsub = (n + 7) / 8;
        const int shift = th_shift(hi - lo);
        for (int i = tid; i < TH_NW * 256; i += TH_NT) (&sh.hist[0][0][0])[i] = 0;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < TH_PER; i += 8)
            if (key[i] >= lo && key[i] <= hi) atomicAdd(&sh.hist[0][w][(key[i] - lo) >> shift], 1);
        __syncthreads();
        if (tid < 256) {
            int t = 0;
#pragma unroll
            for (int q = 0; q < TH_NW; ++q) t += sh.hist[0][q][tid];
            sh.hist[1][0][tid] = t;
        }
        __syncthreads();
        if (w == 0)
            for (int q = 0; q < nq; ++q) th_find(sh.hist[1][0], min(nsub, 2 * ((krem[q] + 7) / 8) + 8), q, sh);
        __syncthreads();
        unsigned cut[2];
        int cnt[2] = {0, 0};
        for (int q = 0; q < nq; ++q) cut[q] = lo + ((unsigned)sh.bin[q] << shift);
#pragma unroll
        for (int i = 0; i < TH_PER; ++i) {
            cnt[0] += key[i] >= cut[0];
            if (nq > 1) cnt[1] += key[i] >= cut[1];
        }
        for (int q = 0; q < nq; ++q) {
            int v = cnt[q];
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
            if (lane == 0) sh.cnt[q][w] = v;
        }
        __syncthreads();
        for (int q = 0; q < nq; ++q) {
            int tot = 0;
#pragma unroll
            for (int x = 0; x < TH_NW; ++x) tot += sh.cnt[q][x];
            if (tot >= krem[q]) qlo[q] = cut[q];
        }
    }
    // Narrowing, both ranks in the same passes: each pass histograms the keys
    // of each open range into 256 bins of width 2^shift and keeps the bin of
    // the rank; a span shrinks 256-fold per pass, so at most four passes.
    for (int pass = 0; pass < 4; ++pass) {
        const bool open0 = qlo[0] < qhi[0], open1 = nq > 1 && qlo[1] < qhi[1];
        if (!open0 && !open1) break;  // block-uniform
        const int sh0 = open0 ? th_shift(qhi[0] - qlo[0]) : 0;
        const int sh1 = open1 ? th_shift(qhi[1] - qlo[1]) : 0;
        for (int i = tid; i < 2 * TH_NW * 256; i += TH_NT) (&sh.hist[0][0][0])[i] = 0;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < TH_PER; ++i) {
            if (open0 && key[i] >= qlo[0] && key[i] <= qhi[0]) atomicAdd(&sh.hist[0][w][(key[i] - qlo[0]) >> sh0], 1);
            if (open1 && key[i] >= qlo[1] && key[i] <= qhi[1]) atomicAdd(&sh.hist[1][w][(key[i] - qlo[1]) >> sh1], 1);
        }
        __syncthreads();
        {  // per-wave histograms summed into wave slot 0 (thread t < 256 sums bin t of both ranks)
            int t0 = 0, t1 = 0;
            if (tid < 256) {
#pragma unroll
                for (int q = 0; q < TH_NW; ++q) {
                    t0 += sh.hist[0][q][tid];
                    t1 += sh.hist[1][q][tid];
                }
            }
            __syncthreads();
            if (tid < 256) {
                sh.hist[0][0][tid] = t0;
                sh.hist[1][0][tid] = t1;
            }
        }
        __syncthreads();
        if (w == 0 && open0) th_find(sh.hist[0][0], krem[0], 0, sh);
        if (w == 1 && open1) th_find(sh.hist[1][0], krem[1], 1, sh);
        __syncthreads();
        if (open0) {
            krem[0] -= sh.above[0];
            const unsigned nlo = qlo[0] + ((unsigned)sh.bin[0] << sh0);
            const unsigned top = nlo + ((1u << sh0) - 1u);
            qhi[0] = top < qhi[0] ? top : qhi[0];
            qlo[0] = nlo;
        }
        if (open1) {
            krem[1] -= sh.above[1];
            const unsigned nlo = qlo[1] + ((unsigned)sh.bin[1] << sh1);
            const unsigned top = nlo + ((1u << sh1) - 1u);
            qhi[1] = top < qhi[1] ? top : qhi[1];
            qlo[1] = nlo;
        }
        __syncthreads();
    }
    if (tid == 0) {
        a.theta_safe[b] = th_lower(key_to_score(qlo[0]));
        if (a.theta_fast != nullptr) a.theta_fast[b] = th_lower(key_to_score(qlo[1]));
    }
}

// Source: the candidate regions of one user's pieces, staged MG_PB pieces
// per batch in LDS.
template <int MG_PB>
struct PieceShared {
    int64_t base[MG_PB];
    int pref[MG_PB + 1];
    int wsum[SEL_NT / kWave];
};

template <int MG_PB>
struct PieceSrc {
    const uint64_t* keys;
    const int* pcnt;
    const int64_t* preg;
    int64_t p0, p1;
    int64_t n;  // total keys
    PieceShared<MG_PB>* ps;
    __device__ int64_t total() const { return n; }
    // Calls f(key, e) for every key, e = its index in the concatenation of
    // the pieces' regions.
    template <class F>
    __device__ void walk(F&& f) const {
        const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
        int ebase = 0;
        for (int64_t pb = p0; pb < p1; pb += MG_PB) {
            const int np = (int)min((int64_t)MG_PB, p1 - pb);
            // exclusive scan of the batch's counts (4 per thread)
            // (indices clamped into the batch, np >= 1: every load is in
            // flight before the first is used, none behind a branch of its own)
            int cv[MG_PB / SEL_NT];
            int64_t bv[MG_PB / SEL_NT];
#pragma unroll
            for (int i = 0; i < MG_PB / SEL_NT; ++i) {
                const int64_t p = pb + min(tid * (MG_PB / SEL_NT) + i, np - 1);
                cv[i] = pcnt[p];
                bv[i] = preg[p];
            }
            int tsum = 0;
#pragma unroll
            for (int i = 0; i < MG_PB / SEL_NT; ++i) {
                const int p = tid * (MG_PB / SEL_NT) + i;
                if (p < np) ps->base[p] = bv[i];
                else cv[i] = 0;
                tsum += cv[i];
            }
            int incl = tsum;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int t = __shfl_up(incl, o);
                if (lane >= o) incl += t;
            }
            if (lane == 63) ps->wsum[w] = incl;
            __syncthreads();
            int off = 0;
            for (int q = 0; q < w; ++q) off += ps->wsum[q];
            int run = off + incl - tsum;
#pragma unroll
            for (int i = 0; i < MG_PB / SEL_NT; ++i) {
                ps->pref[tid * (MG_PB / SEL_NT) + i] = run;
                run += cv[i];
            }
            if (tid == SEL_NT - 1) ps->pref[MG_PB] = run;
            __syncthreads();
            // Each thread walks one contiguous range of the batch's entries: one
            // binary search for its first piece, then forward across piece ends.
            const int tot = ps->pref[MG_PB];
            const int per = (tot + SEL_NT - 1) / SEL_NT;
            const int e_beg = min(tid * per, tot), e_end = min(e_beg + per, tot);
            if (e_beg < e_end) {
                int lo_p = 0, hi_p = np - 1;  // last piece with pref <= e_beg
                while (lo_p < hi_p) {
                    const int mid = (lo_p + hi_p + 1) >> 1;
                    if (ps->pref[mid] <= e_beg) lo_p = mid;
                    else hi_p = mid - 1;
                }
                int pi = lo_p;
                int next = ps->pref[pi + 1];
                int64_t off = ps->base[pi] - ps->pref[pi];  // entry e of piece pi is keys[off + e]
                for (int e0 = e_beg; e0 < e_end; e0 += SEL_UNR) {
                    // addresses first (LDS only), then the loads together; an
                    // entry past the range reads the range's last one again
                    int64_t at[SEL_UNR];
#pragma unroll
                    for (int q = 0; q < SEL_UNR; ++q) {
                        const int e = min(e0 + q, e_end - 1);
                        while (e >= next) {  // crossed into the next non-empty piece
                            ++pi;
                            next = ps->pref[pi + 1];
                            off = ps->base[pi] - ps->pref[pi];
                        }
                        at[q] = off + e;
                    }
                    uint64_t kv[SEL_UNR];
#pragma unroll
                    for (int q = 0; q < SEL_UNR; ++q) kv[q] = keys[at[q]];
#pragma unroll
                    for (int q = 0; q < SEL_UNR; ++q)
                        if (e0 + q < e_end) f(kv[q], ebase + e0 + q);
                }
            }
            ebase += tot;
            __syncthreads();
        }
    }
    template <class F>
    __device__ void for_each(F&& f) const {
        walk([&](uint64_t key, int) { f(key); });
    }
    // Every key to dst[e] (needs total() entries of room).
    __device__ void gather(uint64_t* dst) const {
        walk([&](uint64_t key, int e) { dst[e] = key; });
    }
};

// Merge builds: the default, and a smaller one (a 2,048-key gather and
// 512-piece batches: 37 instead of 76 KB of LDS, four blocks on a CU instead of
// two) for users expected to hold few pieces and candidates.  Either is exact
// for any input; the size only decides how fast.
constexpr int MG_GCAP_SMALL = kMergeSmallGather, MG_PB_SMALL = kMergeSmallPieces, MG_PB_LARGE = 1024;

template <int GCAP, int MG_PB>
__global__ __launch_bounds__(SEL_NT) void merge_kernel(MergeArgs a) {
    __shared__ SelSharedT<GCAP> sh;
    __shared__ PieceShared<MG_PB> ps;
    __shared__ float2 s_ml[SEL_NT / kWave];
    __shared__ unsigned long long s_n[SEL_NT / kWave];
    __shared__ int s_ovf[SEL_NT / kWave];
    __shared__ int s_slot;
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    if (a.mode == 2 && a.user_flag[b] == 0) return;  // rescue merge: flagged users only
    if (a.mode == 3 && a.nst[b].status == 0) return;  // bounded rescue merge: flagged users only
    if (b == 0 && tid == 0 && a.clear_err != nullptr) {
        a.clear_err[0] = 0;
        a.clear_err[1] = 0;
        // no threshold pass cleared the rescue count, and nothing adds to it
        if (a.mode == 0 && a.rescued != nullptr) *a.rescued = 0;
    }
    int64_t p0, p1;
    if (a.piece_begin != nullptr) {
        p0 = a.piece_begin[b];
        p1 = a.piece_begin[b + 1];
    } else {
        p0 = (int64_t)b * a.P;
        p1 = p0 + a.P;
    }
    const uint64_t* keys = a.keys;
    const int* pcnt = a.pcnt;
    const int64_t* preg = a.preg;
    unsigned long long ntot = 0;
    if (a.mode == 3) {
        // the keys collected for this user (its lse was written by mode 1)
        if (tid == 0 && a.ccnt[b] > a.ccol) a.ccnt[b] = a.ccol;
        __syncthreads();
        keys = a.coll;
        pcnt = a.ccnt;
        preg = a.cbase;
        p0 = b;
        p1 = b + 1;
        ntot = (unsigned long long)a.ccnt[b];
    } else {
    // lse and candidate count over the user's pieces
    LseState st;
    st.init();
    unsigned long long n = 0;
    int ovf = 0;  // bounded regions: the user's overflow region counted more keys than it holds
    // four pieces per thread and round, their loads issued together (indices
    // clamped into the user's pieces); merged in the same order as one by one
    for (int64_t pq = p0 + tid; pq < p1; pq += 4 * SEL_NT) {
        float pm4[4], pl4[4];
        int pc4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t p = min(pq + (int64_t)i * SEL_NT, p1 - 1);
            pm4[i] = a.pm[p];
            pl4[i] = a.pl[p];
            pc4[i] = a.pcnt[p];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (pq + (int64_t)i * SEL_NT < p1) {
                st.merge(pm4[i], pl4[i]);
                n += (unsigned long long)pc4[i];
                // (bounded regions: a user's last record is its overflow region's)
                ovf |= a.cap > 0 && pq + (int64_t)i * SEL_NT == p1 - 1 && pc4[i] > a.ovf_cap;
            }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const float m2 = __shfl_xor(st.m, o), l2 = __shfl_xor(st.l, o);
        st.merge(m2, l2);
        n += __shfl_xor(n, o);
        ovf |= __shfl_xor(ovf, o);
    }
    if (lane == 0) { s_ml[w] = make_float2(st.m, st.l); s_n[w] = n; s_ovf[w] = ovf; }
    __syncthreads();
    LseState tot;
    tot.init();
    ovf = 0;
    for (int q = 0; q < SEL_NT / kWave; ++q) { tot.merge(s_ml[q].x, s_ml[q].y); ntot += s_n[q]; ovf |= s_ovf[q]; }
    const bool short_k =
        a.mode == 1 && ntot < (unsigned long long)a.K && (!a.safe_exact || a.theta_fast[b] > a.theta_safe[b]);
    if (a.cap > 0 && a.mode == 1) {
        // bounded regions: every user's rescue state is (re)set here
        const bool flag = short_k || ovf;
        if (tid == 0) {
            NarrowState ns{};
            if (flag) {
                a.out_lse[b] = tot.l > 0.f ? tot.m + __builtin_amdgcn_logf(tot.l) * kLn2 : -INFINITY;
                // lower bound of the keys to consider: the fast threshold when
                // it let K keys through, else the K-th sampled score's (exact
                // sample) or every finite score
                const float tf = a.theta_fast[b], ts = a.theta_safe[b];
                const float tl = ntot >= (unsigned long long)a.K ? tf : (a.safe_exact ? fminf(ts, tf) : -FLT_MAX);
                ns.lo = (uint64_t)order_key(fmaxf(tl, -FLT_MAX)) << 32;
                const uint64_t hi = ((uint64_t)order_key(tot.m) << 32) | 0xFFFFFFFFull;  // the user's largest key
                ns.k_rem = a.K;
                if (tot.l == 0.f || hi < ns.lo || (ntot >= (unsigned long long)a.K && ntot <= (unsigned long long)a.ccol)) {
                    ns.status = 2;  // no key at all, or all of them fit: collect at once
                } else {
                    const uint64_t wdt = hi - ns.lo;
                    const int bits = 64 - __builtin_clzll(wdt | 1ull);
                    ns.shift = bits > kNarrowBits ? bits - kNarrowBits : 0;
                    ns.status = 1;
                    atomicAdd(a.rc, 1);  // one more user counting
                }
                a.ccnt[b] = 0;
                a.cbase[b] = (int64_t)b * a.ccol;
                a.user_flag[b] = 1;
                a.tile_flag[b / MF_TU] = 1;
                atomicAdd((unsigned long long*)a.rescued, 1ull);
                // the user's row joins the gathered rows of the rescue passes
                const int slot = atomicAdd(a.rc + 1, 1);
                a.map[slot] = b;
                s_slot = slot;
            }
            a.nst[b] = ns;
        }
        if (flag) {
            uint4* hrow = (uint4*)(a.hist + (int64_t)b * kNarrowBins);
            for (int i = tid; i < kNarrowBins / 4; i += SEL_NT) hrow[i] = make_uint4(0u, 0u, 0u, 0u);
            __syncthreads();
            const int slot = s_slot;
            const int64_t n16 = (int64_t)a.D * a.es / 16;  // 16-byte chunks of a row
            const uint4* src = (const uint4*)((const uint8_t*)a.H + (int64_t)b * a.D * a.es);
            uint4* dst = (uint4*)((uint8_t*)a.hgat + (int64_t)slot * a.D * a.es);
            for (int64_t i = tid; i < n16; i += SEL_NT) dst[i] = src[i];
            return;
        }
    }
    if (short_k) {
        // the fast threshold let fewer than K items through: the rescue pass
        // recomputes this user with the K-th sampled score (when that is
        // lower: else every item it would keep was kept, e.g. a user with
        // fewer than K allowed items)
        if (tid == 0) {
            a.user_flag[b] = 1;
            a.tile_flag[b / MF_TU] = 1;
            atomicAdd((unsigned long long*)a.rescued, 1ull);
        }
        return;
    }
    if (tid == 0)
        a.out_lse[b] = tot.l > 0.f ? tot.m + __builtin_amdgcn_logf(tot.l) * kLn2 : -INFINITY;
    }

    const int K = a.K;
    const int keff = (int)min((unsigned long long)K, ntot);
    int32_t* oidx = a.out_idx + (int64_t)b * K;
    float* osc = a.out_scores + (int64_t)b * K;
    if (keff > 0) {
        PieceSrc<MG_PB> src{keys, pcnt, preg, p0, p1, (int64_t)ntot, &ps};
        block_select<true>(src, keff, sh);
        // the K keys in ranking order: rank placement for a few hundred
        // (quadratic compares, one barrier), wave sorts and a rank merge for more
        if (keff <= 256) {
            block_rank_place(sh.out, keff, sh.gbuf, keff);
        } else {
            block_sort_into(sh.out, keff, sh.gbuf);
        }
        __syncthreads();
    }
    for (int i = tid; i < K; i += SEL_NT) {
        if (i < keff) {
            const uint64_t key = sh.gbuf[i];
            oidx[i] = (int32_t)key_id(key);
            osc[i] = key_score(key);
        } else {
            oidx[i] = -1;
            osc[i] = -INFINITY;
        }
    }
}

// One counting pass's pick for a flagged user over bounded regions: the bin
// holding the user's k_rem-th key from the top becomes the next range (its
// keys then split 4,096 ways), or, once the keys at or above the bin's start
// fit the collect region, the final bound.  Bins are 2^shift keys wide, so a
// range narrows 12 bits a pass and a bin of width 1 holds one key: at most
// six passes for 64-bit keys.  The histogram row is zeroed for the next pass.
constexpr int NR_NT = 256;
static_assert(kNarrowBins == NR_NT * 16, "16 bins per thread");

__global__ __launch_bounds__(NR_NT) void narrow_kernel(NarrowArgs a) {
    __shared__ uint32_t s_w[NR_NT / kWave];
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    if (a.nst[b].status != 1) return;
    const NarrowState st = a.nst[b];
    uint4* hrow = (uint4*)(a.hist + (int64_t)b * kNarrowBins) + tid * 4;  // bins 16 tid .. 16 tid + 15
    uint32_t v[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint4 q = hrow[i];
        v[4 * i] = q.x;
        v[4 * i + 1] = q.y;
        v[4 * i + 2] = q.z;
        v[4 * i + 3] = q.w;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) hrow[i] = make_uint4(0u, 0u, 0u, 0u);
    uint32_t tsum = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) tsum += v[i];
    uint32_t incl = tsum;  // inclusive prefix sum over the threads
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t t = __shfl_up(incl, o);
        if (lane >= o) incl += t;
    }
    if (lane == 63) s_w[w] = incl;
    __syncthreads();
    uint32_t total = 0;
    for (int q = 0; q < NR_NT / kWave; ++q) {
        if (q < w) incl += s_w[q];
        total += s_w[q];
    }
    const uint32_t above = total - incl;  // keys in the bins of the threads above this one
    const uint32_t kr = (uint32_t)st.k_rem;
    if (total < kr) {  // fewer keys than wanted at or above lo: keep them all
        if (tid == 0) {
            a.nst[b].status = 2;
            atomicSub(a.rc, 1);
        }
        return;
    }
    if (above < kr && kr <= above + tsum) {  // exactly one thread: the one holding the k_rem-th key
        bool found = false;
        uint32_t cum = above, cum_at = 0, vj = 0;
        int j = 0;
#pragma unroll
        for (int i = 15; i >= 0; --i) {
            if (!found && cum + v[i] >= kr) {
                found = true;
                j = tid * 16 + i;
                cum_at = cum;
                vj = v[i];
            }
            cum += v[i];
        }
        NarrowState ns = st;
        ns.lo = st.lo + ((uint64_t)j << st.shift);
        // keys at or above the bin's start: those above the range, those of
        // the bins above it and the bin's own
        const int64_t count_ge = (int64_t)(a.K - st.k_rem) + cum_at + vj;
        if (count_ge <= a.ccol || st.shift == 0) {
            ns.status = 2;
            atomicSub(a.rc, 1);
        } else {
            ns.k_rem = st.k_rem - (int)cum_at;
            ns.shift = st.shift > kNarrowBits ? st.shift - kNarrowBits : 0;
        }
        a.nst[b] = ns;
    }
}

// ---------------------------------------------------------------------------
// Batched top-K of dense score rows (beam step)
// ---------------------------------------------------------------------------
// Source: a segment of one fp32 score row; the key of column base + e is
// rank_key(score, base + e).
struct DenseRowSrc {
    const float* row;  // the segment's first score
    int64_t n;
    int64_t base;      // column of row[0]
    __device__ int64_t total() const { return n; }
    template <class F>
    __device__ void for_each(F&& f) const {
        for (int64_t e0 = threadIdx.x; e0 < n; e0 += (int64_t)SEL_NT * SEL_UNR) {
            float v[SEL_UNR];
#pragma unroll
            for (int q = 0; q < SEL_UNR; ++q)  // clamped (n >= 1 here): the loads are in flight together
                v[q] = row[min(e0 + (int64_t)q * SEL_NT, n - 1)];
#pragma unroll
            for (int q = 0; q < SEL_UNR; ++q) {
                const int64_t e = e0 + (int64_t)q * SEL_NT;
                if (e < n) f(rank_key(v[q], (uint32_t)(base + e)));
            }
        }
    }
    __device__ void gather(uint64_t* dst) const {
        for (int64_t e = threadIdx.x; e < n; e += SEL_NT) dst[e] = rank_key(row[e], (uint32_t)(base + e));
    }
};

// Source: the per-chunk partial results of one row, chunk c holding
// min(K, its length) keys at part + c * K.
struct PartialSrc {
    const uint64_t* part;
    int nchunk, K;
    int64_t N, C;
    __device__ int cnt(int c) const { return (int)min((int64_t)K, min(C, N - (int64_t)c * C)); }
    __device__ int64_t total() const {
        int64_t t = 0;
        for (int c = 0; c < nchunk; ++c) t += cnt(c);
        return t;
    }
    template <class F>
    __device__ void walk(F&& f) const {
        int e = 0;
        for (int c = 0; c < nchunk; ++c) {
            const int n = cnt(c);
            for (int i = threadIdx.x; i < n; i += SEL_NT) f(part[(int64_t)c * K + i], e + i);
            e += n;
        }
    }
    template <class F>
    __device__ void for_each(F&& f) const {
        walk([&](uint64_t key, int) { f(key); });
    }
    __device__ void gather(uint64_t* dst) const {
        walk([&](uint64_t key, int e) { dst[e] = key; });
    }
};

// The k largest keys of a source in ranking order, written out (or, for an
// intermediate chunk, as raw keys).
template <class Src, class Sh>
__device__ void topk_emit(const Src& src, int k, int K, Sh& sh, int32_t* oidx, float* osc, uint64_t* okeys) {
    const int tid = threadIdx.x;
    if (k > 0) {
        block_select<true>(src, k, sh);
        if (okeys != nullptr) {  // partial result: any order
            for (int i = tid; i < k; i += SEL_NT) okeys[i] = sh.out[i];
            return;
        }
        if (k <= 256) {
            block_rank_place(sh.out, k, sh.gbuf, k);
        } else {
            block_sort_into(sh.out, k, sh.gbuf);
        }
        __syncthreads();
    }
    for (int i = tid; i < K; i += SEL_NT) {
        if (i < k) {
            const uint64_t key = sh.gbuf[i];
            oidx[i] = (int32_t)key_id(key);
            osc[i] = key_score(key);
        } else {
            oidx[i] = -1;
            osc[i] = -INFINITY;
        }
    }
}

// Block (r, c): the top-K of chunk c of row r -- the final result when the row
// is one chunk, else its keys for the merge.  GCAP: the selection's LDS
// gather; the smaller build fits about twice the blocks on a CU, which pays
// for small K (width-128 beam step 51 -> 43 us) and not for K of 512 or more.
template <int GCAP>
__global__ __launch_bounds__(SEL_NT) void topk_chunk_kernel(TopkRowsArgs a) {
    __shared__ SelSharedT<GCAP> sh;
    const int r = blockIdx.x / a.nchunk, c = blockIdx.x - r * a.nchunk;
    const int64_t c0 = (int64_t)c * a.C;
    const int64_t n = min(a.C, a.N - c0);
    DenseRowSrc src{a.scores + (int64_t)r * a.ld + c0, n, c0};
    const int k = (int)min((int64_t)a.K, n);
    if (a.nchunk == 1)
        topk_emit(src, k, a.K, sh, a.out_idx + (int64_t)r * a.K, a.out_scores + (int64_t)r * a.K, nullptr);
    else
        topk_emit(src, k, a.K, sh, nullptr, nullptr, a.part + ((int64_t)r * a.nchunk + c) * a.K);
}

// Block r: the top-K of the row's chunk results.
__global__ __launch_bounds__(SEL_NT) void topk_merge_rows_kernel(TopkRowsArgs a) {
    __shared__ SelShared sh;
    const int r = blockIdx.x;
    PartialSrc src{a.part + (int64_t)r * a.nchunk * a.K, a.nchunk, a.K, a.N, a.C};
    const int k = (int)min((int64_t)a.K, a.N);
    topk_emit(src, k, a.K, sh, a.out_idx + (int64_t)r * a.K, a.out_scores + (int64_t)r * a.K, nullptr);
}

// ---------------------------------------------------------------------------
// Batched top-K by register-resident radix selection
// ---------------------------------------------------------------------------
// A block of TK_NT threads holds up to TK_NT * V keys in registers (V per
// thread; slot j of thread t is key j * TK_NT + t) and narrows down the k-th
// largest by deciding its bits from the top.  For each bit it counts the keys
// that agree with the bits decided so far and have this bit set (a ballot
// and a scalar popcount per key and wave, one barrier to add the four waves'
// counts) and sets the bit when they are at least the k still wanted.  It
// stops as soon as the keys that agree with the decided bits (the group) are
// all wanted, or are at most TK_SMALL: the group is then ranked in LDS by
// plain comparison.  Only when more than TK_SMALL keys share one score word
// is the index word decided the same way.  Per bit that is two vector
// instructions per key, with no atomics.  Keys are the 64-bit ranking keys
// (score word, inverted column) of the dense path, so the order is the same.
constexpr int TK_NT = 256;
constexpr int TK_V = 64;              // keys per thread of a row segment
constexpr int TK_SEG = TK_NT * TK_V;  // columns per segment block
constexpr int TK_MV = 32;             // keys per thread of the row merge
constexpr int TK_SMALL = 256;         // group size ranked by comparison
static_assert(TK_SEG == kTopkSeg && TK_NT * TK_MV == kTopkMergeKeys, "the plan's segment and merge sizes");
static_assert(TK_NT == SEL_NT, "the final sort is the selection's block sort");

struct TkShared {
    int cnt[2][TK_NT / kWave];
    int wsel[TK_NT / kWave];
    uint64_t grp[TK_SMALL];        // the group, when it is ranked by comparison
    alignas(16) uint64_t sel[GENREC_KMAX];  // the k selected keys (read two at a time)
    uint64_t sorted[GENREC_KMAX];  // the same in ranking order
};

// Block sum of one wave-uniform count per wave.  `par` alternates between
// calls: a wave that has passed this call's barrier writes the other slot
// next time, while slow waves may still be reading this one.
__device__ __forceinline__ int tk_block_sum(int c, int& par, TkShared& sh) {
    if ((threadIdx.x & 63) == 0) sh.cnt[par][threadIdx.x >> 6] = c;
    __syncthreads();
    int t = 0;
#pragma unroll
    for (int q = 0; q < TK_NT / kWave; ++q) t += sh.cnt[par][q];
    par ^= 1;
    return t;
}

// Bit decisions from the top for the krem-th largest of the words w(j) over
// the slots with in(j) (m of them, m >= krem >= 1), until the group -- the
// slots whose word agrees with the decided bits -- is wholly wanted
// (m == krem) or holds at most `small` slots.  On return `mask` marks the
// decided bits, P holds them (zeros elsewhere), m is the group's size and
// krem the number wanted from it; the slots above the group are all wanted.
template <int V, class W, class In>
__device__ __forceinline__ void tk_radix(const W& w, const In& in, int small, int& m, int& krem, uint32_t& P,
                                         uint32_t& mask, int& par, TkShared& sh) {
    P = 0;
    mask = 0;
    for (int b = 31; b >= 0 && m != krem && m > small; --b) {
        const uint32_t t = (P >> b) | 1u;  // the decided bits, then bit b set
        int c = 0;
#pragma unroll
        for (int j = 0; j < V; ++j) {
            c += __popcll(__ballot(in(j) && (w(j) >> b) == t));
            // a few compare results live at a time (not all V in scalar registers)
            if ((j & 7) == 7) __builtin_amdgcn_sched_barrier(0);
        }
        c = tk_block_sum(c, par, sh);
        mask |= 1u << b;
        if (c >= krem) {
            P |= 1u << b;
            m = c;
        } else {
            krem -= c;
            m -= c;
        }
    }
}

// Slots with pred(j) to dst[0..), key(j) each, in no particular order (at most
// cap written); returns how many there are.
template <int V, class Pred, class Key>
__device__ __forceinline__ int tk_compact(const Pred& pred, const Key& key, uint64_t* dst, int cap, TkShared& sh) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int c = 0;
#pragma unroll
    for (int j = 0; j < V; ++j) {
        c += __popcll(__ballot(pred(j)));
        if ((j & 7) == 7) __builtin_amdgcn_sched_barrier(0);
    }
    if (lane == 0) sh.wsel[w] = c;
    __syncthreads();
    int base = 0, total = 0;
#pragma unroll
    for (int q = 0; q < TK_NT / kWave; ++q) {
        base += q < w ? sh.wsel[q] : 0;
        total += sh.wsel[q];
    }
#pragma unroll
    for (int j = 0; j < V; ++j) {
        const bool s = pred(j);
        const uint64_t bm = __ballot(s);
        const int pos = base + __popcll(bm & ((1ull << lane) - 1ull));
        if (s && pos < cap) dst[pos] = key(j);
        base += __popcll(bm);
    }
    __syncthreads();
    return total;
}

// The k largest of the valid keys (n_valid >= k >= 1) into sh.sel[0..k), in
// no particular order.  hi(j) / lo(j): the key words of slot j; valid(j): the
// slot holds a key.  Invalid slots must have hi(j) == 0, which never agrees
// with a decided set bit, so the score-word decisions need no validity test.
template <int V, class Hi, class Lo, class Valid>
__device__ __forceinline__ void tk_select(const Hi& hi, const Lo& lo, const Valid& valid, int n_valid, int k,
                                          TkShared& sh) {
    int par = 0;
    int m = n_valid, krem = k;
    uint32_t P, pmask;
    tk_radix<V>(hi, [](int) { return true; }, TK_SMALL, m, krem, P, pmask, par, sh);
    auto key = [&](int j) { return ((uint64_t)hi(j) << 32) | lo(j); };
    if (m == krem) {
        tk_compact<V>([&](int j) { return valid(j) && (hi(j) & pmask) >= P; }, key, sh.sel, GENREC_KMAX, sh);
    } else if (m <= TK_SMALL) {
        // the keys above the group, then the krem largest of the group
        const int above = k - krem;
        tk_compact<V>([&](int j) { return valid(j) && (hi(j) & pmask) > P; }, key, sh.sel, above, sh);
        tk_compact<V>([&](int j) { return valid(j) && (hi(j) & pmask) == P; }, key, sh.grp, TK_SMALL, sh);
        block_rank_place(sh.grp, m, sh.sel + above, krem);
        __syncthreads();
    } else {
        // more than TK_SMALL keys share the score word P (every bit decided):
        // the krem lowest columns among them, i.e. the largest index words
        uint32_t Q, qmask;
        tk_radix<V>(lo, [&](int j) { return valid(j) && hi(j) == P; }, 0, m, krem, Q, qmask, par, sh);
        tk_compact<V>([&](int j) { return valid(j) && (hi(j) > P || (hi(j) == P && (lo(j) & qmask) >= Q)); }, key,
                      sh.sel, GENREC_KMAX, sh);
    }
}

// sh.sel[0..k) in ranking order to the row's outputs, padded to K.
__device__ void tk_emit(int k, int K, TkShared& sh, int32_t* oidx, float* osc) {
    if (k <= 256) block_rank_place(sh.sel, k, sh.sorted, k);
    else block_sort_into(sh.sel, k, sh.sorted);
    __syncthreads();
    for (int i = threadIdx.x; i < K; i += TK_NT) {
        if (i < k) {
            const uint64_t key = sh.sorted[i];
            oidx[i] = (int32_t)key_id(key);
            osc[i] = key_score(key);
        } else {
            oidx[i] = -1;
            osc[i] = -INFINITY;
        }
    }
}

// The k largest of a block's keys (V slots a thread, k <= 1,024 groups; the
// one-block row route for 256 < k <= 512)
// when a bound leaves few enough: each thread's slots form four groups, T =
// the k-th largest of the 1,024 group maxima (one block sort), and k groups
// hold a key >= T, so the k largest keys are among the keys that reach T --
// for unordered scores about 1.35 k of them at k = 512.  Those are compacted
// (whole 64-bit keys) and sorted into sh.sorted; returns how many (>= k).
// More than GENREC_KMAX keys at T (exact ties): returns -1, having written
// only LDS scratch.  hi(j): slot j's order key (0: no key); key(j): its
// 64-bit key.
template <int V, class Hi, class Key>
__device__ __forceinline__ int tk_bound_sort(const Hi& hi, const Key& key, int k, TkShared& sh) {
    static_assert(V % 4 == 0 && V <= 64 && 4 * TK_NT <= GENREC_KMAX, "four groups a thread, a 64-bit pass mask");
    constexpr int GK = V / 4;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        uint32_t m = 0u;
#pragma unroll
        for (int j = q * GK; j < (q + 1) * GK; ++j) m = max(m, hi(j));
        sh.sel[tid * 4 + q] = ((uint64_t)m << 32) | (uint32_t)(tid * 4 + q);
    }
    __syncthreads();
    block_sort_into(sh.sel, 4 * TK_NT, sh.sorted);
    __syncthreads();
    const uint32_t T = (uint32_t)(sh.sorted[k - 1] >> 32);  // 0 when fewer than k groups hold a key: every key
    uint64_t mask = 0;
#pragma unroll
    for (int j = 0; j < V; ++j) mask |= (hi(j) != 0u && hi(j) >= T) ? (1ull << j) : 0ull;
    const int c = __popcll(mask);
    int incl = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(incl, o);
        if (lane >= o) incl += t;
    }
    if (lane == 63) sh.wsel[w] = incl;
    __syncthreads();
    int base = incl - c, total = 0;
#pragma unroll
    for (int q = 0; q < TK_NT / kWave; ++q) {
        base += q < w ? sh.wsel[q] : 0;
        total += sh.wsel[q];
    }
    __syncthreads();  // the counts are read before anyone reuses them
    if (total > GENREC_KMAX) return -1;  // block-uniform
#pragma unroll
    for (int j = 0; j < V; ++j)
        if ((mask >> j) & 1ull) sh.sel[base++] = key(j);
    __syncthreads();
    block_sort_into(sh.sel, total, sh.sorted);
    __syncthreads();
    return total;
}

// Order keys of a row's first n >= 1 scores, slot j of thread t holding
// column j * TK_NT + t (key 0 past the row).  Every load is issued before
// the first is used: a slot past the row reads the row's last score and
// drops it, where a guarded load would sit behind a branch of its own and be
// waited for before the next one starts (64 round trips to memory in turn).
template <int V>
__device__ __forceinline__ void load_row_keys(const float* row, int n, uint32_t (&hv)[V]) {
    const int tid = threadIdx.x;
    float v[V];
#pragma unroll
    for (int j = 0; j < V; ++j) v[j] = row[min(j * TK_NT + tid, n - 1)];
#pragma unroll
    for (int j = 0; j < V; ++j) hv[j] = j * TK_NT + tid < n ? order_key(v[j]) : 0u;
}

// Block (r, s): the top-K keys of segment s (TK_SEG columns) of row r for the
// row merge, in no particular order (all K places written, zero keys past the
// segment's count).
__global__ __launch_bounds__(TK_NT) void topk_seg_kernel(TopkRowsArgs a) {
    __shared__ TkShared sh;
    const int tid = threadIdx.x;
    const int r = blockIdx.x / a.nchunk, s = blockIdx.x - r * a.nchunk;
    const int64_t c0 = (int64_t)s * TK_SEG;
    const int n = (int)min((int64_t)TK_SEG, a.N - c0);
    const float* row = a.scores + (int64_t)r * a.ld + c0;
    uint32_t hv[TK_V];
    load_row_keys<TK_V>(row, n, hv);
    // Opaque from here on: otherwise the compiler carries "slot past the row
    // => word 0" into every bit decision and keeps all V row-end masks live
    // in scalar registers (spilled) across the whole selection.
#pragma unroll
    for (int j = 0; j < TK_V; ++j) asm volatile("" : "+v"(hv[j]));
    const uint32_t lo0 = 0xFFFFFFFFu - (uint32_t)(c0 + tid);  // index word of slot 0
    const int k = min(a.K, n);
    uint64_t* dst = a.part + ((int64_t)r * a.nchunk + s) * a.K;
    // (the bound from group maxima, which serves whole rows, measured slower
    // here: its two block sorts cost what the bit decisions do)
    tk_select<TK_V>([&](int j) { return hv[j]; }, [&](int j) { return lo0 - (uint32_t)(j * TK_NT); },
                    [&](int j) {
                        // recomputed at each use (an opaque copy of the thread
                        // index), not kept as V live masks across the selection
                        int t = tid;
                        asm volatile("" : "+v"(t));
                        return j * TK_NT + t < n;
                    },
                    n, k, sh);
    for (int i = tid; i < a.K; i += TK_NT) dst[i] = i < k ? sh.sel[i] : 0ull;
}

// Block r: the whole row (N <= TK_SEG) in registers, its top-K written out.
// For K <= 256: T = the K-th largest of the threads' maxima (at least K keys
// reach it, so the top K are among the keys >= T -- for unordered scores a
// few times K of them), compacted into LDS and ranked; K <= 512: the bound
// from 1,024 group maxima; more than the LDS list holds (heavy ties), or
// K > 512: the bit-by-bit selection.
struct TkRowShared {
    TkShared tk;
    uint32_t tmax[TK_NT];
    uint32_t tred[TK_NT / kWave];
    int wcnt[TK_NT / kWave];
};

__global__ __launch_bounds__(TK_NT) void topk_row_kernel(TopkRowsArgs a) {
    __shared__ TkRowShared srow;
    TkShared& sh = srow.tk;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int r = blockIdx.x;
    const int n = (int)a.N;
    const float* row = a.scores + (int64_t)r * a.ld;
    uint32_t hv[TK_V];
    load_row_keys<TK_V>(row, n, hv);
#pragma unroll
    for (int j = 0; j < TK_V; ++j) asm volatile("" : "+v"(hv[j]));  // as in the segment kernel
    const int K = a.K;
    const int k = min(K, n);
    int32_t* oidx = a.out_idx + (int64_t)r * K;
    float* osc = a.out_scores + (int64_t)r * K;
    if (K <= TK_SMALL) {  // block-uniform
        uint32_t mx = 0u;
#pragma unroll
        for (int j = 0; j < TK_V; ++j) mx = max(mx, hv[j]);
        srow.tmax[tid] = mx;
        __syncthreads();
        // rank of this thread's maximum among all of them (strictly larger);
        // a thread without keys has maximum 0, which qualifies only when fewer
        // than K threads hold a key: then T = 0 admits every key
        int rk = 0;
        const uint4* t4 = (const uint4*)srow.tmax;
#pragma unroll 8
        for (int q = 0; q < TK_NT / 4; ++q) {
            const uint4 v = t4[q];
            rk += (v.x > mx) + (v.y > mx) + (v.z > mx) + (v.w > mx);
        }
        uint32_t tc = rk < K ? mx : 0xFFFFFFFFu;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) tc = min(tc, (uint32_t)__shfl_xor((int)tc, o));
        if (lane == 0) srow.tred[w] = tc;
        __syncthreads();
        uint32_t T = srow.tred[0];
#pragma unroll
        for (int q = 1; q < TK_NT / kWave; ++q) T = min(T, srow.tred[q]);
        // keys >= T: a 64-bit mask per thread, counted and scanned
        uint64_t mask = 0;
#pragma unroll
        for (int j = 0; j < TK_V; ++j) mask |= (hv[j] != 0u && hv[j] >= T) ? (1ull << j) : 0ull;
        const int c = __popcll(mask);
        int incl = c;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int t = __shfl_up(incl, o);
            if (lane >= o) incl += t;
        }
        if (lane == 63) srow.wcnt[w] = incl;
        __syncthreads();
        int base = incl - c, total = 0;
#pragma unroll
        for (int q = 0; q < TK_NT / kWave; ++q) {
            base += q < w ? srow.wcnt[q] : 0;
            total += srow.wcnt[q];
        }
        if (total <= GENREC_KMAX) {  // block-uniform
            // slot by slot (a constant index keeps hv in registers; a loop
            // over the mask's set bits would index it at run time)
            const uint32_t lo0 = 0xFFFFFFFFu - (uint32_t)tid;  // index word of slot 0
#pragma unroll
            for (int j = 0; j < TK_V; ++j)
                if ((mask >> j) & 1ull) sh.sel[base++] = ((uint64_t)hv[j] << 32) | (uint64_t)(lo0 - (uint32_t)(j * TK_NT));
            __syncthreads();
            // total >= k (T = 0 when fewer than K keys exist).  Up to 256 keys:
            // each one's rank = the keys above it (all distinct: the index
            // word), two per 16-byte read; more: wave sorts and a rank merge.
            // (256 rows of 16,384: 13.7 us; 14.7 with the sort for all,
            // 18.0 with the general rank placement.)
            if (total <= TK_NT) {
                if (tid < total) {
                    const uint64_t x = sh.sel[tid];
                    int rk2 = 0;
                    const ulonglong2* c2 = (const ulonglong2*)sh.sel;
#pragma unroll 4
                    for (int j = 0; j < total / 2; ++j) {
                        const ulonglong2 y = c2[j];
                        rk2 += (y.x > x) + (y.y > x);
                    }
                    if (total & 1) rk2 += sh.sel[total - 1] > x ? 1 : 0;
                    if (rk2 < k) sh.sorted[rk2] = x;
                }
            } else {
                block_sort_into(sh.sel, total, sh.sorted);
            }
            __syncthreads();
            for (int i = tid; i < K; i += TK_NT) {
                if (i < k) {
                    const uint64_t key = sh.sorted[i];
                    oidx[i] = (int32_t)key_id(key);
                    osc[i] = key_score(key);
                } else {
                    oidx[i] = -1;
                    osc[i] = -INFINITY;
                }
            }
            return;
        }
        __syncthreads();  // the counts above are read before the selection reuses the buffers
    } else if (K <= kTopkBoundMaxK) {  // block-uniform
        const uint32_t lo0 = 0xFFFFFFFFu - (uint32_t)tid;
        const int got = tk_bound_sort<TK_V>(
            [&](int j) { return hv[j]; },
            [&](int j) { return ((uint64_t)hv[j] << 32) | (uint64_t)(lo0 - (uint32_t)(j * TK_NT)); }, k, sh);
        if (got >= 0) {
            for (int i = tid; i < K; i += TK_NT) {
                if (i < k) {
                    const uint64_t key = sh.sorted[i];
                    oidx[i] = (int32_t)key_id(key);
                    osc[i] = key_score(key);
                } else {
                    oidx[i] = -1;
                    osc[i] = -INFINITY;
                }
            }
            return;
        }
    }
    const uint32_t lo0 = 0xFFFFFFFFu - (uint32_t)tid;
    if (k > 0)
        tk_select<TK_V>([&](int j) { return hv[j]; }, [&](int j) { return lo0 - (uint32_t)(j * TK_NT); },
                        [&](int j) {
                            int t = tid;
                            asm volatile("" : "+v"(t));
                            return j * TK_NT + t < n;
                        },
                        n, k, sh);
    tk_emit(k, K, sh, oidx, osc);
}

// Block r: the top-K of the row's segment results (nchunk * K <= TK_NT * TK_MV
// keys, zero keys in unused places).
__global__ __launch_bounds__(TK_NT) void topk_rowmerge_kernel(TopkRowsArgs a) {
    __shared__ TkShared sh;
    const int tid = threadIdx.x;
    const int r = blockIdx.x;
    const int total = a.nchunk * a.K;
    const uint64_t* src = a.part + (int64_t)r * total;
    uint32_t kh[TK_MV], kl[TK_MV];
    uint64_t kv[TK_MV];
#pragma unroll
    for (int j = 0; j < TK_MV; ++j) kv[j] = src[min(j * TK_NT + tid, total - 1)];  // clamped, as in load_row_keys
#pragma unroll
    for (int j = 0; j < TK_MV; ++j) {
        const uint64_t key = j * TK_NT + tid < total ? kv[j] : 0ull;
        kh[j] = (uint32_t)(key >> 32);
        kl[j] = (uint32_t)key;
        asm volatile("" : "+v"(kh[j]), "+v"(kl[j]));  // as in the segment kernel
    }
    // keys held: K from every segment but the last, which holds min(K, its length)
    const int64_t n_last = a.N - (int64_t)(a.nchunk - 1) * TK_SEG;
    const int n_valid = (a.nchunk - 1) * a.K + (int)min((int64_t)a.K, n_last);
    const int k = (int)min((int64_t)a.K, a.N);
    // a real key is never zero (its index word is at least 2^31)
    tk_select<TK_MV>([&](int j) { return kh[j]; }, [&](int j) { return kl[j]; },
                     [&](int j) { return (kh[j] | kl[j]) != 0u; }, n_valid, k, sh);
    tk_emit(k, a.K, sh, a.out_idx + (int64_t)r * a.K, a.out_scores + (int64_t)r * a.K);
}

// ---------------------------------------------------------------------------
// Batched top-K, filter route (long rows, K <= 512): a sampled bound per row,
// the keys at or above it listed, the list ranked
// ---------------------------------------------------------------------------
constexpr int TF_CAP = TK_NT * TK_MV;  // keys of a row's list (one per slot of the ranking block)
constexpr int TF_NSUB = kWave;         // the list's parts: part s takes the columns = s (mod 64)
constexpr int TF_SUB = TF_CAP / TF_NSUB;
constexpr int TF_COLS = 4096;          // columns per filter block
constexpr int TF_V = TF_COLS / TK_NT;
static_assert(TF_CAP == kTopkFiltCap && TF_COLS == kTopkFiltCols && TF_NSUB == kTopkFiltParts,
              "the plan's list, list parts and filter block sizes");
static_assert(TF_COLS % kWave == 0 && TK_NT % kWave == 0, "lane l of every filter wave reads columns = l (mod 64)");

// Block r: the bound of row r.  Slot j of thread t samples column
// q * (N / 256) + (t & 63) with run q = 4 j + t / 64, so each wave reads 64
// contiguous columns per slot and the 256 runs spread evenly over the row
// (N > 16,384: a run never passes the row's end).  T = the sj-th largest of
// the threads' sample maxima, found as in the row kernel (each thread ranks
// its maximum against all of them); at least sj sampled keys reach it.
__global__ __launch_bounds__(TK_NT) void topk_sample_kernel(TopkRowsArgs a) {
    __shared__ __align__(16) uint32_t tmax[TK_NT];  // read 16 bytes at a time
    __shared__ uint32_t tred[TK_NT / kWave];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int r = blockIdx.x;
    const int64_t rs = a.N / 256;
    const float* row = a.scores + (int64_t)r * a.ld + lane;
    float v[TK_V];
#pragma unroll
    for (int j = 0; j < TK_V; ++j) v[j] = row[(int64_t)(4 * j + w) * rs];
    uint32_t mx = 0u;
#pragma unroll
    for (int j = 0; j < TK_V; ++j) mx = max(mx, order_key(v[j]));
    tmax[tid] = mx;
    __syncthreads();
    int rk = 0;
    const uint4* t4 = (const uint4*)tmax;
#pragma unroll 8
    for (int q = 0; q < TK_NT / 4; ++q) {
        const uint4 u = t4[q];
        rk += (u.x > mx) + (u.y > mx) + (u.z > mx) + (u.w > mx);
    }
    uint32_t tc = rk < a.sj ? mx : 0xFFFFFFFFu;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) tc = min(tc, (uint32_t)__shfl_xor((int)tc, o));
    if (lane == 0) tred[w] = tc;
    __syncthreads();
    if (tid == 0) {
        uint32_t T = tred[0];
#pragma unroll
        for (int q = 1; q < TK_NT / kWave; ++q) T = min(T, tred[q]);
        a.tthr[r] = T;
    }
    if (tid < TF_NSUB) a.tcnt[(int64_t)r * TF_NSUB + tid] = 0;
}

// Block (r, b): columns [b TF_COLS, (b + 1) TF_COLS) of row r; every key at
// or above the row's bound is listed.  The list has 64 parts of TF_SUB keys;
// lane l of every wave reads columns = l (mod 64) and appends its keys to
// part l with one atomic add on that part's count, so a row's appends spread
// over 64 counters (one counter per row, taken by every wave, made this pass
// 153 instead of 21 us on 64 rows of 262,144) and the keys of any run of
// columns over all parts.  Keys past a
// full part are counted, not written: the ranking block then takes the whole
// row.
__global__ __launch_bounds__(TK_NT) void topk_filter_kernel(TopkRowsArgs a) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int r = blockIdx.x / a.nchunk, b = blockIdx.x - r * a.nchunk;
    const int64_t c0 = (int64_t)b * TF_COLS;
    const int n = (int)min((int64_t)TF_COLS, a.N - c0);
    const float* row = a.scores + (int64_t)r * a.ld + c0;
    const uint32_t T = a.tthr[r];
    float v[TF_V];
#pragma unroll
    for (int j = 0; j < TF_V; ++j) v[j] = row[min(j * TK_NT + tid, n - 1)];  // clamped: all in flight together
    uint32_t hv[TF_V];
    uint32_t mask = 0u;
#pragma unroll
    for (int j = 0; j < TF_V; ++j) {
        hv[j] = order_key(v[j]);
        mask |= (j * TK_NT + tid < n && hv[j] >= T) ? (1u << j) : 0u;
    }
    const int c = __popc(mask);
    if (c == 0) return;
    int pos = atomicAdd(a.tcnt + (int64_t)r * TF_NSUB + lane, c);
    uint64_t* dst = a.part + (int64_t)r * TF_CAP + lane * TF_SUB;
    const uint32_t lo0 = 0xFFFFFFFFu - (uint32_t)(c0 + tid);  // index word of slot 0
#pragma unroll
    for (int j = 0; j < TF_V; ++j) {
        if ((mask >> j) & 1u) {
            if (pos < TF_SUB) dst[pos] = ((uint64_t)hv[j] << 32) | (uint64_t)(lo0 - (uint32_t)(j * TK_NT));
            ++pos;
        }
    }
}

static_assert(SEL_NT == TK_NT, "the ranking block's fallback runs the histogram narrowing with its threads");

constexpr int TF_BITS = 11;              // key bits decided per ranking pass
constexpr int TF_BINS = 1 << TF_BITS;
struct TfRank {
    int hist[TF_BINS];
    int wsum[TK_NT / kWave];
    int bin, above;
    alignas(16) uint64_t sel[GENREC_KMAX];  // the k selected keys (room for block_sort_into's runs)
    uint64_t sorted[GENREC_KMAX];
};

union TfShared {
    TkShared tk;
    SelShared sel;
    TfRank rk;
};

// The k-th largest of the block's keys (slot j of each thread; 0: no key;
// all keys distinct, at least k of them), decided TF_BITS bits at a time from
// the top: a histogram of the keys that agree with the bits decided so far,
// then the bin that holds the k-th of them.  Stops early once that bin holds
// exactly the keys still wanted; returns T with exactly k keys >= T.
template <int V, class Key>
__device__ __forceinline__ uint64_t tf_kth_key(const Key& key, int k, TfRank& sh) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    constexpr int PER = TF_BINS / TK_NT;  // bins per thread, counted from the top
    uint64_t prefix = 0, dmask = 0;
    int k_rem = k;
    for (int shift = 64; shift > 0;) {
        const int nb = min(TF_BITS, shift);
        shift -= nb;
#pragma unroll
        for (int i = 0; i < PER; ++i) sh.hist[i * TK_NT + tid] = 0;
        __syncthreads();
#pragma unroll
        for (int j = 0; j < V; ++j) {
            const uint64_t x = key(j);
            if (x != 0ull && ((x ^ prefix) & dmask) == 0ull) atomicAdd(&sh.hist[(int)(x >> shift) & ((1 << nb) - 1)], 1);
        }
        __syncthreads();
        // thread t owns bins TF_BINS - 1 - (PER t + i), i < PER (higher bins first)
        int h[PER], tsum = 0;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            h[i] = sh.hist[TF_BINS - 1 - (PER * tid + i)];
            tsum += h[i];
        }
        int incl = tsum;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int t = __shfl_up(incl, o);
            if (lane >= o) incl += t;
        }
        if (lane == 63) sh.wsum[w] = incl;
        __syncthreads();
        int run = incl - tsum;
#pragma unroll
        for (int q = 0; q < TK_NT / kWave; ++q) run += q < w ? sh.wsum[q] : 0;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            if (run < k_rem && k_rem <= run + h[i]) {  // exactly one bin of one thread
                sh.bin = TF_BINS - 1 - (PER * tid + i);
                sh.above = run;
            }
            run += h[i];
        }
        __syncthreads();
        const int d = sh.bin, above = sh.above;
        const int in_bin = sh.hist[d];
        __syncthreads();  // the histogram and the choice are read before the next pass rewrites them
        prefix |= (uint64_t)d << shift;
        dmask |= (uint64_t)((1 << nb) - 1) << shift;
        k_rem -= above;
        if (in_bin == k_rem) break;  // every key of the bin is wanted: T = the bin's lowest key bound
    }
    return prefix;
}

// Block r: the top K of row r from its list.  Slot j of thread t is group
// g = 4 t + j / 8 (tk_bound_sort's groups), place j % 8; it reads key
// g / 64 + 16 (j % 8) of list part g % 64, so that the keys at the front of
// every part are shared evenly by the groups and the bound from the 1,024
// group maxima admits few more than K keys.  A list shorter than K keys or
// a part that overflowed: the histogram narrowing over the whole row.
__global__ __launch_bounds__(TK_NT) void topk_cand_kernel(TopkRowsArgs a) {
    __shared__ TfShared sh;
    __shared__ int s_tot, s_max;
    const int tid = threadIdx.x;
    const int r = blockIdx.x;
    const int K = a.K;
    const int k = (int)min((int64_t)K, a.N);
    int32_t* oidx = a.out_idx + (int64_t)r * K;
    float* osc = a.out_scores + (int64_t)r * K;
    const int* pc = a.tcnt + (int64_t)r * TF_NSUB;
    if (tid < kWave) {  // wave 0: the parts' total and largest count
        int t = pc[tid], m = t;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
            t += __shfl_xor(t, o);
            m = max(m, __shfl_xor(m, o));
        }
        if (tid == 0) {
            s_tot = t;
            s_max = m;
        }
    }
    __syncthreads();
    const int cnt = s_tot;
    if (cnt < k || s_max > TF_SUB) {  // block-uniform
        DenseRowSrc src{a.scores + (int64_t)r * a.ld, a.N, 0};
        topk_emit(src, k, K, sh.sel, oidx, osc, nullptr);
        return;
    }
    const uint64_t* lst = a.part + (int64_t)r * TF_CAP;
    constexpr int GK = TK_MV / 4;
    int pcnt[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) pcnt[q] = pc[(4 * tid + q) % TF_NSUB];
    uint64_t kv[TK_MV];
#pragma unroll
    for (int j = 0; j < TK_MV; ++j) {  // every place is inside the list; unwritten ones are dropped below
        const int g = 4 * tid + j / GK;
        kv[j] = lst[(g % TF_NSUB) * TF_SUB + g / TF_NSUB + (TK_NT * 4 / TF_NSUB) * (j % GK)];
    }
    uint32_t kh[TK_MV], kl[TK_MV];
#pragma unroll
    for (int j = 0; j < TK_MV; ++j) {
        const int g = 4 * tid + j / GK;
        const uint64_t key = g / TF_NSUB + (TK_NT * 4 / TF_NSUB) * (j % GK) < pcnt[j / GK] ? kv[j] : 0ull;
        kh[j] = (uint32_t)(key >> 32);
        kl[j] = (uint32_t)key;
        asm volatile("" : "+v"(kh[j]), "+v"(kl[j]));  // as in the segment kernel
    }
    auto key = [&](int j) { return ((uint64_t)kh[j] << 32) | (uint64_t)kl[j]; };
    const uint64_t T = tf_kth_key<TK_MV>(key, k, sh.rk);
    // the k keys >= T, compacted and sorted
    const int lane = tid & 63, w = tid >> 6;
    uint32_t m = 0u;
#pragma unroll
    for (int j = 0; j < TK_MV; ++j) m |= key(j) >= T && key(j) != 0ull ? (1u << j) : 0u;
    const int c = __popc(m);
    int incl = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(incl, o);
        if (lane >= o) incl += t;
    }
    if (lane == 63) sh.rk.wsum[w] = incl;
    __syncthreads();
    int base = incl - c;
#pragma unroll
    for (int q = 0; q < TK_NT / kWave; ++q) base += q < w ? sh.rk.wsum[q] : 0;
#pragma unroll
    for (int j = 0; j < TK_MV; ++j)
        if ((m >> j) & 1u) sh.rk.sel[base++] = key(j);
    __syncthreads();
    block_sort_into(sh.rk.sel, k, sh.rk.sorted);
    __syncthreads();
    for (int i = tid; i < K; i += TK_NT) {
        if (i < k) {
            const uint64_t x = sh.rk.sorted[i];
            oidx[i] = (int32_t)key_id(x);
            osc[i] = key_score(x);
        } else {
            oidx[i] = -1;
            osc[i] = -INFINITY;
        }
    }
}

// ---------------------------------------------------------------------------
// Streaming (VALU) path: few users, fp32 inputs, per-user candidate lists
// ---------------------------------------------------------------------------
constexpr int ST_NT = 256;
constexpr int ST_U = 8;  // rows in flight per wave

template <typename T>
struct Vec16;
template <>
struct Vec16<uint16_t> {
    static constexpr int N = 8;
    static __device__ __forceinline__ float dot(uint4 e, uint4 h, float acc) {
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, e.x), __builtin_bit_cast(bf16x2_t, h.x), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, e.y), __builtin_bit_cast(bf16x2_t, h.y), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, e.z), __builtin_bit_cast(bf16x2_t, h.z), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, e.w), __builtin_bit_cast(bf16x2_t, h.w), acc, false);
        return acc;
    }
};
template <>
struct Vec16<float> {
    static constexpr int N = 4;
    static __device__ __forceinline__ float dot(uint4 e, uint4 h, float acc) {
        acc = fmaf(__uint_as_float(e.x), __uint_as_float(h.x), acc);
        acc = fmaf(__uint_as_float(e.y), __uint_as_float(h.y), acc);
        acc = fmaf(__uint_as_float(e.z), __uint_as_float(h.z), acc);
        acc = fmaf(__uint_as_float(e.w), __uint_as_float(h.w), acc);
        return acc;
    }
};

// Sum eight per-lane partials over the wave so that lanes 8g..8g+7 end with
// the total of partial g (a butterfly reduce-scatter: 10 shuffles, not 48).
__device__ __forceinline__ float reduce_scatter8(float (&v)[ST_U], int lane) {
    const bool b5 = lane & 32, b4 = lane & 16, b3 = lane & 8;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float send = b5 ? v[i] : v[i + 4];
        const float keep = b5 ? v[i + 4] : v[i];
        v[i] = keep + __shfl_xor(send, 32);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const float send = b4 ? v[i] : v[i + 2];
        const float keep = b4 ? v[i + 2] : v[i];
        v[i] = keep + __shfl_xor(send, 16);
    }
    {
        const float send = b3 ? v[0] : v[1];
        const float keep = b3 ? v[1] : v[0];
        v[0] = keep + __shfl_xor(send, 8);
    }
    float s = v[0];
    s += __shfl_xor(s, 4);
    s += __shfl_xor(s, 2);
    s += __shfl_xor(s, 1);
    return s;
}

static_assert(ST_NT == CAND_PIECE, "one thread per list entry of a piece");
static_assert(ST_NT == TK_NT, "the fused finish is the register-resident selection of one block");
static_assert(ST_NT * 32 == kFusedMaxM, "the fused path's largest catalog: 32 keys per thread of the finishing block");

// ---------------------------------------------------------------------------
// Fused small-catalog path: one launch for the whole call
// ---------------------------------------------------------------------------
// Each block of the streaming pass writes its rows' scores into the user's
// dense score row and its (max, sum-exp) piece; the block that arrives last
// for a user finishes that user: lse from the pieces, and the top-K of the
// row by the register-resident radix selection (FV keys per thread, so rows
// of up to ST_NT * FV scores).
//
// Finding the last block without fences or a contended counter.  Every
// value one block hands to another (score rows, pieces, flags) is written
// with agent-scope stores (sc1: written through to the device's point of
// coherence) and read with agent-scope loads, so no L2 writeback or
// invalidation (a whole-cache operation per wave) is needed.  A block first
// waits until its own stores have completed, then sets its flag to the call's
// ticket (40 bits, unique to the call, never 0 or all ones, from the host),
// waits again, and reads all of its user's flags: whichever block sees every
// flag holding the ticket may finish the user.  Since each block's flag is
// complete before it reads the others, the last block to set its flag sees
// them all.  Several blocks can see them all; an exchange on the user's
// election word picks one (the first to find a value other than the ticket
// there), and it clears the flags and the word when done, so that a replay of
// the same captured call (same ticket) starts clean.  Stale workspace
// contents are recognised by their ticket: only a word that happens to hold
// this call's ticket could be misread.
template <class V>
__device__ __forceinline__ void put_agent(V* p, V v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <class V>
__device__ __forceinline__ V get_agent(const V* p) {
    return __hip_atomic_load((V*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// every vector memory operation of this wave completed (stores acknowledged)
__device__ __forceinline__ void wait_stores() { __builtin_amdgcn_s_waitcnt(0); }

// Block-uniform: true for the block that finishes the user whose flags are
// flags[0 .. P); `mine` is this block's flag.
__device__ bool arrive_elect(uint64_t* flags, uint64_t* mine, uint64_t* elect, uint64_t ticket, int P, int* s_red) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    wait_stores();
    __syncthreads();  // every wave's stores of this block have completed
    if (tid == 0) {
        put_agent(mine, ticket);
        wait_stores();
    }
    __syncthreads();
    int c = 0;
    for (int q = tid; q < P; q += blockDim.x) c += get_agent(flags + q) == ticket ? 1 : 0;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) c += __shfl_xor(c, o);
    if (lane == 0) s_red[w] = c;
    __syncthreads();
    int all = 0;
    for (int q = 0; q < (int)(blockDim.x >> 6); ++q) all += s_red[q];
    __syncthreads();
    if (all < P) return false;
    if (tid == 0) {
        const uint64_t prev = __hip_atomic_exchange(elect, ticket, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_red[0] = prev != ticket ? 1 : 0;
    }
    __syncthreads();
    return s_red[0] != 0;
}

// Order key of a dense-row score; masked items (-inf) are no key (0, below
// every score's key: order_key is never 0 for a non-NaN value).
__device__ __forceinline__ uint32_t row_key(float s) { return s == -INFINITY ? 0u : order_key(s); }

// The finishing block of a user.  One round of loads brings the user's
// pieces (the blocks' (max, sum-exp), at most one per thread: P <= 256) and
// its dense score row (FV keys per thread, kept in LDS as order keys too).
// lse merges the pieces.  For the top-K (K <= 256) the threshold T is the
// K-th largest of the P block maxima: each thread ranks its block's maximum
// against all P (LDS broadcast reads, four keys at a time) and T is the
// smallest maximum of rank < K.  At least K blocks hold a key >= T, so at
// least K keys reach T and all of the top K do.  Those keys -- about K + K/2
// when the rows are exchangeable -- are compacted as 64-bit ranking keys
// (score word, inverted column: distinct) and each is placed at its rank.
// More than kFastCap keys at T (many equal scores) or K > 256: the
// register-resident radix selection instead, exact in every case.  This code
// runs once per user on one block, so every step is spread over the block's
// threads: a serial chain (one wave deciding bits one at a time, one thread
// per candidate walking a long loop) costs microseconds here.
constexpr int kFastCap = GENREC_KMAX;
constexpr int kFusedKeys = ST_NT * 32;  // keys per user at most (32 per thread)

struct FastShared {
    uint32_t keys[kFusedKeys];  // the row's order keys, slot j of thread t at j * ST_NT + t (0: none)
    uint32_t bmax[ST_NT];       // order keys of the block maxima (0: none)
    uint32_t tred[ST_NT / kWave];
    int wcnt[ST_NT / kWave];
    float2 ml[ST_NT / kWave];
};

// Radix selection over the keys staged in LDS (FV per thread), then the
// ranked output.
template <int FV>
__device__ __noinline__ void fused_topk_radix(const uint32_t* lkeys, int K, TkShared& sh, int32_t* oidx,
                                              float* osc) {
    const int tid = threadIdx.x;
    uint32_t hv[FV];
#pragma unroll
    for (int j = 0; j < FV; ++j) hv[j] = lkeys[j * ST_NT + tid];
#pragma unroll
    for (int j = 0; j < FV; ++j) asm volatile("" : "+v"(hv[j]));
    int cv = 0;
#pragma unroll
    for (int j = 0; j < FV; ++j) cv += __popcll(__ballot(hv[j] != 0u));
    // slot 1 of the count pair: the selection's first count writes slot 0
    // while a slow wave may still be reading this one
    int par = 1;
    const int n_valid = tk_block_sum(cv, par, sh);
    const int k = min(K, n_valid);
    const uint32_t lo0 = 0xFFFFFFFFu - (uint32_t)tid;  // index word of slot 0
    if (k > 0)
        tk_select<FV>([&](int j) { return hv[j]; }, [&](int j) { return lo0 - (uint32_t)(j * ST_NT); },
                      [&](int j) { return hv[j] != 0u; }, n_valid, k, sh);
    tk_emit(k, K, sh, oidx, osc);
}

template <int FV>
__device__ void fused_finish(const StreamArgs& a, int b, TkShared& sh, FastShared& fs) {
    static_assert(FV <= 32, "a 32-bit pass mask per thread");
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int n = (int)a.n_items, P = a.P, K = a.K;
    const float* row = a.rows + (int64_t)b * a.n_items;
    // every load issued before any is waited for: indices are clamped into
    // range instead of branching around the loads
    const int pq = min(tid, P - 1);
    const float pmv = get_agent(a.pm + (int64_t)b * P + pq), plv = get_agent(a.pl + (int64_t)b * P + pq);
    float rv[FV];
#pragma unroll
    for (int j = 0; j < FV; ++j) rv[j] = get_agent(row + min(j * ST_NT + tid, n - 1));
    uint32_t hv[FV];
#pragma unroll
    for (int j = 0; j < FV; ++j) {
        hv[j] = j * ST_NT + tid < n ? row_key(rv[j]) : 0u;
        fs.keys[j * ST_NT + tid] = hv[j];
    }
    const bool has_piece = tid < P;
    // lse over the pieces; the pieces' maxima for the threshold
    LseState st;
    st.init();
    if (has_piece) st.merge(pmv, plv);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) st.merge(__shfl_xor(st.m, o), __shfl_xor(st.l, o));
    if (lane == 0) fs.ml[w] = make_float2(st.m, st.l);
    const uint32_t mykey = has_piece ? row_key(pmv) : 0u;
    fs.bmax[tid] = mykey;
    __syncthreads();
    if (tid == 0) {
        LseState t;
        t.init();
        for (int q = 0; q < ST_NT / kWave; ++q) t.merge(fs.ml[q].x, fs.ml[q].y);
        a.out_lse[b] = t.l > 0.f ? t.m + __builtin_amdgcn_logf(t.l) * kLn2 : -INFINITY;
    }
    int32_t* oidx = a.out_idx + (int64_t)b * K;
    float* osc = a.out_scores + (int64_t)b * K;
    if (K > ST_NT) {  // block-uniform
        fused_topk_radix<FV>(fs.keys, K, sh, oidx, osc);
        return;
    }
    // T: the smallest block maximum whose rank (maxima strictly larger) is
    // below K; with fewer than K blocks holding a key, a zero maximum
    // qualifies and T = 0 admits every key (fewer than K blocks: T = 0 too)
    uint32_t tcand = 0xFFFFFFFFu;
    if (has_piece) {
        int r = 0;
        const uint4* bm4 = (const uint4*)fs.bmax;
#pragma unroll 4
        for (int q = 0; q < (P + 3) / 4; ++q) {  // entries past P hold 0: never larger
            const uint4 v = bm4[q];
            r += (v.x > mykey) + (v.y > mykey) + (v.z > mykey) + (v.w > mykey);
        }
        if (r < K) tcand = mykey;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) tcand = min(tcand, (uint32_t)__shfl_xor((int)tcand, o));
    // keys at T: a pass mask per thread (slot j = bit j), counted and scanned
    uint32_t T;
    {
        if (lane == 0) fs.tred[w] = tcand;
        __syncthreads();
        T = fs.tred[0];
#pragma unroll
        for (int q = 1; q < ST_NT / kWave; ++q) T = min(T, fs.tred[q]);
        if (P < K) T = 0u;
    }
    uint32_t mask = 0;
#pragma unroll
    for (int j = 0; j < FV; ++j) mask |= (hv[j] != 0u && hv[j] >= T) ? (1u << j) : 0u;
    const int c = __popc(mask);
    int incl = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(incl, o);
        if (lane >= o) incl += t;
    }
    if (lane == 63) fs.wcnt[w] = incl;
    __syncthreads();
    int base = incl - c, total = 0;
#pragma unroll
    for (int q = 0; q < ST_NT / kWave; ++q) {
        base += q < w ? fs.wcnt[q] : 0;
        total += fs.wcnt[q];
    }
    if (total > kFastCap) {  // block-uniform
        fused_topk_radix<FV>(fs.keys, K, sh, oidx, osc);
        return;
    }
    uint64_t* cand = sh.sel;
    for (uint32_t m = mask; m != 0u; m &= m - 1u) {
        const int j = __ffs(m) - 1;
        cand[base++] = ((uint64_t)fs.keys[j * ST_NT + tid] << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)(j * ST_NT + tid));
    }
    __syncthreads();
    // total >= K unless fewer than K keys exist (T = 0: all of them)
    const int k = min(K, total);
    if (total <= ST_NT) {
        // rank of each candidate = the number of larger keys (all distinct)
        if (tid < total) {
            const uint64_t x = cand[tid];
            int r = 0;
            const ulonglong2* c2 = (const ulonglong2*)cand;
#pragma unroll 4
            for (int j = 0; j < total / 2; ++j) {
                const ulonglong2 y = c2[j];
                r += (y.x > x) + (y.y > x);
            }
            if (total & 1) r += cand[total - 1] > x ? 1 : 0;
            if (r < k) sh.sorted[r] = x;
        }
    } else {
        block_sort_into(cand, total, sh.sorted);
    }
    __syncthreads();
    for (int i = tid; i < K; i += ST_NT) {
        if (i < k) {
            const uint64_t key = sh.sorted[i];
            oidx[i] = (int32_t)key_id(key);
            osc[i] = key_score(key);
        } else {
            oidx[i] = -1;
            osc[i] = -INFINITY;
        }
    }
}

template <bool FUSED>
struct FusedShared {};
template <>
struct FusedShared<true> {
    TkShared tk;
    FastShared fast;
    int red[ST_NT / kWave];
};

template <typename T, int MODE, int FV = 0>
__global__ __launch_bounds__(ST_NT) void stream_score_kernel(StreamArgs a) {
    __shared__ int s_cnt;
    __shared__ float2 s_ml[ST_NT / kWave];
    __shared__ int s_cold[MODE == 2 ? CAND_PIECE : 1];  // list mode: ids still to gather
    __shared__ int s_wc[ST_NT / kWave];
    __shared__ FusedShared<MODE == 3> fsh;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    constexpr int VEC = Vec16<T>::N;

    int b;
    int64_t n, region, piece, jbeg = 0, e0 = 0;
    if (MODE == 2) {
        piece = blockIdx.x;
        if (piece >= *a.n_pieces) return;
        const CandPiece rec = a.table[piece];
        b = rec.user;
        n = rec.len;
        e0 = rec.e0;
        region = e0;
    } else {
        const int cidx = blockIdx.x / a.B;
        b = blockIdx.x - cidx * a.B;
        jbeg = (int64_t)cidx * a.CH;
        n = min((int64_t)a.CH, a.n_items - jbeg);
        piece = (int64_t)b * a.P + cidx;
        region = (int64_t)b * a.M + jbeg;
    }
    if (tid == 0) s_cnt = 0;
    __syncthreads();

    const T* E = (const T*)a.E;
    const T* h = (const T*)a.H + (int64_t)b * a.D;
    float th = -FLT_MAX;
    if (MODE != 0 && a.theta != nullptr) th = fmaxf(a.theta[b], -FLT_MAX);
    LseState st;
    st.init();

    if (MODE == 2) {
        // One thread per entry: ids outside [0, M) are counted and skipped; a
        // hot id's score is looked up in the dense hot scores; the remaining
        // ids go, in list order, to a block-wide list that the gather loop
        // below works through.
        const int e = tid;
        int id = 0;
        bool valid = false;
        if (e < n) {
            id = a.ids[e0 + e];
            valid = id >= 0 && (int64_t)id < a.M;
        }
        const uint64_t badmask = __ballot(e < n && !valid);
        if (lane == 0 && badmask) atomicAdd((unsigned long long*)a.err, (unsigned long long)__popcll(badmask));
        bool cold = valid;
        if (valid && a.hot_idx != nullptr) {
            const int hi = a.hot_idx[id];
            if (hi >= 0) {
                cold = false;
                const float s = a.s_hot[(int64_t)b * a.t_hot + hi];
                st.add(s);
                if (s >= th) {
                    const int pos = atomicAdd(&s_cnt, 1);
                    a.keys[region + pos] = rank_key(s, (uint32_t)id);
                }
            }
        }
        const uint64_t cm = __ballot(cold);
        if (lane == 0) s_wc[w] = __popcll(cm);
        __syncthreads();
        int base = 0, tot = 0;
#pragma unroll
        for (int q = 0; q < ST_NT / kWave; ++q) {
            base += q < w ? s_wc[q] : 0;
            tot += s_wc[q];
        }
        if (cold) s_cold[base + __popcll(cm & ((1ull << lane) - 1ull))] = id;
        n = tot;
        __syncthreads();
    }

    for (int64_t g0 = (int64_t)w * ST_U; g0 < n; g0 += (ST_NT / kWave) * ST_U) {
        int64_t item[ST_U];
        bool ok[ST_U];
        if (MODE == 2) {
#pragma unroll
            for (int u = 0; u < ST_U; ++u) {
                ok[u] = g0 + u < n;
                item[u] = ok[u] ? s_cold[g0 + u] : 0;
            }
        } else {
#pragma unroll
            for (int u = 0; u < ST_U; ++u) {
                ok[u] = g0 + u < n;
                const int64_t j = jbeg + g0 + u;  // pass index -> catalog row (one tile per sample window)
                item[u] = mf_sample_tile(j >> 8, a.tile_stride, a.M >> 8) * 256 + (j & 255);
            }
        }
        float acc[ST_U];
#pragma unroll
        for (int u = 0; u < ST_U; ++u) acc[u] = 0.f;
#pragma unroll 2
        for (int d = lane * VEC; d < a.D; d += kWave * VEC) {
            const uint4 hv = *(const uint4*)(h + d);
            uint4 ev[ST_U];
#pragma unroll
            for (int u = 0; u < ST_U; ++u)
                ev[u] = ok[u] ? *(const uint4*)(E + item[u] * a.D + d) : make_uint4(0, 0, 0, 0);
#pragma unroll
            for (int u = 0; u < ST_U; ++u) acc[u] = Vec16<T>::dot(ev[u], hv, acc[u]);
        }
        const float s = reduce_scatter8(acc, lane);
        const int u = lane >> 3;
        bool mine = (lane & 7) == 0;
#pragma unroll
        for (int q = 0; q < ST_U; ++q)
            if (q == u) mine = mine && ok[q];
        if (mine) {
            int64_t it = 0;
#pragma unroll
            for (int q = 0; q < ST_U; ++q)
                if (q == u) it = item[q];
            float sv = s;
            if (MODE != 2 && a.mask != nullptr && !((a.mask[(int64_t)b * a.mask_stride + (it >> 5)] >> (it & 31)) & 1u))
                sv = -INFINITY;  // masked item: nothing to the sum, never a candidate
            if (MODE == 0) {
                a.sample_out[(int64_t)b * a.n_items + jbeg + g0 + u] = sv;
            } else if (MODE == 3) {
                put_agent(a.rows + (int64_t)b * a.n_items + jbeg + g0 + u, sv);
                if (sv != -INFINITY) st.add(sv);
            } else if (sv != -INFINITY) {
                const float s = sv;
                st.add(s);
                if (s >= th) {
                    const int pos = atomicAdd(&s_cnt, 1);
                    a.keys[region + pos] = rank_key(s, (uint32_t)it);
                }
            }
        }
    }
    if (MODE == 0) return;

    // (max, sum-exp) over the wave, then over the four waves.
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const float m2 = __shfl_xor(st.m, o), l2 = __shfl_xor(st.l, o);
        st.merge(m2, l2);
    }
    if (lane == 0) s_ml[w] = make_float2(st.m, st.l);
    __syncthreads();
    if (tid == 0) {
        LseState t;
        t.init();
        for (int q = 0; q < ST_NT / kWave; ++q) t.merge(s_ml[q].x, s_ml[q].y);
        if (MODE == 3) {
            put_agent(a.pm + piece, t.m);
            put_agent(a.pl + piece, t.l);
        } else {
            a.pm[piece] = t.m;
            a.pl[piece] = t.l;
            a.pcnt[piece] = s_cnt;
            a.preg[piece] = region;
        }
    }
    if constexpr (MODE == 3) {
        if (tid == 0 && blockIdx.x == 0) {  // the call's header: no candidate errors, no rescued users
            a.err[0] = 0;
            a.err[1] = 0;
            a.err[3] = 0;
        }
        uint64_t* flags = a.arrive + (int64_t)b * a.P;  // user b's blocks, by chunk
        if (!arrive_elect(flags, flags + piece - (int64_t)b * a.P, a.elect + b, a.ticket, a.P, fsh.red)) return;
        fused_finish<FV>(a, b, fsh.tk, fsh.fast);
        // clean for the next call: flags and election word back to zero
        for (int q = tid; q < a.P; q += ST_NT) put_agent(flags + q, (uint64_t)0);
        if (tid == 0) put_agent(a.elect + b, (uint64_t)0);
    }
}

// ---------------------------------------------------------------------------
// Candidate lists: CSR offsets -> pieces of at most CAND_PIECE entries
// ---------------------------------------------------------------------------
constexpr int PL_NT = 1024;

__global__ __launch_bounds__(PL_NT) void cand_plan_kernel(CandPlanArgs a) {
    __shared__ int64_t s_wmax[PL_NT / kWave];
    __shared__ int s_wsum[PL_NT / kWave];
    __shared__ int64_t s_carry_end;
    __shared__ int s_carry_pieces;
    __shared__ int s_bad;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    if (tid == 0) {
        s_carry_end = 0;
        s_carry_pieces = 0;
        s_bad = 0;
        a.err[0] = 0;
        a.err[1] = 0;
    }
    __syncthreads();
    for (int base = 0; base < a.B; base += PL_NT) {
        const int b = base + tid;
        int64_t o0 = 0, o1 = 0;
        if (b < a.B) {
            o0 = a.offsets[b];
            o1 = a.offsets[b + 1];
        }
        // prefix max of earlier list ends: a list must start at or after it
        int64_t endv = b < a.B ? o1 : 0;
        int64_t incl = endv;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int64_t t = __shfl_up(incl, o);
            if (lane >= o) incl = t > incl ? t : incl;
        }
        if (lane == 63) s_wmax[w] = incl;
        __syncthreads();
        int64_t prev = s_carry_end;
        for (int q = 0; q < w; ++q) prev = s_wmax[q] > prev ? s_wmax[q] : prev;
        int64_t excl = __shfl_up(incl, 1);
        if (lane > 0) prev = excl > prev ? excl : prev;
        const bool valid = b < a.B && o0 >= prev && o0 >= 0 && o1 >= o0 && o1 <= a.nnz;
        if (b < a.B && !valid) atomicAdd(&s_bad, 1);
        const int64_t len = valid ? o1 - o0 : 0;
        const int np = (int)((len + CAND_PIECE - 1) / CAND_PIECE);
        // exclusive scan of piece counts
        int pinc = np;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int t = __shfl_up(pinc, o);
            if (lane >= o) pinc += t;
        }
        if (lane == 63) s_wsum[w] = pinc;
        __syncthreads();
        int pofs = s_carry_pieces;
        for (int q = 0; q < w; ++q) pofs += s_wsum[q];
        const int first = pofs + pinc - np;
        if (b < a.B) {
            a.piece_begin[b] = first;
            for (int j = 0; j < np; ++j) {
                CandPiece rec;
                rec.user = b;
                rec.len = (int)min((int64_t)CAND_PIECE, len - (int64_t)j * CAND_PIECE);
                rec.e0 = o0 + (int64_t)j * CAND_PIECE;
                a.table[first + j] = rec;
            }
        }
        __syncthreads();  // every read of the carries and wave partials is done
        if (tid == PL_NT - 1) s_carry_pieces = first + np;
        if (tid == 0) {
            int64_t m = s_carry_end;
            for (int q = 0; q < PL_NT / kWave; ++q) m = s_wmax[q] > m ? s_wmax[q] : m;
            s_carry_end = m;
        }
        __syncthreads();
    }
    if (tid == 0) {
        a.piece_begin[a.B] = s_carry_pieces;
        *a.n_pieces = s_carry_pieces;
        a.err[1] = s_bad;
    }
}

// ---------------------------------------------------------------------------
// Candidate lists, hot head: which catalog rows to score densely
// ---------------------------------------------------------------------------
constexpr int HOT_NT = 256;
constexpr int HOT_PER = kHotBlock / HOT_NT;  // ids per thread in the compaction

__global__ __launch_bounds__(HOT_NT) void hot_clear_kernel(HotArgs a) {
    const int64_t stride = (int64_t)gridDim.x * HOT_NT;
    for (int64_t i = (int64_t)blockIdx.x * HOT_NT + threadIdx.x; i < a.M; i += stride) a.cnt[i] = 0;
    if (blockIdx.x == 0) {
        for (int i = threadIdx.x; i < kHotBins; i += HOT_NT) a.hist[i] = 0;
        if (threadIdx.x < 4) a.meta[threadIdx.x] = 0;
    }
}

// How many list entries name each catalog id, estimated from every
// kHotSample-th entry of the id array (all lists, in range ids): the hot set
// only steers where scores are computed, never what they are, so an estimate
// does; sampling cuts the device-wide atomics on popular ids 16-fold.
__global__ __launch_bounds__(HOT_NT) void hot_count_kernel(HotArgs a) {
    const int64_t n_samples = (a.nnz + kHotSample - 1) / kHotSample;
    const int64_t stride = (int64_t)gridDim.x * HOT_NT;
    for (int64_t t = (int64_t)blockIdx.x * HOT_NT + threadIdx.x; t < n_samples; t += stride) {
        const int id = a.ids[t * kHotSample];
        if (id >= 0 && (int64_t)id < a.M) atomicAdd(&a.cnt[id], 1);
    }
}

// Histogram of the non-zero counts (bin = min(count, 4095)).
__global__ __launch_bounds__(HOT_NT) void hot_hist_kernel(HotArgs a) {
    __shared__ int h[kHotBins];
    for (int i = threadIdx.x; i < kHotBins; i += HOT_NT) h[i] = 0;
    __syncthreads();
    const int64_t stride = (int64_t)gridDim.x * HOT_NT;
    for (int64_t i = (int64_t)blockIdx.x * HOT_NT + threadIdx.x; i < a.M; i += stride) {
        const int c = a.cnt[i];
        if (c > 0) atomicAdd(&h[min(c, kHotBins - 1)], 1);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < kHotBins; i += HOT_NT)
        if (h[i]) atomicAdd(&a.hist[i], h[i]);
}

// One block: the threshold c = the smallest count >= c_min whose suffix
// (items with at least c entries) holds at most t_max items; none such: no
// hot rows.  meta[0] = c, meta[1] = the number of hot rows.
constexpr int HOT_PICK_NT = 1024;
__global__ __launch_bounds__(HOT_PICK_NT) void hot_pick_kernel(HotArgs a) {
    __shared__ int s_w[HOT_PICK_NT / kWave];
    constexpr int PER = kHotBins / HOT_PICK_NT;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    // thread t owns bins kHotBins-1-(PER t .. PER t + PER - 1): highest first
    int v[PER], tsum = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        v[i] = a.hist[kHotBins - 1 - (tid * PER + i)];
        tsum += v[i];
    }
    int incl = tsum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(incl, o);
        if (lane >= o) incl += t;
    }
    if (lane == 63) s_w[w] = incl;
    __syncthreads();
    int run = incl - tsum;
    for (int q = 0; q < w; ++q) run += s_w[q];
    if (tid == 0) a.meta[0] = 0x7FFFFFFF;  // no hot rows unless a bin qualifies below
    __syncthreads();
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int bin = kHotBins - 1 - (tid * PER + i);
        run += v[i];  // now the suffix count of `bin`
        // bins are visited from the top, so suffix(bin) only grows; the
        // threshold is the lowest qualifying bin
        const int below = bin - 1;  // suffix(below) = run + hist[below]
        if (bin >= a.c_min && run <= a.t_max) {
            const bool lowest = bin == a.c_min || run + a.hist[below] > a.t_max;
            if (lowest) {
                a.meta[0] = bin;
                a.meta[1] = run;
            }
        }
    }
}

// Bit i: catalog id id0 + i is hot (count >= c; clear past the catalog).
// The HOT_PER counts are fetched before any is tested -- four 16-byte loads
// where the ids are all in range, else clamped ones -- rather than one
// guarded load after another.
static_assert(HOT_PER == 16, "four 16-byte loads of counts per thread");
__device__ __forceinline__ uint32_t hot_mask(const HotArgs& a, int64_t id0, int c) {
    int v[HOT_PER];
    if (id0 + HOT_PER <= a.M) {  // id0 is a multiple of HOT_PER: 64-byte aligned
        const int4* p = (const int4*)(a.cnt + id0);
#pragma unroll
        for (int q = 0; q < HOT_PER / 4; ++q) {
            const int4 x = p[q];
            v[4 * q] = x.x;
            v[4 * q + 1] = x.y;
            v[4 * q + 2] = x.z;
            v[4 * q + 3] = x.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < HOT_PER; ++i) v[i] = a.cnt[min(id0 + i, a.M - 1)];
    }
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < HOT_PER; ++i) m |= (id0 + i < a.M && v[i] >= c) ? 1u << i : 0u;
    return m;
}

// Hot ids per block of kHotBlock catalog ids.
__global__ __launch_bounds__(HOT_NT) void hot_blockcount_kernel(HotArgs a) {
    __shared__ int s_w[HOT_NT / kWave];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int c = a.meta[0];
    const int64_t id0 = (int64_t)blockIdx.x * kHotBlock + (int64_t)tid * HOT_PER;
    int n = __popc(hot_mask(a, id0, c));
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) n += __shfl_xor(n, o);
    if (lane == 0) s_w[w] = n;
    __syncthreads();
    if (tid == 0) {
        int t = 0;
        for (int q = 0; q < HOT_NT / kWave; ++q) t += s_w[q];
        a.hblk[blockIdx.x] = t;
    }
}

// One block: exclusive scan of the per-block counts, in place.
__global__ __launch_bounds__(HOT_PICK_NT) void hot_scan_kernel(HotArgs a) {
    __shared__ int s_w[HOT_PICK_NT / kWave];
    __shared__ int s_carry;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    if (tid == 0) s_carry = 0;
    __syncthreads();
    for (int64_t base = 0; base < a.n_hblk; base += HOT_PICK_NT) {
        const int64_t i = base + tid;
        const int v = i < a.n_hblk ? a.hblk[i] : 0;
        int incl = v;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int t = __shfl_up(incl, o);
            if (lane >= o) incl += t;
        }
        if (lane == 63) s_w[w] = incl;
        __syncthreads();
        int pre = s_carry;
        for (int q = 0; q < w; ++q) pre += s_w[q];
        if (i < a.n_hblk) a.hblk[i] = pre + incl - v;
        __syncthreads();
        if (tid == HOT_PICK_NT - 1) s_carry = pre + incl;
        __syncthreads();
    }
}

// Hot index of every catalog id (-1: not hot) and the hot ids in id order.
__global__ __launch_bounds__(HOT_NT) void hot_assign_kernel(HotArgs a) {
    __shared__ int s_w[HOT_NT / kWave];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int c = a.meta[0];
    const int64_t id0 = (int64_t)blockIdx.x * kHotBlock + (int64_t)tid * HOT_PER;
    const uint32_t hm = hot_mask(a, id0, c);
    const int n = __popc(hm);
    int incl = n;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(incl, o);
        if (lane >= o) incl += t;
    }
    if (lane == 63) s_w[w] = incl;
    __syncthreads();
    int pos = a.hblk[blockIdx.x] + incl - n;
    for (int q = 0; q < w; ++q) pos += s_w[q];
#pragma unroll
    for (int i = 0; i < HOT_PER; ++i) {
        const int64_t id = id0 + i;
        if (id < a.M) {
            const bool hotv = (hm >> i) & 1u;
            a.hot_idx[id] = hotv ? pos : -1;
            if (hotv) a.hot_ids[pos++] = (int)id;
        }
    }
}

// The hot catalog rows, gathered in hot-index order (rows past the hot count
// are left as they are: their dense scores are never looked up).
__global__ __launch_bounds__(HOT_NT) void hot_gather_kernel(HotArgs a) {
    const int r = blockIdx.x;
    if (r >= a.meta[1]) return;
    const uint4* src = (const uint4*)(a.E + (int64_t)a.hot_ids[r] * a.D);
    uint4* dst = (uint4*)(a.e_hot + (int64_t)r * a.D);
    for (int i = threadIdx.x; i < a.D / 8; i += HOT_NT) dst[i] = src[i];
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
// ---------------------------------------------------------------------------
// Cross-entropy over the catalog: bookkeeping kernels around the MFMA passes
// ---------------------------------------------------------------------------
constexpr int CE_NT = 256;

// Effective weight per example: the caller's weight (1 when none), 0 for a
// label outside [0, M); err[0] = the number of such labels, err[1] = 0.
// One block.
__global__ __launch_bounds__(1024) void ce_prep_kernel(CeArgs a) {
    __shared__ int s_bad;
    if (threadIdx.x == 0) s_bad = 0;
    __syncthreads();
    int bad = 0;
    for (int b = threadIdx.x; b < a.B; b += blockDim.x) {
        const int32_t y = a.labels[b];
        const bool ok = y >= 0 && (int64_t)y < a.M;
        a.w_eff[b] = ok ? (a.weights != nullptr ? a.weights[b] : 1.f) : 0.f;
        bad += ok ? 0 : 1;
    }
    if (bad) atomicAdd(&s_bad, bad);
    __syncthreads();
    if (threadIdx.x == 0) {
        a.err[0] = s_bad;
        a.err[1] = 0;
    }
}

// Per example b: lse_b from the logsumexp pieces of the MFMA pass, the
// label's score s_y = h_b . e_y (fp32 sum of exact bf16 products) and
// loss_b = w_b (lse_b - s_y); an example whose label is out of range has
// weight 0 and loss 0.
__global__ __launch_bounds__(CE_NT) void ce_finish_kernel(CeArgs a) {
    __shared__ float s_m[CE_NT / kWave], s_l[CE_NT / kWave], s_d[CE_NT / kWave];
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    LseState st;
    st.init();
    for (int p = tid; p < a.P; p += CE_NT) st.merge(a.pm[(int64_t)b * a.P + p], a.pl[(int64_t)b * a.P + p]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) st.merge(__shfl_xor(st.m, o), __shfl_xor(st.l, o));
    const int32_t y = a.labels[b];
    const bool ok = y >= 0 && (int64_t)y < a.M;
    float dot = 0.f;
    if (ok) {
        const uint16_t* h = a.H + (int64_t)b * a.D;
        const uint16_t* e = a.E + (int64_t)y * a.D;
        for (int d = tid * 8; d < a.D; d += CE_NT * 8) {
            const uint4 hv = *(const uint4*)(h + d), ev = *(const uint4*)(e + d);
            dot = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, hv.x), __builtin_bit_cast(bf16x2_t, ev.x), dot, false);
            dot = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, hv.y), __builtin_bit_cast(bf16x2_t, ev.y), dot, false);
            dot = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, hv.z), __builtin_bit_cast(bf16x2_t, ev.z), dot, false);
            dot = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, hv.w), __builtin_bit_cast(bf16x2_t, ev.w), dot, false);
        }
    }
    dot = wave_sum(dot);
    if (lane == 0) { s_m[w] = st.m; s_l[w] = st.l; s_d[w] = dot; }
    __syncthreads();
    if (tid == 0) {
        LseState t;
        t.init();
        float sy = 0.f;
        for (int q = 0; q < CE_NT / kWave; ++q) { t.merge(s_m[q], s_l[q]); sy += s_d[q]; }
        const float lse = t.l > 0.f ? t.m + __builtin_amdgcn_logf(t.l) * kLn2 : -INFINITY;
        a.out_lse[b] = lse;
        a.out_loss[b] = ok ? a.w_eff[b] * (lse - sy) : 0.f;
    }
}

// out[c][r] = in[r][c] through a 64 x 64 LDS tile; rows r in [R, ld_out) of
// the output are zero.
constexpr int TR_T = 64;
__global__ __launch_bounds__(256) void transpose_kernel(TransposeArgs a) {
    __shared__ uint16_t tile[TR_T][TR_T + 2];
    const int64_t c0 = (int64_t)blockIdx.x * TR_T, r0 = (int64_t)blockIdx.y * TR_T;
    const int tid = threadIdx.x;
    for (int i = tid; i < TR_T * (TR_T / 8); i += 256) {
        const int rr = i >> 3, cc = (i & 7) * 8;
        const int64_t r = r0 + rr, cb = c0 + cc;
        uint16_t v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        if (r < a.R) {
            const uint16_t* src = a.in + r * a.ld_in + cb;
            if (cb + 7 < a.C) {
                const uint4 q = *(const uint4*)src;
                const uint32_t w4[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[2 * e] = (uint16_t)w4[e];
                    v[2 * e + 1] = (uint16_t)(w4[e] >> 16);
                }
            } else {
                for (int e = 0; e < 8; ++e)
                    if (cb + e < a.C) v[e] = src[e];
            }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) tile[rr][cc + e] = v[e];
    }
    __syncthreads();
    for (int i = tid; i < TR_T * (TR_T / 8); i += 256) {
        const int cc = i >> 3, rr = (i & 7) * 8;
        const int64_t c = c0 + cc, r = r0 + rr;
        if (c >= a.C || r >= a.ld_out) continue;
        uint16_t v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = tile[rr + e][cc];
        uint16_t* dst = a.out + (a.blocked ? (r >> 5) * a.C * 32 + c * 32 + (r & 31) : c * a.ld_out + r);
        if (r + 7 < a.ld_out) {
            // streaming store: the transposed chunk is read back two kernels
            // later and does not fit the caches anyway
            typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
            const u32x4_t q4 = {v[0] | ((uint32_t)v[1] << 16), v[2] | ((uint32_t)v[3] << 16),
                                v[4] | ((uint32_t)v[5] << 16), v[6] | ((uint32_t)v[7] << 16)};
            __builtin_nontemporal_store(q4, (u32x4_t*)dst);
        } else {
            for (int e = 0; e < 8; ++e)
                if (r + e < a.ld_out) dst[e] = v[e];
        }
    }
}

__global__ __launch_bounds__(256) void sum_splits_kernel(const float* in, int n, int64_t stride, int64_t count,
                                                         float* out) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < count; i += (int64_t)gridDim.x * 256) {
        float t = 0.f;
        for (int z = 0; z < n; ++z) t += in[z * stride + i];
        out[i] = t;
    }
}

hipError_t launch_ce_prep(const CeArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(ce_prep_kernel, dim3(1), dim3(1024), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_ce_finish(const CeArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(ce_finish_kernel, dim3(a.B), dim3(CE_NT), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_transpose(const TransposeArgs& a, hipStream_t s) {
    const int64_t gx = (a.C + TR_T - 1) / TR_T, gy = (a.ld_out + TR_T - 1) / TR_T;
    if (gx <= 0 || gy <= 0) return hipSuccess;
    if (gy > 65535 || gx > 2147483647) return hipErrorInvalidValue;
    hipLaunchKernelGGL(transpose_kernel, dim3((unsigned)gx, (unsigned)gy), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_sum_splits(const float* in, int n, int64_t stride, int64_t count, float* out, hipStream_t s) {
    if (count <= 0) return hipSuccess;
    const int64_t g = std::min<int64_t>((count + 255) / 256, 4096);
    hipLaunchKernelGGL(sum_splits_kernel, dim3((unsigned)g), dim3(256), 0, s, in, n, stride, count, out);
    return hipGetLastError();
}

hipError_t launch_mfma_split(const MfmaArgs& a, int mode, int splits, hipStream_t s) {
    const dim3 grid(a.UT * a.P, splits);
    const bool ktail = (a.D % MF_BK) != 0;
    if (mode == 3) {
        if (ktail) hipLaunchKernelGGL((mfma_score_kernel<3, true, false>), grid, dim3(MF_NT), 0, s, a);
        else hipLaunchKernelGGL((mfma_score_kernel<3, false, false>), grid, dim3(MF_NT), 0, s, a);
    } else if (mode == 4) {
        if (ktail) return hipErrorInvalidValue;  // the products run over zero-padded reductions
        hipLaunchKernelGGL((mfma_score_kernel<4, false, false>), grid, dim3(MF_NT), 0, s, a);
    } else if (mode == 5) {
        if (ktail || a.k_split % MF_BK != 0) return hipErrorInvalidValue;
        hipLaunchKernelGGL((mfma_score_kernel<5, false, false>), grid, dim3(MF_NT), 0, s, a);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_mfma(const MfmaArgs& a, int mode, hipStream_t s, int splits) {
    if (splits < 1 || (splits > 1 && mode != 0) || (mode != 0 && mode != 1 && mode != 6)) return hipErrorInvalidValue;
    const dim3 grid(a.UT * a.P, splits);
    const bool masked = a.mask != nullptr;
    if (a.f32) {
        // fp32 operands: k-steps of 16 elements
        const bool ktail = (a.D % (MF_BK / 2)) != 0;
#define GENREC_MFMA32(MO, KT, MK) \
    hipLaunchKernelGGL((mfma_score_kernel<MO, KT, MK, true>), grid, dim3(MF_NT), 0, s, a)
        if (mode == 0) {
            if (masked) {
                if (ktail) GENREC_MFMA32(0, true, true); else GENREC_MFMA32(0, false, true);
            } else {
                if (ktail) GENREC_MFMA32(0, true, false); else GENREC_MFMA32(0, false, false);
            }
        } else if (mode == 6) {
            if (masked) {
                if (ktail) GENREC_MFMA32(6, true, true); else GENREC_MFMA32(6, false, true);
            } else {
                if (ktail) GENREC_MFMA32(6, true, false); else GENREC_MFMA32(6, false, false);
            }
        } else {
            if (masked) {
                if (ktail) GENREC_MFMA32(1, true, true); else GENREC_MFMA32(1, false, true);
            } else {
                if (ktail) GENREC_MFMA32(1, true, false); else GENREC_MFMA32(1, false, false);
            }
        }
#undef GENREC_MFMA32
        return hipGetLastError();
    }
    const bool ktail = (a.D % MF_BK) != 0;
#define GENREC_MFMA(MO, KT, MK) hipLaunchKernelGGL((mfma_score_kernel<MO, KT, MK>), grid, dim3(MF_NT), 0, s, a)
    if (mode == 0) {
        if (masked) {
            if (ktail) GENREC_MFMA(0, true, true); else GENREC_MFMA(0, false, true);
        } else {
            if (ktail) GENREC_MFMA(0, true, false); else GENREC_MFMA(0, false, false);
        }
    } else if (mode == 6) {
        if (masked) {
            if (ktail) GENREC_MFMA(6, true, true); else GENREC_MFMA(6, false, true);
        } else {
            if (ktail) GENREC_MFMA(6, true, false); else GENREC_MFMA(6, false, false);
        }
    } else {
        if (masked) {
            if (ktail) GENREC_MFMA(1, true, true); else GENREC_MFMA(1, false, true);
        } else {
            if (ktail) GENREC_MFMA(1, true, false); else GENREC_MFMA(1, false, false);
        }
    }
#undef GENREC_MFMA
    return hipGetLastError();
}

hipError_t launch_fused(const StreamArgs& a, bool f32, int64_t grid, hipStream_t s) {
    // the finishing block holds one piece per thread and 32 row keys per thread
    if (grid <= 0 || a.n_items > (int64_t)kFusedKeys || a.P > ST_NT || grid != (int64_t)a.B * a.P)
        return hipErrorInvalidValue;
    const int64_t per = (a.n_items + ST_NT - 1) / ST_NT;  // keys per thread of the finishing block
#define GENREC_FUSED(T, FV) hipLaunchKernelGGL((stream_score_kernel<T, 3, FV>), dim3(grid), dim3(ST_NT), 0, s, a)
    if (f32) {
        if (per <= 8) GENREC_FUSED(float, 8);
        else if (per <= 16) GENREC_FUSED(float, 16);
        else GENREC_FUSED(float, 32);
    } else {
        if (per <= 8) GENREC_FUSED(uint16_t, 8);
        else if (per <= 16) GENREC_FUSED(uint16_t, 16);
        else GENREC_FUSED(uint16_t, 32);
    }
#undef GENREC_FUSED
    return hipGetLastError();
}

hipError_t launch_stream(const StreamArgs& a, int mode, bool f32, int64_t grid, hipStream_t s) {
    if (grid <= 0) return hipSuccess;
    if (f32) {
        if (mode == 0) hipLaunchKernelGGL((stream_score_kernel<float, 0>), dim3(grid), dim3(ST_NT), 0, s, a);
        else if (mode == 1) hipLaunchKernelGGL((stream_score_kernel<float, 1>), dim3(grid), dim3(ST_NT), 0, s, a);
        else hipLaunchKernelGGL((stream_score_kernel<float, 2>), dim3(grid), dim3(ST_NT), 0, s, a);
    } else {
        if (mode == 0) hipLaunchKernelGGL((stream_score_kernel<uint16_t, 0>), dim3(grid), dim3(ST_NT), 0, s, a);
        else if (mode == 1) hipLaunchKernelGGL((stream_score_kernel<uint16_t, 1>), dim3(grid), dim3(ST_NT), 0, s, a);
        else hipLaunchKernelGGL((stream_score_kernel<uint16_t, 2>), dim3(grid), dim3(ST_NT), 0, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_threshold(const ThresholdArgs& a, hipStream_t s) {
    if (a.n_sample > (int64_t)TH_KEYS || a.n_sample % 4 != 0) return hipErrorInvalidValue;
    // many threads for few users; keys per thread sized to the sample
    const bool half = a.n_sample <= (int64_t)(TH_KEYS / 2);
    if (a.B <= 512) {
        if (half) hipLaunchKernelGGL((threshold_kernel<1024, TH_KEYS / 2>), dim3(a.B), dim3(1024), 0, s, a);
        else hipLaunchKernelGGL((threshold_kernel<1024, TH_KEYS>), dim3(a.B), dim3(1024), 0, s, a);
    } else {
        if (half) hipLaunchKernelGGL((threshold_kernel<256, TH_KEYS / 2>), dim3(a.B), dim3(256), 0, s, a);
        else hipLaunchKernelGGL((threshold_kernel<256, TH_KEYS>), dim3(a.B), dim3(256), 0, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_topk_rows(const TopkRowsArgs& a, hipStream_t s) {
    if (a.R <= 0) return hipSuccess;
    if ((int64_t)a.R * a.nchunk > 2147483647) return hipErrorInvalidValue;  // one block per (row, chunk)
    if (a.reg == 2) {  // one block per row, the row in registers
        if (a.N > TK_SEG || a.nchunk != 1 || a.K > GENREC_KMAX || a.K < 1) return hipErrorInvalidValue;
        hipLaunchKernelGGL(topk_row_kernel, dim3(a.R), dim3(TK_NT), 0, s, a);
        return hipGetLastError();
    }
    if (a.reg == 3) {  // the filter route
        if (a.N <= TK_SEG || a.K > kTopkBoundMaxK || a.K < 1 || a.C != TF_COLS ||
            (int64_t)a.nchunk * TF_COLS < a.N || a.sj < 1 || a.sj > TK_NT || !a.tthr || !a.tcnt || !a.part)
            return hipErrorInvalidValue;
        hipLaunchKernelGGL(topk_sample_kernel, dim3(a.R), dim3(TK_NT), 0, s, a);
        hipLaunchKernelGGL(topk_filter_kernel, dim3((unsigned)((int64_t)a.R * a.nchunk)), dim3(TK_NT), 0, s, a);
        hipLaunchKernelGGL(topk_cand_kernel, dim3(a.R), dim3(TK_NT), 0, s, a);
        return hipGetLastError();
    }
    if (a.reg) {
        if (a.C != TK_SEG || a.K > GENREC_KMAX || a.nchunk < 2 || (int64_t)a.nchunk * a.K > TK_NT * TK_MV)
            return hipErrorInvalidValue;
        hipLaunchKernelGGL(topk_seg_kernel, dim3((unsigned)((int64_t)a.R * a.nchunk)), dim3(TK_NT), 0, s, a);
        hipLaunchKernelGGL(topk_rowmerge_kernel, dim3(a.R), dim3(TK_NT), 0, s, a);
        return hipGetLastError();
    }
    const dim3 grid((unsigned)((int64_t)a.R * a.nchunk));
    if (a.K <= 256) hipLaunchKernelGGL((topk_chunk_kernel<MG_GCAP_SMALL>), grid, dim3(SEL_NT), 0, s, a);
    else hipLaunchKernelGGL((topk_chunk_kernel<SEL_GCAP>), grid, dim3(SEL_NT), 0, s, a);
    if (a.nchunk > 1) hipLaunchKernelGGL(topk_merge_rows_kernel, dim3(a.R), dim3(SEL_NT), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t s) {
    if (a.small)
        hipLaunchKernelGGL((merge_kernel<MG_GCAP_SMALL, MG_PB_SMALL>), dim3(a.B), dim3(SEL_NT), 0, s, a);
    else
        hipLaunchKernelGGL((merge_kernel<SEL_GCAP, MG_PB_LARGE>), dim3(a.B), dim3(SEL_NT), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_narrow(const NarrowArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(narrow_kernel, dim3(a.B), dim3(NR_NT), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_hot_select(const HotArgs& a, hipStream_t s) {
    const int fill_grid = (int)std::min<int64_t>(4096, ceil_div(a.M, HOT_NT));
    hipLaunchKernelGGL(hot_clear_kernel, dim3(fill_grid), dim3(HOT_NT), 0, s, a);
    const int64_t n_samples = (a.nnz + kHotSample - 1) / kHotSample;
    if (n_samples > 0)
        hipLaunchKernelGGL(hot_count_kernel, dim3((unsigned)std::min<int64_t>(4096, ceil_div(n_samples, HOT_NT))),
                           dim3(HOT_NT), 0, s, a);
    // few blocks: each adds its LDS histogram to the global one once
    hipLaunchKernelGGL(hot_hist_kernel, dim3((unsigned)std::min<int64_t>(256, ceil_div(a.M, HOT_NT))), dim3(HOT_NT), 0, s, a);
    hipLaunchKernelGGL(hot_pick_kernel, dim3(1), dim3(HOT_PICK_NT), 0, s, a);
    hipLaunchKernelGGL(hot_blockcount_kernel, dim3((unsigned)a.n_hblk), dim3(HOT_NT), 0, s, a);
    hipLaunchKernelGGL(hot_scan_kernel, dim3(1), dim3(HOT_PICK_NT), 0, s, a);
    hipLaunchKernelGGL(hot_assign_kernel, dim3((unsigned)a.n_hblk), dim3(HOT_NT), 0, s, a);
    hipLaunchKernelGGL(hot_gather_kernel, dim3((unsigned)a.t_max), dim3(HOT_NT), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_cand_plan(const CandPlanArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(cand_plan_kernel, dim3(1), dim3(PL_NT), 0, s, a);
    return hipGetLastError();
}

}  // namespace genrec
