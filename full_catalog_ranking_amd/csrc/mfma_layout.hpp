// Tile geometry of the MFMA scoring kernel: which catalog / user row and
// k-chunk every lane moves into LDS, and where the MFMA fragment reads find
// it.  Host+device so that the host test build can enumerate every case and
// check bounds and the write/read agreement without a GPU.
#pragma once

#if defined(__HIPCC__)
#define GENREC_HD __host__ __device__
#else
#define GENREC_HD
#endif

namespace genrec {

constexpr int MF_TI = 256;   // items per tile (MFMA rows)
constexpr int MF_TU = 256;   // users per tile (MFMA columns)
constexpr int MF_BK = 32;    // reduction depth per LDS stage
constexpr int MF_NS = 4;     // LDS ring stages (3 in flight while one is read): 128 KiB; 5 stages time the same
constexpr int MF_NT = 512;   // threads: 8 waves (2 per SIMD) in a 2 x 4 layout of 128 x 64 wave tiles
constexpr int MF_NW = MF_NT / 64;
constexpr int MF_WU = 64;    // users per wave tile
constexpr int MF_UB = MF_WU / 32;  // 32-wide user blocks per wave tile
constexpr int MF_ROWB = MF_BK * 2;                   // bytes per staged row (64)
constexpr int MF_STAGE = (MF_TI + MF_TU) * MF_ROWB;  // 32 KiB per stage
constexpr int MF_DMA = 2;    // 16-byte DMA ops per lane per operand per stage
static_assert(MF_DMA * MF_NW * 64 * 16 == MF_TI * MF_ROWB, "DMA ops must cover one operand stage");

// 16-byte chunk swizzle within a 64-byte staged row.  The fragment read of a
// wave takes 32 consecutive rows at k-chunk c (lanes 0-31) and c+1 (lanes
// 32-63); on gfx950 that ds_read_b128 runs at the full 256 B/clk (no bank-
// conflict cycles in the SQ_LDS_BANK_CONFLICT counter) with the chunk xor-ed
// by bits 2-3 of the row, while e.g. bits 1-2 xor bits 3-4 cost a 2-way
// conflict.
GENREC_HD inline int mf_swz(int row) { return (row >> 2) & 3; }

// DMA: wave w, op j writes the 1 KiB of staged rows (j*NW + w)*16 .. +16;
// lane l writes 16 bytes at l*16, i.e. staged row (j*NW + w)*16 + l/4 at
// chunk position l%4, holding global k-chunk (l%4) ^ swz(row).
GENREC_HD inline int mf_dma_row0(int w, int lane) { return w * 16 + (lane >> 2); }  // staged row of op 0
GENREC_HD inline int mf_dma_row(int w, int lane, int j) { return mf_dma_row0(w, lane) + MF_NW * 16 * j; }
// swz(row) is the same for every op j of a lane (NW*16*j = 128 j changes
// neither bit field it reads), so one k-chunk offset serves all ops.
GENREC_HD inline int mf_dma_kchunk(int w, int lane) { return (lane & 3) ^ mf_swz(mf_dma_row0(w, lane)); }
GENREC_HD inline int mf_dma_lds_byte(int w, int lane, int j) { return (j * MF_NW + w) * 1024 + lane * 16; }
// Byte offset, within one operand tile of rows of row_bytes bytes, that lane
// `lane` of wave `w` reads for op j (the k-chunk of the stage's k0 is added
// through the tile base): its staged row's start plus its 16-byte k-chunk.
GENREC_HD inline long long mf_dma_voff_bytes(int w, int lane, int j, long long row_bytes) {
    return (long long)mf_dma_row(w, lane, j) * row_bytes + mf_dma_kchunk(w, lane) * 16;
}
// The same for rows of D bf16 elements.
GENREC_HD inline long long mf_dma_voff(int w, int lane, int j, int D) { return mf_dma_voff_bytes(w, lane, j, 2LL * D); }

// The sampled pre-pass scores one full catalog tile out of every window of G
// (tiles [t G, t G + G) clipped to the full_tiles whole tiles): window t's
// tile sits at a fixed pseudo-random position inside it (an integer hash of
// t), not always at its start, so that a catalog stored in a periodic or
// clustered order is not sampled in step with it.  G = 1: tile t itself.
GENREC_HD inline long long mf_sample_tile(long long t, long long G, long long full_tiles) {
    if (G <= 1) return t;
    const long long w0 = t * G;
    const long long span = full_tiles - w0 < G ? full_tiles - w0 : G;
    unsigned h = (unsigned)(t + 1) * 0x9E3779B1u;
    h ^= h >> 15;
    h *= 0x85EBCA77u;
    h ^= h >> 13;
    return span > 0 ? w0 + (long long)(h % (unsigned)span) : w0;
}

// Fragment read: byte offset of (staged row, k-chunk) within an operand stage.
GENREC_HD inline int mf_frag_lds_byte(int row, int kchunk) { return row * MF_ROWB + ((kchunk ^ mf_swz(row)) << 4); }

}  // namespace genrec
