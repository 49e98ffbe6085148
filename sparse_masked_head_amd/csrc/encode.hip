// Two-level mask encoder on the GPU.
//
// Format ("Accelerating Sparse Transformer Inference on GPU", gist.science
// explainer, Technical summary > Methodology > 1. Unified MHA module,
// storage-format items): 64x64 outer tiles; empty tiles are left out; full
// tiles are listed by column only; partial tiles are listed and carry one
// uint64 bitmap per 8x8 inner tile.  Exact layout: include/smh.h.
//
// Input: a stack of G masks [G][S][S]; the encoding has G * n outer-tile
// rows (mask after mask).  Work unit: a segment of one outer-tile row
// (seg_plan), numbered row by row, left to right, so the encoding is the
// concatenation of the segments' tile lists in that order.
//   strip pass (one workgroup per segment): stream the segment's 64-row
//     strip, one window (64 rows x 512 bytes) at a time with the next
//     window's loads in flight; build the inner-tile words of every tile in
//     LDS and count its elements; classify the tiles (full / partial /
//     empty) and write the segment's tile columns, partial-tile words,
//     tile counts, valid-pair count and covered query rows to scratch;
//   scan (one workgroup): exclusive prefix of the segments' tile counts,
//     row pointers, statistics and the heavy-first row order;
//   placement (one workgroup per segment): copy the segment's columns and
//     words to their final places, the columns among its row's first four
//     stored tiles to the row's summary (row_info), and write the row-wise
//     entries of its sparse tiles.
// With at most kFusedMaxSegs segments and kFusedRows rows the scan runs as
// one extra workgroup (the first) of the placement launch and each
// placement workgroup adds up the counts before it itself (cheap at that
// size, and one launch fewer).  No
// workgroup ever waits for another.  Every output is a pure function of
// the mask: the result is deterministic and equals appending tiles row by
// row, column by column.
#include <math.h>
#include <mutex>

#include "bits.h"
#include "smh_internal.h"

namespace smh {
namespace {

// High bit of each byte of w set iff that byte is nonzero.
__device__ inline uint32_t nonzero_bytes(uint32_t w) {
    return (((w & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | w) & 0x80808080u;
}

// Collapse the four byte flags of nonzero_bytes() into bits 0..3.
// After the shift the flags sit at bits 0, 8, 16, 24; multiplying by
// 1 + 2^7 + 2^14 + 2^21 moves flag k to bit 21 + k with no carries.
__device__ inline uint32_t gather4(uint32_t hb) {
    return ((hb >> 7) * 0x00204081u >> 21) & 0xFu;
}

// 8 mask bytes (two dwords, byte c = column c) -> one 8-bit inner-tile row.
__device__ inline uint32_t row_bits8(uint32_t lo, uint32_t hi) {
    return gather4(nonzero_bytes(lo)) | (gather4(nonzero_bytes(hi)) << 4);
}

typedef uint32_t u4v __attribute__((ext_vector_type(4)));

// How the strip pass reads a mask row: kAligned64 (S % 64 == 0: whole
// 16-byte pieces, no bounds beyond the tile count), kAligned16 (S % 16 == 0:
// whole pieces, rows and pieces past S read as zero), kDwords (rows are not
// 16-byte aligned: the aligned dwords that hold the piece's valid bytes,
// funnel-shifted into place; elements past S read as zero).  Every dword
// loaded holds at least one byte of the mask.
enum LoadMode { kAligned64 = 0, kAligned16 = 1, kDwords = 2 };

// Loads of one window: thread t reads, for k = 0..7, mask row 8k + (t >> 5)
// of the strip (strip row 0 = mask row row0), bytes 16*(t & 31) .. +15 of
// the window (tile (t & 31) >> 2, columns 16*(t & 3) .. +15 of it).  Each
// wavefront instruction reads two contiguous 512-byte row pieces.  Tiles
// at or past n, and elements outside the S x S mask, hold no mask bytes:
// the aligned modes still load such a piece (from column 0, and the last
// row, of the strip: in bounds) and window_valid() tells which pieces to
// zero when they are used; kDwords loads them as zero.  (A load under a
// per-lane condition became a branch, and the compiler then waited for
// every outstanding load, the next window's among them, before using any.)
template <int kMode>
__device__ __forceinline__ void load_window(u4v (&v)[8], const uint8_t *strip,
                                            int S, int n, int row0, int J0, int t) {
    const int r0 = t >> 5, c = t & 31;
    const bool ok = J0 + (c >> 2) < n;
    const int col = 64 * J0 + 16 * c;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const uint8_t *p = strip + (size_t)(8 * k + r0) * S + col;
        const bool row_ok = row0 + 8 * k + r0 < S;
        if (kMode == kAligned64) {
            v[k] = *reinterpret_cast<const u4v *>(ok ? p : strip + (size_t)(8 * k + r0) * S);
        } else if (kMode == kAligned16) {
            const size_t rr = (size_t)min(8 * k + r0, S - 1 - row0);
            v[k] = *reinterpret_cast<const u4v *>(strip + rr * S + (ok && col < S ? col : 0));
        } else {
            uint32_t wd[4] = {0, 0, 0, 0};
            if (ok && row_ok && col < S) {
                const int nb = min(16, S - col);  // valid bytes of the piece
                const uintptr_t at = reinterpret_cast<uintptr_t>(p);
                const uint32_t *w = reinterpret_cast<const uint32_t *>(at & ~(uintptr_t)3);
                const int sh = (int)(at & 3);
                const int nd = (sh + nb + 3) >> 2;  // dwords holding them, <= 5
                uint32_t x[5];
#pragma unroll
                for (int i = 0; i < 5; ++i) x[i] = i < nd ? w[i] : 0u;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    // bytes sh .. sh+3 of (x[i+1] : x[i]), then the bytes past S cleared
                    const uint32_t y = __builtin_amdgcn_alignbyte(x[i + 1], x[i], sh);
                    const int keep = nb - 4 * i;
                    wd[i] = keep >= 4 ? y : keep <= 0 ? 0u : y & ((1u << (8 * keep)) - 1u);
                }
            }
            v[k] = u4v{wd[0], wd[1], wd[2], wd[3]};
        }
    }
}

// Bit k: piece k of load_window holds mask bytes (always, for kDwords,
// whose loads already read zero outside the mask).
template <int kMode>
__device__ __forceinline__ uint32_t window_valid(int S, int n, int row0, int J0, int t) {
    if (kMode == kDwords) return 0xFFu;
    const int r0 = t >> 5, c = t & 31;
    const bool ok = J0 + (c >> 2) < n;
    const int col = 64 * J0 + 16 * c;
    uint32_t vm = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const bool row_ok = row0 + 8 * k + r0 < S;
        const bool valid = ok && (kMode == kAligned64 || (row_ok && col < S));
        vm |= (uint32_t)valid << k;
    }
    return vm;
}

template <typename T> __device__ inline T block_sum(T x, T *sh) {
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = x;
    __syncthreads();
    const T r = sh[0] + sh[1] + sh[2] + sh[3];
    __syncthreads();  // sh may be reused right away
    return r;
}

__device__ inline int block_max(int x, int *sh) {
    for (int off = 32; off > 0; off >>= 1) x = max(x, __shfl_xor(x, off));
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = x;
    __syncthreads();
    const int r = max(max(sh[0], sh[1]), max(sh[2], sh[3]));
    __syncthreads();
    return r;
}


constexpr int kMaxSegTiles = kWin * kMaxSegWin;  // 64
// Words per tile of a strip pass's LDS copy of a segment's inner-tile words:
// 64 and one of padding.  The byte writes that build the words put one
// wavefront's lanes on 8 tiles x 4 words at a time; with tiles 512 bytes
// apart all of them fell on 4 of the LDS banks, with 520 on about 14
// (encode 1-2.5% faster).
constexpr int kLW = 65;
constexpr int kMaxN = SMH_MAX_S / 64;              // outer tiles per side
// Scan sizes: rows of the encoding it holds in LDS, and bins of its
// stored-tile-count histogram (counts 0..n; 0 = rank by direct comparison
// with every row instead).  The fused form (scan as one workgroup of the
// placement launch) is kept small because every placement workgroup
// reserves its LDS.
constexpr int kScanRows = SMH_MAX_ENC_ROWS, kScanBins = kMaxN + 1;
constexpr int kFusedRows = 1024, kFusedBins = 0;
constexpr int kFusedMaxSegs = 2048;

struct Seg {  // per-segment scratch (EncLayout)
    uint64_t *cnt, *off, *nnz, *any, *sp;
    int32_t *fcol, *pcol, *pop;
    uint64_t *words;
    int32_t *ecnt;  // [segment][group]: row-wise entries of its sparse tiles
    int rowfmt;     // the row-wise entries are built (S <= 65536)
    int cap;  // tiles of room per segment
};

// Sparse partial tiles (count << kSpShift | valid pairs) of a segment or a
// sum of segments: the pairs stay below 2^40 and the count below 2^24.
constexpr int kSpShift = 40;
constexpr uint64_t kSpLow = (1ull << kSpShift) - 1;

// The row-wise entries of the segment's sparse tiles (tkind bit 18), per
// group q of 16 query rows (inner-tile rows 2q, 2q + 1), are one per key
// that some row of the group sees: rows << 16 | key.  The strip pass only
// counts them (wavefront w: tiles w, w + 4, ...; lane (ir, ic) owns word
// (ir, ic), the lanes of even ir count their column block's live keys for
// group ir / 2 from their word and the word below it) and stores the
// segment's total per group; the placement pass, which knows where the
// row's lists start, writes them (place_entries).
__device__ void strip_entry_counts(int s, int nwin, Seg sg, uint64_t (*lw)[kLW],
                                   const int *tkind) {
    __shared__ int ecnt_t[4][4];  // per wavefront and group
    const int t = threadIdx.x, w = t >> 6, lane = t & 63;
    const int ir = lane >> 3, ic = lane & 7, q = ir >> 1;
    const bool top = (ir & 1) == 0;
    const int ntile = kWin * nwin;
    int c = 0;
    for (int l = w; l < ntile; l += 4)
        if ((tkind[l] & (1 << 18)) && top)
            c += __popc(live_columns(lw[l][lane] | lw[l][lane + 8]));
    c += __shfl_xor(c, 1);
    c += __shfl_xor(c, 2);
    c += __shfl_xor(c, 4);
    c += __shfl_xor(c, 8);  // the two inner-tile rows' lanes: ir and ir ^ 1
    if (lane == 16 * q) ecnt_t[w][q] = c;
    __syncthreads();
    if (t < 4) sg.ecnt[4 * (size_t)s + t] = ecnt_t[0][t] + ecnt_t[1][t] + ecnt_t[2][t] + ecnt_t[3][t];
}

// Shared tail of the strip passes: classify the segment's tiles (wavefront
// 0, lane = tile), write its columns, counts, valid pairs and covered rows
// (any64, read in lane 0 of wavefront 0: bit r = query row r of the strip),
// then its partial-tile words (one wavefront per tile).  wsum[l][0..3] add
// up to tile l's valid elements.
__device__ void strip_classify(int s, int nwin, int w0, int n, Seg sg,
                               uint64_t (*lw)[kLW], int (*wsum)[4], int *tkind,
                               uint64_t any64) {
    __shared__ int seg_sparse;  // the segment has a sparse partial tile
    const int t = threadIdx.x, w = t >> 6, lane = t & 63;
    if (w == 0) {
        const int wi = lane >> 3, J = kWin * (w0 + wi) + (lane & 7);
        const bool valid = wi < nwin && J < n;
        const int cnt = valid ? wsum[lane][0] + wsum[lane][1] + wsum[lane][2] +
                                    wsum[lane][3]
                              : 0;
        const bool full = cnt == 64 * 64, part = cnt > 0 && !full;
        const uint64_t mf = __ballot(full), mp = __ballot(part);
        const uint64_t below = (1ull << lane) - 1;
        const int rf = __popcll(mf & below), rp = __popcll(mp & below);
        tkind[lane] = full ? (1 << 17) | rf
                    : part ? (1 << 16) | rp | (cnt <= SMH_SPARSE_TILE_MAX ? 1 << 18 : 0)
                           : 0;
        if (full) sg.fcol[(size_t)s * sg.cap + rf] = J;
        if (part) {
            sg.pcol[(size_t)s * sg.cap + rp] = J;
            sg.pop[(size_t)s * sg.cap + rp] = cnt;
        }
        const bool sparse = part && cnt <= SMH_SPARSE_TILE_MAX;
        long long nz = cnt, spz = sparse ? cnt : 0;
        for (int off = 32; off > 0; off >>= 1) {
            nz += __shfl_xor(nz, off);
            spz += __shfl_xor(spz, off);
        }
        const uint64_t ms = __ballot(sparse);
        if (lane == 0) {
            seg_sparse = ms != 0;
            sg.cnt[s] = ((uint64_t)__popcll(mf) << 32) | (uint64_t)__popcll(mp);
            sg.nnz[s] = (uint64_t)nz;
            sg.any[s] = any64;
            sg.sp[s] = ((uint64_t)__popcll(ms) << kSpShift) | (uint64_t)spz;
        }
    }
    __syncthreads();
    for (int l = w; l < kWin * nwin; l += 4) {
        const int k = tkind[l];
        if (k & (1 << 16))
            sg.words[((size_t)s * sg.cap + (k & 0xFFFF)) * 64 + lane] = lw[l][lane];
    }
    if (sg.rowfmt) {
        if (seg_sparse)
            strip_entry_counts(s, nwin, sg, lw, tkind);
        else if (t < 4)
            sg.ecnt[4 * (size_t)s + t] = 0;
    }
}

template <int kMode>
__global__ __launch_bounds__(256) void enc_strip(const uint8_t *__restrict__ mask,
                                                 int S, int n, SegPlan plan, Seg sg) {
    // segment s: row s / per_row of the encoding = outer-tile row I of mask g
    // inner-tile words of the segment's tiles (tile l = 8 * window + j)
    __shared__ uint64_t lw[kMaxSegTiles][kLW];
    __shared__ int wsum[kMaxSegTiles][4];  // tile counts per wavefront
    __shared__ int tkind[kMaxSegTiles];    // rank | 1<<16 partial | 1<<17 full
    __shared__ uint32_t rows_any[8];

    const int t = threadIdx.x, w = t >> 6, lane = t & 63;
    const int s = blockIdx.x;
    const int row = s / plan.per_row, seg_c = s - row * plan.per_row;
    const int g = row / n, I = row - g * n;
    const int nw = (n + kWin - 1) / kWin;
    const int w0 = seg_c * plan.win;
    const int nwin = min(plan.win, nw - w0);  // windows in this segment

    {
        const uint8_t *strip = mask + (size_t)g * S * S + (size_t)64 * I * S;
        uint8_t *wb = reinterpret_cast<uint8_t *>(&lw[0][0]);
        const int r0 = t >> 5, c = t & 31, jj = c >> 2, quarter = c & 3;
        uint32_t any_rows = 0;  // bit k: row 8k + r0 has a valid element
        // one window's words and counts (window wi of the segment, its
        // pieces in v; pieces holding no mask bytes count as zero)
        auto process = [&](const u4v(&v)[8], int wi) __attribute__((always_inline)) {
            const uint32_t vm = window_valid<kMode>(S, n, 64 * I, kWin * (w0 + wi), t);
            uint8_t *tb = wb + (size_t)(kWin * wi + jj) * (8 * kLW);
            int cnt = 0;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                // inner tiles (k, 2*quarter) and (k, 2*quarter+1), their row r0
                const uint32_t keep = 0u - ((vm >> k) & 1u);
                const uint32_t b0 = row_bits8(v[k][0], v[k][1]) & keep;
                const uint32_t b1 = row_bits8(v[k][2], v[k][3]) & keep;
                tb[(k * 8 + 2 * quarter) * 8 + r0] = (uint8_t)b0;
                tb[(k * 8 + 2 * quarter + 1) * 8 + r0] = (uint8_t)b1;
                cnt += __popc(b0) + __popc(b1);
                any_rows |= (uint32_t)((b0 | b1) != 0) << k;
            }
            // lanes of one tile within this wavefront: quarters (xor 1, 2)
            // and the two row offsets (xor 32)
            cnt += __shfl_xor(cnt, 1);
            cnt += __shfl_xor(cnt, 2);
            cnt += __shfl_xor(cnt, 32);
            if (lane < 32 && quarter == 0) wsum[kWin * wi + jj][w] = cnt;
        };
        // Two register sets, used in turn (the loop unrolled by two): the
        // next window's loads are issued before this one is processed, and
        // every path issues the same loads (past the last window, the last
        // one again: cache hits), so the compiler's waits count exactly the
        // loads still in flight.  (With one set copied from the other, the
        // wait at the top of the loop covered the next window's loads too.)
        u4v va[8], vb[8];
        auto win_at = [&](int wi) __attribute__((always_inline)) {
            return kWin * (w0 + min(wi, nwin - 1));
        };
        load_window<kMode>(va, strip, S, n, 64 * I, win_at(0), t);
        for (int wi = 0; wi < nwin; wi += 2) {
            load_window<kMode>(vb, strip, S, n, 64 * I, win_at(wi + 1), t);
            process(va, wi);
            if (wi + 1 >= nwin) break;
            load_window<kMode>(va, strip, S, n, 64 * I, win_at(wi + 2), t);
            process(vb, wi + 1);
        }
        // query rows covered in this segment: OR over the 32 lanes sharing r0
        uint32_t a = any_rows;
#pragma unroll
        for (int off = 1; off < 32; off <<= 1) a |= __shfl_xor(a, off);
        if (c == 0) rows_any[r0] = a;
    }
    __syncthreads();
    // bit 8k + r: query row 8k + r of the strip (one ballot in wavefront 0,
    // lane 8k + r reading bit k of rows_any[r]; strip_classify reads it there)
    uint64_t any64 = 0;
    if (w == 0)
        any64 = __builtin_amdgcn_ballot_w64(((rows_any[lane & 7] >> (lane >> 3)) & 1u) != 0);
    strip_classify(s, nwin, w0, n, sg, lw, wsum, tkind, any64);
}

// ---- masks described by a pattern (smh_pattern) instead of stored ----

struct Pattern {
    int causal, window, grow, gcol;
    const uint8_t *blocks;    // [n][n] block map or null
    uint32_t keep16, rand16;  // probabilities as thresholds out of 2^16
    uint64_t seed;
};

// Bits lo .. hi of a 64-bit word (0 <= lo <= hi <= 63).
__device__ inline uint64_t bit_range(int lo, int hi) {
    return (~0ull >> (63 - hi)) & (~0ull << lo);
}

// SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
// generators", OOPSLA 2014): output number k (from 0) of the stream seeded
// with `seed` is the mix function applied to the state seed + (k + 1) *
// gamma; consecutive outputs step the state by gamma.
constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;
__device__ inline uint64_t splitmix64_mix(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

// Bit c (c < 64) set iff element e0 + c of the row-major S x S mask draws
// below thr: element e draws bits 16 (e % 4) .. 16 (e % 4) + 15 of
// SplitMix64 output e / 4.  The 17 outputs from e0 / 4 on cover elements
// 4 (e0 / 4) .. +67; their 68 decisions are built four at a time (one
// nibble per output) and shifted into place once.
__device__ inline uint64_t draw_bits(uint64_t seed, uint64_t e0, uint32_t thr) {
    if (thr == 0) return 0;
    if (thr >= 65536u) return ~0ull;
    const uint64_t g0 = e0 >> 2;
    const int sh = (int)(e0 & 3);
    uint64_t lo = 0;  // decisions of elements 4 g0 .. 4 g0 + 63
    uint32_t hi = 0;  // elements 4 g0 + 64 .. + 67
    uint64_t state = seed + (g0 + 1) * kGamma;  // of output g0
#pragma unroll
    for (int q = 0; q < 17; ++q, state += kGamma) {
        const uint64_t x = splitmix64_mix(state);
        const uint32_t a = (uint32_t)x, b = (uint32_t)(x >> 32);
        const uint32_t nib = (uint32_t)((a & 0xFFFFu) < thr) |
                             ((uint32_t)((a >> 16) < thr) << 1) |
                             ((uint32_t)((b & 0xFFFFu) < thr) << 2) |
                             ((uint32_t)((b >> 16) < thr) << 3);
        if (q < 16)
            lo |= (uint64_t)nib << (4 * q);
        else
            hi = nib;
    }
    return sh ? (lo >> sh) | ((uint64_t)hi << (64 - sh)) : lo;
}

// Row i of the pattern's mask over columns 64J .. 64J+63 (bit c = column
// 64J + c).  Valid: inside S x S, j <= i when causal, and any of: the band
// |i - j| <= window, a global row or column, a listed block (map value 1:
// every element; other nonzero values: elements drawn with keep16), else
// an element drawn with rand16.
__device__ inline uint64_t pattern_row_bits(const Pattern &p, int S, int n,
                                            int i, int J) {
    const int c0 = 64 * J;
    if (i >= S || c0 >= S) return 0;
    uint64_t lim = S - c0 >= 64 ? ~0ull : bit_range(0, S - c0 - 1);
    if (p.causal) {
        if (i < c0) return 0;
        if (i - c0 < 63) lim &= bit_range(0, i - c0);
    }
    if (i < p.grow) return lim;
    uint64_t m = 0;
    if (p.window >= 0) {
        const long long lo = max((long long)i - p.window, (long long)c0);
        const long long hi = min((long long)i + p.window, (long long)c0 + 63);
        if (lo <= hi) m |= bit_range((int)(lo - c0), (int)(hi - c0));
    }
    if (p.gcol > c0) m |= p.gcol - c0 >= 64 ? ~0ull : bit_range(0, p.gcol - c0 - 1);
    const int blk = p.blocks ? p.blocks[(size_t)(i >> 6) * n + J] : 0;
    if (blk == 1) return lim;
    if ((~m & lim) != 0)
        m |= draw_bits(p.seed, (uint64_t)i * S + c0, blk ? p.keep16 : p.rand16);
    return m & lim;
}

// Strip pass of a pattern: the same segments and outputs as enc_strip, with
// the inner-tile words computed instead of loaded.  Lane = query row of the
// strip; wavefront w takes tiles w and w + 4 of each window.
__global__ __launch_bounds__(256) void enc_pattern_strip(Pattern p, int S, int n,
                                                         SegPlan plan, Seg sg) {
    __shared__ uint64_t lw[kMaxSegTiles][kLW];
    __shared__ int wsum[kMaxSegTiles][4];
    __shared__ int tkind[kMaxSegTiles];
    __shared__ uint64_t wany[4];
    const int t = threadIdx.x, w = t >> 6, lane = t & 63;
    const int s = blockIdx.x;
    const int I = s / plan.per_row, seg_c = s - I * plan.per_row;
    const int nw = (n + kWin - 1) / kWin;
    const int w0 = seg_c * plan.win;
    const int nwin = min(plan.win, nw - w0);
    const int i = 64 * I + lane, ir = lane >> 3, r = lane & 7;
    uint8_t *wb = reinterpret_cast<uint8_t *>(&lw[0][0]);
    bool any = false;
    for (int wi = 0; wi < nwin; ++wi) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int jj = w + 4 * h, J = kWin * (w0 + wi) + jj;
            const uint64_t m = J < n ? pattern_row_bits(p, S, n, i, J) : 0;
            any |= m != 0;
            uint8_t *tb = wb + (size_t)(kWin * wi + jj) * (8 * kLW);
#pragma unroll
            for (int ic = 0; ic < 8; ++ic) tb[(ir * 8 + ic) * 8 + r] = (uint8_t)(m >> (8 * ic));
            int cnt = __popcll(m);
            for (int off = 32; off > 0; off >>= 1) cnt += __shfl_xor(cnt, off);
            if (lane < 4) wsum[kWin * wi + jj][lane] = lane == 0 ? cnt : 0;
        }
    }
    const uint64_t a = __ballot(any);
    if (lane == 0) wany[w] = a;
    __syncthreads();
    strip_classify(s, nwin, w0, n, sg, lw, wsum, tkind,
                   wany[0] | wany[1] | wany[2] | wany[3]);
}

// Exclusive scan over the 256 threads of a workgroup.
__device__ inline unsigned long long block_exclusive_scan(unsigned long long x,
                                                          unsigned long long *sh) {
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    unsigned long long incl = x;
    for (int d = 1; d < 64; d <<= 1) {
        const unsigned long long y = __shfl_up(incl, d);
        if (lane >= d) incl += y;
    }
    if (lane == 63) sh[w] = incl;
    __syncthreads();
    unsigned long long before = 0;
    for (int q = 0; q < w; ++q) before += sh[q];
    const unsigned long long r = before + incl - x;
    __syncthreads();
    return r;
}

// Exclusive scan of the segments' tile counts, row pointers, statistics and
// the heavy-first schedule (one workgroup of 256 threads) over the R = G * n
// rows of the encoding.  Writes each segment's offsets when `offsets` is
// set.  Thread t owns a run of whole rows; every load of the first pass is
// independent of the others, so the pass costs one memory round trip.
// Schedule: row J's rank = rows with more stored tiles + rows before J with
// as many.  Up to a few hundred rows each thread compares its rows with
// every row (a loop of uniform length, whose loads pipeline); for more, the
// first term comes from a histogram of the counts and the second from a
// running histogram over blocks of 256 rows plus a count inside J's block.
template <int kRows, int kBins>
__device__ void scan_body(int S, int n, int R, int G, SegPlan plan, Seg sg,
                          smh_mask_enc enc, bool offsets) {
    constexpr int kH = kBins > 0 ? kBins : 1;
    // full << 16 | partial (each <= n <= 2048); without bins, then the rank keys
    __shared__ __attribute__((aligned(16))) uint32_t rowc[kRows];
    __shared__ int above[kH];         // histogram, then rows with a larger count
    __shared__ int seen[kH];          // rows of earlier blocks per count
    __shared__ unsigned long long sh_u[4];
    __shared__ long long sh_l[4];
    __shared__ int sh_i[4];
    __shared__ unsigned long long sh_tot;  // full << 32 | partial, all rows
    const int t = threadIdx.x;
    const int C = plan.per_row;
    if constexpr (kBins > 0) {
        for (int c = t; c <= n; c += 256) {
            above[c] = 0;
            seen[c] = 0;
        }
        __syncthreads();
    }
    const int rows_per = (R + 255) / 256;
    const int r_lo = min(R, t * rows_per), r_hi = min(R, r_lo + rows_per);
    unsigned long long own = 0;
    long long nnz = 0, empty = 0, spw = 0, ents = 0;
    int mx = 0;
    for (int I = r_lo; I < r_hi; ++I) {
        unsigned long long rc = 0;
        uint64_t an = 0;
#pragma unroll 8
        for (int c = 0; c < C; ++c) {
            rc += sg.cnt[I * C + c];
            nnz += (long long)sg.nnz[I * C + c];
            an |= sg.any[I * C + c];
            spw += (long long)sg.sp[I * C + c];
            // read whatever the format (the array is always there; its
            // sum is dropped without row-wise entries): a load under the
            // flag became a branch with a wait of its own per segment
            const int4 e = reinterpret_cast<const int4 *>(sg.ecnt)[I * C + c];
            ents += (long long)e.x + e.y + e.z + e.w;
        }
        const int f = (int)(rc >> 32), p = (int)(rc & 0xFFFFFFFFull);
        rowc[I] = ((uint32_t)f << 16) | (uint32_t)p;
        if constexpr (kBins > 0) atomicAdd(&above[f + p], 1);
        mx = max(mx, f + p);
        empty += 64 - __popcll(an);
        own += rc;
    }
    if (!sg.rowfmt) ents = 0;
    unsigned long long run = block_exclusive_scan(own, sh_u);  // prefix of row r_lo
    for (int I = r_lo; I < r_hi; ++I) {
        enc.full_row_ptr[I] = (int32_t)(run >> 32);
        enc.part_row_ptr[I] = (int32_t)(run & 0xFFFFFFFFull);
        {   // row summary: list starts and counts; columns past the row's
            // last tile are -1 (the placement writes the others)
            const int f = (int)(rowc[I] >> 16), p = (int)(rowc[I] & 0xFFFFu);
            int4 *ri = reinterpret_cast<int4 *>(enc.row_info + 16 * (size_t)I);
            ri[0] = make_int4((int)(run >> 32), f, (int)(run & 0xFFFFFFFFull), p);
            for (int k = f + p; k < 4; ++k) enc.row_info[16 * (size_t)I + 4 + k] = -1;
        }
        if (offsets) {
            unsigned long long r2 = run;
            for (int c = 0; c < C; ++c) {
                sg.off[I * C + c] = r2;
                r2 += sg.cnt[I * C + c];
            }
        }
        run += ((unsigned long long)(rowc[I] >> 16) << 32) |
               (unsigned long long)(rowc[I] & 0xFFFFu);
    }
    if (t == 255) {  // the last thread ends at the total
        enc.full_row_ptr[R] = (int32_t)(run >> 32);
        enc.part_row_ptr[R] = (int32_t)(run & 0xFFFFFFFFull);
        enc.stats[1] = (int64_t)(run >> 32);
        enc.stats[2] = (int64_t)(run & 0xFFFFFFFFull);
        sh_tot = run;
    }
    nnz = block_sum(nnz, sh_l);
    empty = block_sum(empty, sh_l);
    spw = block_sum(spw, sh_l);
    ents = block_sum(ents, sh_l);
    mx = block_max(mx, sh_i);
    const int nsp = (int)((uint64_t)spw >> kSpShift);
    const long long spnz = (long long)((uint64_t)spw & kSpLow);
    auto cnt_of = [&](int J) { return (int)((rowc[J] >> 16) + (rowc[J] & 0xFFFFu)); };
    if constexpr (kBins == 0) {  // (every row's count is in LDS: barriers above)
        // one key per row, count << 16 | (65535 - row) (row < kRows <= 65536):
        // a row's rank is the number of rows with a larger key (more tiles,
        // or as many and earlier), one unsigned compare per pair; the keys
        // replace the thread's own rows' counts, and are read four at a
        // time (broadcast LDS reads)
        for (int I = r_lo; I < r_hi; ++I)
            rowc[I] = ((uint32_t)cnt_of(I) << 16) | (0xFFFFu - (uint32_t)I);
        __syncthreads();
        const int R4 = R & ~3;
        for (int J = t; J < R; J += 256) {
            const uint32_t kj = rowc[J];
            int rank = 0;
#pragma unroll 4
            for (int J2 = 0; J2 < R4; J2 += 4) {
                const uint4 k4 = *reinterpret_cast<const uint4 *>(&rowc[J2]);
                rank += (int)(k4.x > kj) + (int)(k4.y > kj) + (int)(k4.z > kj) + (int)(k4.w > kj);
            }
            for (int J2 = R4; J2 < R; ++J2) rank += (int)(rowc[J2] > kj);
            enc.row_order[rank] = J;
        }
    } else {
        {   // histogram -> rows with a larger count: R - (rows with count <= c)
            const int per = (n + 1 + 255) / 256;
            const int c_lo = min(n + 1, t * per), c_hi = min(n + 1, c_lo + per);
            unsigned long long h = 0;
            for (int c = c_lo; c < c_hi; ++c) h += (unsigned long long)above[c];
            unsigned long long below = block_exclusive_scan(h, sh_u);
            for (int c = c_lo; c < c_hi; ++c) {
                below += (unsigned long long)above[c];
                above[c] = R - (int)below;
            }
        }
        __syncthreads();
        for (int k0 = 0; k0 < R; k0 += 256) {
            const int J = k0 + t;
            const int cj = J < R ? cnt_of(J) : 0;
            const int k1 = min(R, k0 + 256);
            int ties = 0;
#pragma unroll 8
            for (int J2 = k0; J2 < k1; ++J2)  // uniform length: loads pipeline
                ties += (J2 < J) && cnt_of(J2) == cj;
            if (J < R) enc.row_order[above[cj] + seen[cj] + ties] = J;
            __syncthreads();  // every rank of this block read seen[]
            if (J < R) atomicAdd(&seen[cj], 1);
            __syncthreads();
        }
    }
    if (t == 0) {
        enc.stats[0] = nnz;
        // rows past S do not exist
        enc.stats[3] = empty - (long long)G * (64LL * n - S);
        enc.stats[4] = mx;
        enc.stats[5] = nsp;
        enc.stats[6] = spnz;
        enc.stats[7] = ents;
    }
    // the statistics the kernel choice reads, in every row's summary (one
    // load per workgroup instead of a line that every workgroup waits on);
    // sh_tot was set before the reductions' barriers
    for (int I = t; I < R; I += 256) {
        int4 *ri = reinterpret_cast<int4 *>(enc.row_info + 16 * (size_t)I + 8);
        ri[0] = make_int4((int)(uint32_t)((unsigned long long)nnz & 0xFFFFFFFFull),
                          (int)(nnz >> 32), (int)(sh_tot >> 32),
                          (int)(sh_tot & 0xFFFFFFFFull));
        ri[1] = make_int4(mx, nsp, (int)(uint32_t)((uint64_t)ents & 0xFFFFFFFFull),
                          (int)(ents >> 32));
    }
}

// The scan of at most 64 rows (lane = row), in wavefront 0 alone: the
// outputs of scan_body without segment offsets, with wavefront shuffles
// in place of workgroup barriers (one memory round trip, then only stores).
__device__ void scan_small(int S, int n, int R, int G, SegPlan plan, Seg sg,
                           smh_mask_enc enc) {
    const int lane = threadIdx.x & 63;
    const int C = plan.per_row;
    unsigned long long rc = 0;
    long long nnz = 0, spw = 0, ents = 0;
    uint64_t an = 0;
    if (lane < R) {
#pragma unroll 8
        for (int c = 0; c < C; ++c) {  // independent loads: they pipeline
            rc += sg.cnt[lane * C + c];
            nnz += (long long)sg.nnz[lane * C + c];
            an |= sg.any[lane * C + c];
            spw += (long long)sg.sp[lane * C + c];
            const int4 e = reinterpret_cast<const int4 *>(sg.ecnt)[lane * C + c];
            ents += (long long)e.x + e.y + e.z + e.w;  // (as in scan_body)
        }
    }
    if (!sg.rowfmt) ents = 0;
    const int f = (int)(rc >> 32), p = (int)(rc & 0xFFFFFFFFull), cnt = f + p;
    unsigned long long incl = rc;  // inclusive prefix over rows
    for (int d = 1; d < 64; d <<= 1) {
        const unsigned long long y = __shfl_up(incl, d);
        if (lane >= d) incl += y;
    }
    const unsigned long long run = incl - rc, tot = __shfl(incl, 63);
    long long nz = nnz, empty = lane < R ? 64 - __popcll(an) : 0;
    int mx = lane < R ? cnt : 0;
    for (int o = 32; o > 0; o >>= 1) {
        nz += __shfl_xor(nz, o);
        empty += __shfl_xor(empty, o);
        spw += __shfl_xor(spw, o);
        ents += __shfl_xor(ents, o);
        mx = max(mx, __shfl_xor(mx, o));
    }
    const int nsp = (int)((uint64_t)spw >> kSpShift);
    const long long spnz = (long long)((uint64_t)spw & kSpLow);
    // schedule rank: rows with more stored tiles, then rows before with as
    // many; as in scan_body, on keys count << 16 | (65535 - row) in LDS
    // (lanes past R: key 0, never larger), read four at a time.  One
    // wavefront: its LDS write is done before its reads.
    __shared__ __attribute__((aligned(16))) uint32_t keys[64];
    const uint32_t key = lane < R ? ((uint32_t)cnt << 16) | (0xFFFFu - (uint32_t)lane) : 0u;
    keys[lane] = key;
    int rank = 0;
#pragma unroll
    for (int J2 = 0; J2 < 64; J2 += 4) {
        const uint4 k4 = *reinterpret_cast<const uint4 *>(&keys[J2]);
        rank += (int)(k4.x > key) + (int)(k4.y > key) + (int)(k4.z > key) + (int)(k4.w > key);
    }
    if (lane < R) {
        enc.full_row_ptr[lane] = (int32_t)(run >> 32);
        enc.part_row_ptr[lane] = (int32_t)(run & 0xFFFFFFFFull);
        int4 *ri = reinterpret_cast<int4 *>(enc.row_info + 16 * (size_t)lane);
        ri[0] = make_int4((int)(run >> 32), f, (int)(run & 0xFFFFFFFFull), p);
        for (int k = cnt; k < 4; ++k) enc.row_info[16 * (size_t)lane + 4 + k] = -1;
        ri[2] = make_int4((int)(uint32_t)((unsigned long long)nz & 0xFFFFFFFFull),
                          (int)(nz >> 32), (int)(tot >> 32), (int)(tot & 0xFFFFFFFFull));
        ri[3] = make_int4(mx, nsp, (int)(uint32_t)((uint64_t)ents & 0xFFFFFFFFull),
                          (int)(ents >> 32));
        enc.row_order[rank] = lane;
    }
    if (lane == 0) {
        enc.full_row_ptr[R] = (int32_t)(tot >> 32);
        enc.part_row_ptr[R] = (int32_t)(tot & 0xFFFFFFFFull);
        enc.stats[0] = nz;
        enc.stats[1] = (int64_t)(tot >> 32);
        enc.stats[2] = (int64_t)(tot & 0xFFFFFFFFull);
        enc.stats[3] = empty - (long long)G * (64LL * n - S);  // rows past S do not exist
        enc.stats[4] = mx;
        enc.stats[5] = nsp;
        enc.stats[6] = spnz;
        enc.stats[7] = ents;
    }
}

__global__ __launch_bounds__(256) void enc_scan(int S, int n, int R, int G,
                                                SegPlan plan, Seg sg,
                                                smh_mask_enc enc) {
    scan_body<kScanRows, kScanBins>(S, n, R, G, plan, sg, enc, true);
}

// The row-wise entries of a segment's sparse partial tiles, written at
// their final places: group q's entries of the segment start at
// ent_dst[q] (after the row's earlier segments' entries, in the row's region
// for group q); within it, tiles in column order, then key.  Wavefront q
// writes group q: per sparse tile, lane k takes key 64J + k, its rows among
// the group's 16 (bit k % 8 of each byte of the two inner-tile words of
// column block k / 8), and a ballot over the lanes gives each live key its
// rank, so a tile's entries are one run of contiguous stores.  Lane t < 64
// of the workgroup brings partial tile t's column and valid-element count;
// words: the segment's partial-tile words (64 per tile, in list order, in
// LDS).
__device__ void place_entries(int np, int colp, int popp, const uint64_t *words,
                              uint32_t *__restrict__ row_ent, const size_t *ent_dst) {
    __shared__ int col_t[kMaxSegTiles];  // column of a sparse tile, -1 otherwise
    const int t = threadIdx.x, q = t >> 6, lane = t & 63;
    if (t < kMaxSegTiles)
        col_t[t] = t < np && popp <= SMH_SPARSE_TILE_MAX ? colp : -1;
    __syncthreads();  // also: ent_dst from wavefront 0, the words
    uint32_t *dst = row_ent + ent_dst[q];
    const int jc = lane >> 3, c = lane & 7;
    // lane l holds tile l's column; the sparse tiles are the set bits of
    // `sp`, visited in order with the next one's words read (LDS) before
    // the current one is placed
    const int myJ = lane < np ? col_t[lane] : -1;
    uint64_t sp = __builtin_amdgcn_ballot_w64(myJ >= 0);
    if (sp == 0) return;
    int l = __builtin_ctzll(sp);
    uint64_t wa = words[64 * (size_t)l + 16 * q + jc];
    uint64_t wb = words[64 * (size_t)l + 16 * q + 8 + jc];
    while (sp) {
        const int J = __builtin_amdgcn_readlane(myJ, l);
        sp &= sp - 1;
        const int ln = sp ? __builtin_ctzll(sp) : l;
        const uint64_t na = words[64 * (size_t)ln + 16 * q + jc];
        const uint64_t nb = words[64 * (size_t)ln + 16 * q + 8 + jc];
        const uint32_t rows = column_rows(wa, c) | (column_rows(wb, c) << 8);
        const uint64_t live = __builtin_amdgcn_ballot_w64(rows != 0);
        const int rank = (int)__builtin_amdgcn_mbcnt_hi(
            (uint32_t)(live >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)live, 0u));
        if (rows) dst[rank] = (rows << 16) | (64u * (uint32_t)J + (uint32_t)lane);
        dst += __popcll(live);
        wa = na;
        wb = nb;
        l = ln;
    }
}

// Placement of a segment.  kSelf: workgroup 0 runs the scan (first, so that
// it is dispatched with the first placements instead of after them) and
// workgroup s + 1 places segment s, adding up the tile counts of the
// segments before it.  Otherwise workgroup s places segment s with the
// offsets from enc_scan.  (Taking segments from both ends in turn, so that
// the heavy last rows of a causal mask start early, measured slower on the
// 16k mask: 79.6 against 76.9 us.)  The segment's own columns and
// first words are loaded together with its offsets (they do not depend on
// them), so a small segment is placed after one memory round trip.
template <bool kSelf>
__global__ __launch_bounds__(256) void enc_place(int S, int n, int R, int G,
                                                 SegPlan plan, Seg sg,
                                                 smh_mask_enc enc) {
    __shared__ unsigned long long sh_u[4];
    __shared__ size_t ent_dst[4];  // where the segment's entries of group g go
    const int t = threadIdx.x, s = (int)blockIdx.x - (kSelf ? 1 : 0);
    if constexpr (kSelf) {
        if (s < 0) {
            if (R <= 64) {
                if (threadIdx.x < 64) scan_small(S, n, R, G, plan, sg, enc);
            } else {
                scan_body<kFusedRows, kFusedBins>(S, n, R, G, plan, sg, enc, false);
            }
            return;
        }
    }
    const size_t base = (size_t)s * sg.cap;
    const uint64_t cnt = sg.cnt[s];
    // the segment's place in its row (wavefront 0, lane = segment of the
    // row; per_row <= 64): tiles of the row's segments before it, and the
    // row's full tiles in all, so that the row's first four stored tiles
    // can go to its row_info
    const int row = s / plan.per_row, s0 = row * plan.per_row;
    const uint64_t rcnt = t < plan.per_row ? sg.cnt[s0 + t] : 0;
    // row-wise entries of the row's segments per group (lane = segment)
    const int4 recnt = sg.rowfmt && t < plan.per_row
                           ? reinterpret_cast<const int4 *>(sg.ecnt)[s0 + t]
                           : make_int4(0, 0, 0, 0);
    // columns (t < cap) and the first 256 16-byte chunks of the words
    const int colf = t < sg.cap ? sg.fcol[base + t] : 0;
    const int colp = t < sg.cap ? sg.pcol[base + t] : 0;
    const int popp = t < sg.cap ? sg.pop[base + t] : 0;
    const int4 ecs = sg.rowfmt ? reinterpret_cast<const int4 *>(sg.ecnt)[s] : make_int4(0, 0, 0, 0);
    const bool has_ent = (ecs.x | ecs.y | ecs.z | ecs.w) != 0;
    const u4v *src = reinterpret_cast<const u4v *>(sg.words + base * 64);
    const u4v w0 = t < sg.cap * 32 ? src[t] : u4v{0, 0, 0, 0};
    unsigned long long off;
    if (kSelf) {
        // s < kFusedMaxSegs: a fixed number of predicated loads, all issued
        // before the first is waited for (a loop to s waited for each in
        // turn: up to 8 memory round trips for the last segments)
        uint64_t part[kFusedMaxSegs / 256];
#pragma unroll
        for (int k = 0; k < kFusedMaxSegs / 256; ++k) {
            const int j = t + 256 * k;
            part[k] = j < s ? sg.cnt[j] : 0;
        }
        unsigned long long x = 0;
#pragma unroll
        for (int k = 0; k < kFusedMaxSegs / 256; ++k) x += part[k];
        off = block_sum(x, sh_u);
    } else {
        off = sg.off[s];
    }
    const int pf = (int)(off >> 32), pp = (int)(off & 0xFFFFFFFFull);
    const int nf = (int)(cnt >> 32), np = (int)(cnt & 0xFFFFFFFFull);
    if (t < 64) {  // a segment holds at most 64 tiles: wavefront 0 places them
        const bool before = s0 + t < s;
        int bf = before ? (int)(rcnt >> 32) : 0;
        int bp = before ? (int)(rcnt & 0xFFFFFFFFull) : 0;
        int rf = (int)(rcnt >> 32);
        for (int o = 32; o > 0; o >>= 1) {
            bf += __shfl_xor(bf, o);
            bp += __shfl_xor(bp, o);
            rf += __shfl_xor(rf, o);
        }
        if (sg.rowfmt) {
            // the segment's entries go after those of the row's earlier
            // segments, in the row's region of group q; the row's first
            // segment writes the row's counts
            int rp = (int)(rcnt & 0xFFFFFFFFull);  // the row's partial tiles
            int e[4] = {recnt.x, recnt.y, recnt.z, recnt.w}, be[4], re[4];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                be[g] = before ? e[g] : 0;
                re[g] = e[g];
            }
            for (int o = 32; o > 0; o >>= 1) {
                rp += __shfl_xor(rp, o);
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    be[g] += __shfl_xor(be[g], o);
                    re[g] += __shfl_xor(re[g], o);
                }
            }
            if (t < 4) {
                const size_t p0 = (size_t)(pp - bp);
                if (has_ent)
                    ent_dst[t] = 256 * p0 + 64 * (size_t)t * rp +
                                 (size_t)(t == 0 ? be[0] : t == 1 ? be[1] : t == 2 ? be[2] : be[3]);
                if (s == s0)
                    enc.row_ent_cnt[4 * (size_t)row + t] =
                        t == 0 ? re[0] : t == 1 ? re[1] : t == 2 ? re[2] : re[3];
            }
        }
        else if (s == s0 && t < 4) {
            enc.row_ent_cnt[4 * (size_t)row + t] = 0;  // no row-wise format
        }
        int32_t *ri = enc.row_info + 16 * (size_t)row + 4;
        if (t < nf) {
            enc.full_col_idx[pf + t] = colf;
            if (bf + t < 4) ri[bf + t] = colf;
        }
        if (t < np) {
            enc.part_col_idx[pp + t] = colp;
            enc.part_pop[pp + t] = popp;
            if (rf + bp + t < 4) ri[rf + bp + t] = colp;
        }
    }
    u4v *dst = reinterpret_cast<u4v *>(enc.part_bitmaps + (size_t)pp * 64);
    // with row-wise entries to write, the words also go to LDS (dynamic, cap
    // tiles of room), where place_entries reads them
    extern __shared__ u4v wl[];
    if (t < np * 32) {
        dst[t] = w0;
        if (has_ent) wl[t] = w0;
    }
    // the rest of the words (np <= kMaxSegTiles): every load issued before
    // the first store, which waits for them once (a load-store loop waited
    // a memory round trip per 256 chunks)
    // (unconditional loads: lanes past the words read chunk 0, one cache
    // line for the whole workgroup; a predicated load became a branch with
    // its own wait)
    constexpr int kRest = kMaxSegTiles * 32 / 256 - 1;
    u4v rest[kRest];
#pragma unroll
    for (int k = 0; k < kRest; ++k) {
        const int e = t + 256 * (k + 1);
        rest[k] = src[e < np * 32 ? e : 0];
    }
#pragma unroll
    for (int k = 0; k < kRest; ++k) {
        const int e = t + 256 * (k + 1);
        if (e < np * 32) {
            dst[e] = rest[k];
            if (has_ent) wl[e] = rest[k];
        }
    }
    if (has_ent)
        place_entries(np, colp, popp, reinterpret_cast<const uint64_t *>(wl), enc.row_ent, ent_dst);
}

// S == 0: an empty encoding.  Row pointers {0}, all statistics zero.
__global__ void enc_empty(smh_mask_enc enc) {
    if (threadIdx.x == 0) {
        enc.full_row_ptr[0] = 0;
        enc.part_row_ptr[0] = 0;
    }
    if (threadIdx.x < 8) enc.stats[threadIdx.x] = 0;
}

}  // namespace

namespace {

// The launches of an encode: strip pass (`strip` enqueues it on the
// segments), then the scan and placement.
template <typename StripLaunch>
hipError_t encode_launches(StripLaunch strip, int32_t S, const EncLayout &L,
                           const smh_mask_enc &enc, char *scratch,
                           hipStream_t stream) {
    if (S == 0) {
        hipLaunchKernelGGL(enc_empty, dim3(1), dim3(64), 0, stream, enc);
        return hipGetLastError();
    }
    const int n = (int)L.n, R = (int)L.rows;
    const int G = enc.mask_b * enc.mask_h;
    const SegPlan plan = L.plan;
    if (plan.total <= 0 || plan.win > kMaxSegWin || plan.per_row > 64 ||
        n > kMaxN || R > kScanRows || (int64_t)G * n != L.rows)
        return hipErrorInvalidValue;
    Seg sg;  // the scratch arrays keep their workspace offsets past seg_cnt
    char *sc = scratch - L.seg_cnt;
    sg.cnt = (uint64_t *)(sc + L.seg_cnt);
    sg.off = (uint64_t *)(sc + L.seg_off);
    sg.nnz = (uint64_t *)(sc + L.seg_nnz);
    sg.any = (uint64_t *)(sc + L.seg_any);
    sg.sp = (uint64_t *)(sc + L.seg_sp);
    sg.fcol = (int32_t *)(sc + L.seg_fcol);
    sg.pcol = (int32_t *)(sc + L.seg_pcol);
    sg.pop = (int32_t *)(sc + L.seg_pop);
    sg.ecnt = (int32_t *)(sc + L.seg_ecnt);
    sg.rowfmt = L.rowfmt ? 1 : 0;
    sg.words = (uint64_t *)(sc + L.seg_words);
    sg.cap = (int)L.seg_cap;
    strip(n, plan, sg);
    // placement's LDS for the segment's words (place_entries)
    const size_t wl_bytes = L.rowfmt ? sizeof(uint64_t) * 64 * L.seg_cap : 0;
    if (plan.total <= kFusedMaxSegs && R <= kFusedRows) {
        hipLaunchKernelGGL(enc_place<true>, dim3(plan.total + 1), dim3(256), wl_bytes,
                           stream, S, n, R, G, plan, sg, enc);
    } else {
        hipLaunchKernelGGL(enc_scan, dim3(1), dim3(256), 0, stream, S, n, R, G,
                           plan, sg, enc);
        hipLaunchKernelGGL(enc_place<false>, dim3(plan.total), dim3(256), wl_bytes,
                           stream, S, n, R, G, plan, sg, enc);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_encode(const uint8_t *mask, int32_t S, const EncLayout &L,
                         const smh_mask_enc &enc, char *scratch,
                         hipStream_t stream) {
    auto strip = [&](int n, SegPlan plan, Seg sg) {
        if (S % 64 == 0)
            hipLaunchKernelGGL(enc_strip<kAligned64>, dim3(plan.total), dim3(256),
                               0, stream, mask, S, n, plan, sg);
        else if (S % 16 == 0)
            hipLaunchKernelGGL(enc_strip<kAligned16>, dim3(plan.total), dim3(256),
                               0, stream, mask, S, n, plan, sg);
        else
            hipLaunchKernelGGL(enc_strip<kDwords>, dim3(plan.total), dim3(256), 0,
                               stream, mask, S, n, plan, sg);
    };
    return encode_launches(strip, S, L, enc, scratch, stream);
}

hipError_t launch_encode_pattern(const smh_pattern &pat, int32_t S,
                                 const EncLayout &L, const smh_mask_enc &enc,
                                 char *scratch, hipStream_t stream) {
    Pattern p;
    p.causal = pat.causal != 0;
    p.window = pat.window;
    p.grow = pat.global_rows;
    p.gcol = pat.global_cols;
    p.blocks = pat.blocks;
    p.keep16 = (uint32_t)floorf(pat.block_keep * 65536.0f);
    p.rand16 = (uint32_t)floorf(pat.random_p * 65536.0f);
    p.seed = pat.seed;
    auto strip = [&](int n, SegPlan plan, Seg sg) {
        hipLaunchKernelGGL(enc_pattern_strip, dim3(plan.total), dim3(256), 0,
                           stream, p, S, n, plan, sg);
    };
    return encode_launches(strip, S, L, enc, scratch, stream);
}

// The encoder scratch of smh_encode_masks_noalloc: a fixed array in the
// code object, one copy per device, for callers that cannot allocate.  In
// host code `scratch` names a host-side stand-in, never the device memory:
// kernels and copies get the address static_scratch() looked up.
constexpr int kMaxDevices = 64;
static __device__ __align__(256) char scratch[SMH_STATIC_SCRATCH_BYTES];

hipError_t static_scratch(char **ptr) {
    static std::mutex mu;
    static char *addr[kMaxDevices];
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p || (reinterpret_cast<uintptr_t>(p) & 255)) return hipErrorInvalidValue;
        addr[dev] = static_cast<char *>(p);
    }
    *ptr = addr[dev];
    return hipSuccess;
}

}  // namespace smh
