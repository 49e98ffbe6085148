// Internal declarations shared by the HIP translation units of libsmh.
// Nothing here is part of the public interface (include/smh.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "smh.h"

namespace smh {

// The encoder's unit of work: a segment = up to kMaxSegWin windows of kWin
// outer tiles of one outer-tile row.  Each of the `rows` rows (G masks of
// n outer-tile rows each, mask after mask) is cut into `per_row` segments
// of `win` windows (the last one possibly shorter), enough segments in all
// to keep the chip busy; `total` = rows * per_row.  Segments are numbered
// row by row, left to right.
constexpr int kWin = 8;         // outer tiles per window (512 mask columns)
constexpr int kMaxSegWin = 8;   // windows per segment
struct SegPlan {
    int per_row, win, total;
};
inline SegPlan seg_plan(int rows, int n) {
    SegPlan p{0, 0, 0};
    if (rows <= 0 || n <= 0) return p;
    const int nw = (n + kWin - 1) / kWin;  // windows per row
    // aim at >= 2048 segments: about twice the workgroups that fit on the
    // chip at once, so that later ones stream the mask while earlier ones
    // classify and write (16k mask: 97 us against 107 us with 1024)
    int c = (2048 + rows - 1) / rows;
    c = c < nw ? c : nw;
    const int cmin = (nw + kMaxSegWin - 1) / kMaxSegWin;
    c = c > cmin ? c : cmin;
    p.win = (nw + c - 1) / c;
    p.per_row = (nw + p.win - 1) / p.win;
    p.total = rows * p.per_row;
    return p;
}

// Byte offsets of every array inside the encode workspace of G masks of
// S x S.  Each array starts on a 256-byte boundary: the encoding proper
// (rows = G * n outer-tile rows), then per-segment scratch written by the
// strip pass and read by the placement pass.
struct EncLayout {
    int64_t n;     // outer tiles per side of one mask
    int64_t rows;  // outer-tile rows of the stack (G * n)
    SegPlan plan;
    size_t full_row_ptr, part_row_ptr, full_col_idx, part_col_idx,
        part_bitmaps, stats, row_order, row_info, part_pop, row_ent, row_ent_cnt;
    bool rowfmt;   // the row-wise format of sparse tiles is built (S <= 65536)
    // per segment: tile counts (full << 32 | partial), exclusive offsets
    // (same packing), valid pairs, covered query rows (bit 8k + r = strip
    // row 8k + r), sparse partial tiles (count << 40 | their valid pairs),
    // and its tiles' columns, partial-tile populations and words (room for
    // seg_cap tiles each)
    size_t seg_cnt, seg_off, seg_nnz, seg_any, seg_sp, seg_fcol, seg_pcol,
        seg_pop, seg_words;
    // per segment and 16-row group: row-wise entries of its sparse tiles
    // (count, then room for 64 per tile)
    size_t seg_ecnt;
    size_t seg_cap;
    size_t total;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Longest sequence whose row-wise entries (16-bit keys) are built.
constexpr int kRowFmtMaxS = 65536;

// Caller guarantees 0 <= S <= SMH_MAX_S, G >= 1 and G * n <= SMH_MAX_ENC_ROWS.
inline EncLayout enc_layout(int32_t S, int64_t G) {
    EncLayout L{};
    const int64_t n = ((int64_t)S + 63) / 64;  // ragged S: the last tiles are cut
    const int64_t rows = G * n;
    const size_t cap = size_t(rows) * size_t(n);  // tiles of the stack
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t at = off;
        off = align256(off + (bytes ? bytes : 1));
        return at;
    };
    L.n = n;
    L.rows = rows;
    L.plan = seg_plan((int)rows, (int)n);
    L.full_row_ptr = take(sizeof(int32_t) * (rows + 1));
    L.part_row_ptr = take(sizeof(int32_t) * (rows + 1));
    L.full_col_idx = take(sizeof(int32_t) * cap);
    L.part_col_idx = take(sizeof(int32_t) * cap);
    L.part_bitmaps = take(sizeof(uint64_t) * 64 * cap);
    L.stats = take(sizeof(int64_t) * 8);  // nnz, n_full, n_partial, empty rows, max row tiles, n_sparse, sparse_nnz
    L.row_order = take(sizeof(int32_t) * rows);
    L.row_info = take(sizeof(int32_t) * 16 * rows);
    L.part_pop = take(sizeof(int32_t) * cap);
    L.rowfmt = S <= kRowFmtMaxS;
    L.row_ent = take(L.rowfmt ? sizeof(uint32_t) * 256 * cap : 0);
    L.row_ent_cnt = take(sizeof(int32_t) * 4 * rows);
    const size_t T = (size_t)L.plan.total;
    L.seg_cap = (size_t)L.plan.win * kWin;
    L.seg_cnt = take(sizeof(uint64_t) * T);
    L.seg_off = take(sizeof(uint64_t) * T);
    L.seg_nnz = take(sizeof(uint64_t) * T);
    L.seg_any = take(sizeof(uint64_t) * T);
    L.seg_sp = take(sizeof(uint64_t) * T);
    L.seg_fcol = take(sizeof(int32_t) * T * L.seg_cap);
    L.seg_pcol = take(sizeof(int32_t) * T * L.seg_cap);
    L.seg_pop = take(sizeof(int32_t) * T * L.seg_cap);
    L.seg_words = take(sizeof(uint64_t) * 64 * T * L.seg_cap);
    L.seg_ecnt = take(sizeof(int32_t) * 4 * T);
    L.total = off;
    return L;
}

// The encoding proper is the workspace's first enc_output_bytes; the
// encoder's scratch (the per-segment arrays, from seg_cnt on) follows.
inline size_t enc_output_bytes(const EncLayout &L) { return L.seg_cnt; }
inline size_t enc_scratch_bytes(const EncLayout &L) { return L.total - L.seg_cnt; }

// Encoder of a stack of G = enc.mask_b * enc.mask_h masks [G][S][S]: two or
// three launches on `stream` (strip pass, [scan,] placement).  The encoding
// goes where `enc` points; `scratch` (enc_scratch_bytes(L) bytes, 256-byte
// aligned, no preparation needed) holds the per-segment arrays.
hipError_t launch_encode(const uint8_t *mask, int32_t S, const EncLayout &L,
                         const smh_mask_enc &enc, char *scratch,
                         hipStream_t stream);

// Encoder of the mask a pattern describes (one mask, enc.mask_b = mask_h =
// 1): the pattern strip pass, then the same scan and placement.
hipError_t launch_encode_pattern(const smh_pattern &pat, int32_t S,
                                 const EncLayout &L, const smh_mask_enc &enc,
                                 char *scratch, hipStream_t stream);

// Device address of the library's static encoder scratch on the current
// device (SMH_STATIC_SCRATCH_BYTES bytes; looked up once per device).
hipError_t static_scratch(char **ptr);

// Block-wise kernel launcher.  in_dt: 0 f16, 1 bf16; out_dt: 0/1/2 (f32).
// hybrid: sparse partial tiles (at most SMH_SPARSE_TILE_MAX valid elements)
// go to the gather path where the mask allows (hybrid_allowed).
hipError_t launch_blockwise(const void *q, const void *k, const void *v,
                            void *o, int B, int H, int S, int d, int in_dt,
                            int out_dt, float scale, const smh_mask_enc &enc,
                            int hybrid, hipStream_t stream);

// The gather path reads the row-wise entries (built for S <= 65536) and
// splits rows in an LDS list of at most 1024 partial tiles.
inline bool hybrid_allowed(int S, int n_ot) { return S <= kRowFmtMaxS && n_ot <= 1024; }

// Row-wise kernel launcher, same conventions.
hipError_t launch_rowwise(const void *q, const void *k, const void *v,
                          void *o, int B, int H, int S, int d, int in_dt,
                          int out_dt, float scale, const smh_mask_enc &enc,
                          hipStream_t stream);

// Fused launcher: the cost model runs on the device on the statistics the
// encoder wrote, then every workgroup runs the chosen algorithm.
hipError_t launch_auto(const void *q, const void *k, const void *v, void *o,
                       int B, int H, int S, int d, int in_dt, int out_dt,
                       float scale, const smh_mask_enc &enc,
                       hipStream_t stream);

// Output projection with bias and residual (dt: SMH_F16 or SMH_BF16).
hipError_t launch_out_proj(const void *o, const void *w, const void *bias,
                           const void *res, void *out, int B, int H, int S,
                           int d, int D, int dt, hipStream_t stream);

// Cost model of the selector (host only).  heads = (batch, head) pairs per
// mask of the stack.
smh_kernel select_kernel(const smh_mask_stats &st, int64_t heads, int d,
                         int dtype, double *t_row_us, double *t_blk_us);

}  // namespace smh
