// Internal declarations shared by the HIP translation units of libsmh.
// Nothing here is part of the public interface (include/smh.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "smh.h"

namespace smh {

// The encoder's unit of work: a segment = up to kMaxSegWin windows of kWin
// outer tiles of one outer-tile row.  Each row is cut into `per_row`
// segments of `win` windows (the last one possibly shorter), enough
// segments in all to keep the chip busy; `total` = n * per_row.  Segments
// are numbered row by row, left to right.
constexpr int kWin = 8;         // outer tiles per window (512 mask columns)
constexpr int kMaxSegWin = 8;   // windows per segment
struct SegPlan {
    int per_row, win, total;
};
inline SegPlan seg_plan(int n) {
    SegPlan p{0, 0, 0};
    if (n <= 0) return p;
    const int nw = (n + kWin - 1) / kWin;  // windows per row
    int c = (1024 + n - 1) / n;           // aim at >= 1024 segments
    c = c < nw ? c : nw;
    const int cmin = (nw + kMaxSegWin - 1) / kMaxSegWin;
    c = c > cmin ? c : cmin;
    p.win = (nw + c - 1) / c;
    p.per_row = (nw + p.win - 1) / p.win;
    p.total = n * p.per_row;
    return p;
}

// Byte offsets of every array inside the encode workspace.  Each array
// starts on a 256-byte boundary: the encoding proper, then per-segment
// scratch written by the strip pass and read by the placement pass.
struct EncLayout {
    int64_t n;  // outer tiles per side
    SegPlan plan;
    size_t full_row_ptr, part_row_ptr, full_col_idx, part_col_idx,
        part_bitmaps, stats, row_order;
    // per segment: tile counts (full << 32 | partial), exclusive offsets
    // (same packing), valid pairs, covered query rows (bit 8k + r = strip
    // row 8k + r), and its tiles' columns and partial-tile words (room for
    // seg_cap tiles each)
    size_t seg_cnt, seg_off, seg_nnz, seg_any, seg_fcol, seg_pcol, seg_words;
    size_t seg_cap;
    size_t total;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

inline EncLayout enc_layout(int32_t S) {
    EncLayout L{};
    const int64_t n = S / 64;
    const size_t n2 = size_t(n) * size_t(n);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t at = off;
        off = align256(off + (bytes ? bytes : 1));
        return at;
    };
    L.n = n;
    L.plan = seg_plan((int)n);
    L.full_row_ptr = take(sizeof(int32_t) * (n + 1));
    L.part_row_ptr = take(sizeof(int32_t) * (n + 1));
    L.full_col_idx = take(sizeof(int32_t) * n2);
    L.part_col_idx = take(sizeof(int32_t) * n2);
    L.part_bitmaps = take(sizeof(uint64_t) * 64 * n2);
    L.stats = take(sizeof(int64_t) * 8);  // nnz, n_full, n_partial, empty rows, max row tiles
    L.row_order = take(sizeof(int32_t) * n);
    const size_t T = (size_t)L.plan.total;
    L.seg_cap = (size_t)L.plan.win * kWin;
    L.seg_cnt = take(sizeof(uint64_t) * T);
    L.seg_off = take(sizeof(uint64_t) * T);
    L.seg_nnz = take(sizeof(uint64_t) * T);
    L.seg_any = take(sizeof(uint64_t) * T);
    L.seg_fcol = take(sizeof(int32_t) * T * L.seg_cap);
    L.seg_pcol = take(sizeof(int32_t) * T * L.seg_cap);
    L.seg_words = take(sizeof(uint64_t) * 64 * T * L.seg_cap);
    L.total = off;
    return L;
}

// Encoder: two or three launches on `stream` (strip pass, [scan,]
// placement).
hipError_t launch_encode(const uint8_t *mask, int32_t S, char *ws,
                         const EncLayout &L, const smh_mask_enc &enc,
                         hipStream_t stream);

// Block-wise kernel launcher.  in_dt: 0 f16, 1 bf16; out_dt: 0/1/2 (f32).
hipError_t launch_blockwise(const void *q, const void *k, const void *v,
                            void *o, int B, int H, int S, int d, int in_dt,
                            int out_dt, float scale, const smh_mask_enc &enc,
                            hipStream_t stream);

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

// Cost model of the selector (host only).
smh_kernel select_kernel(const smh_mask_stats &st, int64_t BH, int d,
                         int dtype, double *t_row_us, double *t_blk_us);

}  // namespace smh
