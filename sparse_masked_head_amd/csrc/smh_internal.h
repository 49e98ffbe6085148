// Internal declarations shared by the HIP translation units of libsmh.
// Nothing here is part of the public interface (include/smh.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "smh.h"

namespace smh {

// Byte offsets of every array inside the encode workspace.  Each array
// starts on a 256-byte boundary.  The first block is the encoding proper,
// the second block is scratch used only while encoding.
struct EncLayout {
    int64_t n;  // outer tiles per side
    size_t full_row_ptr, part_row_ptr, full_col_idx, part_col_idx,
        part_bitmaps, stats, row_order;
    size_t row_nf, row_np, row_empty, row_nnz, full_local, part_local,
        tile_words;
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
    L.full_row_ptr = take(sizeof(int32_t) * (n + 1));
    L.part_row_ptr = take(sizeof(int32_t) * (n + 1));
    L.full_col_idx = take(sizeof(int32_t) * n2);
    L.part_col_idx = take(sizeof(int32_t) * n2);
    L.part_bitmaps = take(sizeof(uint64_t) * 64 * n2);
    L.stats = take(sizeof(int64_t) * 8);
    L.row_order = take(sizeof(int32_t) * n);
    L.row_nf = take(sizeof(int32_t) * n);
    L.row_np = take(sizeof(int32_t) * n);
    L.row_empty = take(sizeof(int32_t) * n);
    L.row_nnz = take(sizeof(int64_t) * n);
    L.full_local = take(sizeof(int32_t) * n2);
    L.part_local = take(sizeof(int32_t) * n2);
    L.tile_words = take(sizeof(uint64_t) * 64 * n2);
    L.total = off;
    return L;
}

// Encoder: two launches on `stream` (row strips, then placement).
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
