/* Scalar reference encoder for the two-level mask format.
 *
 * TEST INFRASTRUCTURE ONLY: called from the tests and the benchmark's CPU
 * baseline through ctypes; never linked into the product library and shares
 * no header or code with it.
 *
 * Format ("Accelerating Sparse Transformer Inference on GPU", gist.science
 * explainer, Technical summary > Methodology > 1. Unified MHA module, the
 * storage-format items):
 *   - the S x S mask is cut into 64 x 64 outer tiles (OT);
 *   - an OT with no valid element is not stored at all (it is skipped);
 *   - an OT whose 4096 elements are all valid is "full": only its column
 *     index is listed, BSR style, under full_row_ptr / full_col_idx;
 *   - any other OT is "partial": its column index is listed under
 *     part_row_ptr / part_col_idx and its contents are stored as 64 inner
 *     tiles (IT) of 8 x 8 elements, one uint64 bitmap each.
 * Readings where the pages are silent (64 x 64 OT size, bit 8r+c of an IT
 * for local row r / column c, ITs of an OT in row-major order, column indices
 * ascending within a row, CSR-style int32 row pointers) are listed with the
 * design notes of the repository.
 *
 * The loops below visit the outer tiles row by row in ascending column
 * order and append, which is the definition of the lists.
 *
 * S need not be a multiple of 64: the tiles cover ceil(S/64) * 64 rows and
 * columns, and an element outside the S x S mask is not valid (reading of
 * the pages' "arbitrary mask" for ragged lengths).
 */
#include <stdint.h>
#include <string.h>

/* Element (row, col) of the mask, 0 outside the S x S matrix. */
static int valid(const uint8_t *mask, int64_t S, int64_t row, int64_t col)
{
    return row < S && col < S && mask[row * S + col] != 0;
}

/* Returns 0 on success, -1 if S is not positive.  n_ot = ceil(S / 64).
 * Output capacities: row_ptr arrays n_ot+1, col_idx arrays n_ot*n_ot,
 * bitmaps n_ot*n_ot*64.  stats[0]=nnz, [1]=n_full, [2]=n_partial,
 * [3]=number of query rows (of the S) with no valid key. */
int ref_encode(const uint8_t *mask, int64_t S,
               int32_t *full_row_ptr, int32_t *full_col_idx,
               int32_t *part_row_ptr, int32_t *part_col_idx,
               uint64_t *part_bitmaps, int64_t *stats)
{
    if (S <= 0) return -1;
    const int64_t n_ot = (S + 63) / 64;
    int64_t nnz = 0;
    int32_t n_full = 0, n_part = 0;

    full_row_ptr[0] = 0;
    part_row_ptr[0] = 0;
    for (int64_t I = 0; I < n_ot; ++I) {
        for (int64_t J = 0; J < n_ot; ++J) {
            /* count the valid elements of outer tile (I, J) */
            int64_t cnt = 0;
            for (int64_t r = 0; r < 64; ++r)
                for (int64_t c = 0; c < 64; ++c)
                    cnt += valid(mask, S, 64 * I + r, 64 * J + c);
            nnz += cnt;
            if (cnt == 0) continue;                 /* skipped tile */
            if (cnt == 64 * 64) {                   /* full tile */
                full_col_idx[n_full++] = (int32_t)J;
                continue;
            }
            /* partial tile: 64 inner-tile bitmaps, inner tile (ir, ic)
             * at position ir*8+ic, element (r, c) of it at bit r*8+c */
            uint64_t *bm = part_bitmaps + (int64_t)n_part * 64;
            for (int ir = 0; ir < 8; ++ir)
                for (int ic = 0; ic < 8; ++ic) {
                    uint64_t word = 0;
                    for (int r = 0; r < 8; ++r)
                        for (int c = 0; c < 8; ++c) {
                            int64_t row = 64 * I + 8 * ir + r;
                            int64_t col = 64 * J + 8 * ic + c;
                            if (valid(mask, S, row, col))
                                word |= (uint64_t)1 << (r * 8 + c);
                        }
                    bm[ir * 8 + ic] = word;
                }
            part_col_idx[n_part++] = (int32_t)J;
        }
        full_row_ptr[I + 1] = n_full;
        part_row_ptr[I + 1] = n_part;
    }

    int64_t empty_rows = 0;
    for (int64_t i = 0; i < S; ++i) {
        int any = 0;
        for (int64_t j = 0; j < S && !any; ++j) any = mask[i * S + j] != 0;
        empty_rows += !any;
    }
    stats[0] = nnz;
    stats[1] = n_full;
    stats[2] = n_part;
    stats[3] = empty_rows;
    return 0;
}
