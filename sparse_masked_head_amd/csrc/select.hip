// Host entry of the kernel-choice cost model (select_model.h).
#include "select_model.h"
#include "smh_internal.h"

namespace smh {

smh_kernel select_kernel(const smh_mask_stats &st, int64_t heads, int d,
                         int dtype, double *t_row_us, double *t_blk_us) {
    SelectInput in;
    in.nnz = st.nnz;
    in.n_full = st.n_full;
    in.n_sparse = st.n_sparse;
    in.entries = st.row_entries;
    in.n_partial = st.n_partial;
    in.max_row_tiles = st.max_row_tiles;
    in.heads = heads;
    in.rows = (int64_t)st.mask_b * st.mask_h * ((st.S + 63) / 64);
    in.d = d;
    in.bf16 = dtype == SMH_BF16;
    double tr, tb;
    select_costs_us(in, &tr, &tb);
    if (t_row_us) *t_row_us = tr;
    if (t_blk_us) *t_blk_us = tb;
    return select_model(in) == 1 ? SMH_ROWWISE : SMH_BLOCKWISE;
}

}  // namespace smh
