// Analytical choice between the row-wise and the block-wise kernel.
//
// The pages state that an analytical model picks the kernel from the mask's
// sparsity and the sequence length ("Accelerating Sparse Transformer
// Inference on GPU", gist.science explainer, Technical summary >
// Methodology > 1. Unified MHA module, kernel-selection item; arXiv
// catalogue record, abstract) but give no formula.  This model predicts
// the time of each kernel from the encoding statistics and the problem
// shape and returns the cheaper one.
//
//   block-wise: one workgroup per (head, outer-tile row), 64 x 64 x d tile
//     per step.  Work = stored tiles * heads; partial tiles add a masking
//     cost.  A launch whose workgroups fit in one wave of the chip runs for
//     the length of its heaviest row instead, so
//       T_blk = c0 + max(W_blk / rate_blk, max_row_tiles * t_tile_serial).
//   row-wise: one wavefront per (head, 8-row group); each stored tile costs
//     a fixed score pass plus a probability-times-V pass over the keys any
//     of the 8 rows can see:
//       T_row = c0 + (visits * t_visit + live_keys * t_key) / waves_parallel.
// Sparsity enters through the tile counts and the expected number of live
// keys of a partial tile (from its mean density); the sequence length
// through the tile counts and the per-row serial term.  The coefficients
// are timings measured on MI355X.
#include <math.h>

#include "smh_internal.h"

namespace smh {

namespace {
struct Coef {
    double launch_us;         // fixed cost of a launch
    double blk_tile_us;       // block-wise: one 64x64 tile, whole chip busy
    double blk_part_us;       // block-wise: extra per partial tile
    double blk_serial_us;     // block-wise: one tile on one workgroup
    double row_visit_us;      // row-wise: one (8 rows, tile) visit, chip busy
    double row_key_us;        // row-wise: one live key of a visit
    double row_serial_us;     // row-wise: one visit on one wavefront
};

// index: [d == 128][dtype]
const Coef kCoef[2][2] = {
    {{4.0, 1.2e-3, 0.2e-3, 0.35, 4.0e-4, 2.0e-5, 0.9},
     {4.0, 1.2e-3, 0.2e-3, 0.35, 4.0e-4, 2.0e-5, 0.9}},
    {{4.0, 2.2e-3, 0.2e-3, 0.6, 7.0e-4, 3.0e-5, 1.6},
     {4.0, 2.2e-3, 0.2e-3, 0.6, 7.0e-4, 3.0e-5, 1.6}},
};
}  // namespace

smh_kernel select_kernel(const smh_mask_stats &st, int64_t BH, int d,
                         int dtype, double *t_row_us, double *t_blk_us) {
    const Coef &k = kCoef[d == 128][dtype == SMH_BF16];
    const double tiles = (double)st.n_full + (double)st.n_partial;
    const double heads = (double)BH;
    // block-wise
    const double w_blk =
        heads * (tiles * k.blk_tile_us + st.n_partial * k.blk_part_us);
    const double crit_blk = st.max_row_tiles * k.blk_serial_us;
    const double t_blk = k.launch_us + fmax(w_blk, crit_blk);
    // row-wise: live keys of a partial tile for a group of 8 rows
    double live = 64.0 * st.n_full;
    if (st.n_partial > 0) {
        double rho = ((double)st.nnz - 4096.0 * st.n_full) /
                     (4096.0 * st.n_partial);
        rho = fmin(fmax(rho, 0.0), 1.0);
        live += st.n_partial * 64.0 * (1.0 - pow(1.0 - rho, 8.0));
    }
    const double w_row =
        heads * 8.0 * (tiles * k.row_visit_us + live * k.row_key_us);
    const double crit_row = st.max_row_tiles * k.row_serial_us;
    const double t_row = k.launch_us + fmax(w_row, crit_row);
    if (t_row_us) *t_row_us = t_row;
    if (t_blk_us) *t_blk_us = t_blk;
    return t_row < t_blk ? SMH_ROWWISE : SMH_BLOCKWISE;
}

}  // namespace smh
