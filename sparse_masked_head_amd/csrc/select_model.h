// Cost model that chooses between the row-wise and the block-wise kernel.
//
// The pages state that an analytical model picks the kernel from the mask's
// sparsity and the sequence length ("Accelerating Sparse Transformer
// Inference on GPU", gist.science explainer, Technical summary >
// Methodology > 1. Unified MHA module, kernel-selection item; arXiv
// catalogue record, abstract) but give no formula.  This model predicts
// the time of each kernel from the encoding statistics and the problem
// shape and returns the cheaper one.
//
//   block-wise: one workgroup per (head, outer-tile row), one 64 x 64 x d
//     tile per step.  Work = stored tiles * heads; partial tiles add a
//     masking cost; sparse partial tiles (gather path) cost per tile and per
//     row-wise entry instead.  When the launch fits in one wave of
//     workgroups it runs for the length of its heaviest row instead, whose
//     tiles are taken to split like the mask's (a fraction f sparse, each
//     costing its entries per wavefront, ept = entries / (4 n_sparse)):
//       T_blk = c0 + max(W_blk, max_row_tiles * ((1 - f) t_tile_serial
//                                                 + f * ept * t_entry_serial)).
//   row-wise: one wavefront per (head, 8 query rows); it gathers the keys
//     its rows see from its row's stored tiles, 8 tiles per step, and
//     processes them in chunks of 64:
//       T_row = c0' + max(heads * (tiles * t_gather + 8 * chunks * t_chunk),
//                        max_row_tiles / 8 * t_gather_serial
//                        + (live_max / 64 + 1) * t_chunk_serial),
//     chunks = live / 64 + rows summed over the groups of one inner-tile
//     row index (each group pays at least one chunk).
// Sparsity enters through the tile counts and the expected number of live
// keys per (tile, 8-row group) of a partial tile (from the partial tiles'
// mean density, rho: 64 (1 - (1 - rho)^8)); sequence length through the
// tile counts, the row count and the serial terms.  The coefficients are
// microseconds, fitted (sparse_masked_head_amd/calibrate.py) to a sweep of
// both kernels on MI355X over mask families, S, heads and d.
//
// The same function runs on the host (smh_select_kernel) and inside both
// kernels (SMH_AUTO without host statistics), so it is written without
// library calls and with contraction off: both sides round identically.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

#define SMH_HD __host__ __device__

namespace smh {

// Statistics are totals over the masks of the stack; heads = (batch, head)
// pairs per mask; rows = outer-tile rows of the encoding (masks * n_ot).
struct SelectInput {
    int64_t nnz, n_full, n_partial, max_row_tiles;
    int64_t n_sparse, entries;  // sparse partial tiles, their row-wise entries
    int64_t heads, rows;
    int d, bf16;
};

struct SelectCoef {
    double launch_us;          // fixed cost of a launch
    double blk_tile_us;        // block-wise: one 64x64 tile, whole chip busy
    double blk_part_us;        // block-wise: extra per partial tile
    double blk_serial_us;      // block-wise: one tile on one workgroup
    double row_gather_us;      // row-wise: one (tile, head) gathered, chip busy
    double row_chunk_us;       // row-wise: one 64-key chunk, chip busy
    double row_gather_ser_us;  // row-wise: one 8-tile gather step, one wavefront
    double row_chunk_ser_us;   // row-wise: one chunk on one wavefront
    double blk_entry_us;       // block-wise gather path: one row-wise entry
    double blk_sparse_us;      // block-wise gather path: one sparse tile
    double blk_entry_ser_us;   // gather path: one entry on one wavefront
    double row_launch_us;      // row-wise: fixed cost of a launch
};

#pragma clang fp contract(off)
SMH_HD inline void select_costs_us(const SelectInput &in, double *t_row,
                                   double *t_blk) {
    // fitted on MI355X; fp16 and bf16 share coefficients
    const SelectCoef k64 = {8.0248, 0.0013977, 2.3023e-4, 0.45568,
                            1.7098e-4, 0.0011503, 0.3563, 1.6753,
                            8.5026e-6, 6.2755e-5, 0.019472, 4.8561};
    const SelectCoef k128 = {8.0277, 0.0028768, 5.045e-4, 0.73646,
                             3.3023e-4, 0.0024028, 0.47397, 3.3185,
                             1.4585e-5, 1.935e-4, 0.024057, 3.2402};
    const SelectCoef &k = in.d == 128 ? k128 : k64;
    const double tiles = (double)in.n_full + (double)in.n_partial;
    const double heads = (double)in.heads;
    // the sparse tiles go to the gather path when the encoding holds their
    // row-wise entries (a sparse tile has at least one)
    const double nsp = in.entries > 0 ? (double)in.n_sparse : 0.0;
    const double w_blk =
        heads * ((tiles - nsp) * k.blk_tile_us +
                 ((double)in.n_partial - nsp) * k.blk_part_us +
                 (double)in.entries * k.blk_entry_us + nsp * k.blk_sparse_us);
    const double f = tiles > 0.0 ? nsp / tiles : 0.0;
    const double ept = nsp > 0.0 ? (double)in.entries / (4.0 * nsp) : 0.0;
    const double crit_blk =
        (double)in.max_row_tiles *
        ((1.0 - f) * k.blk_serial_us + f * ept * k.blk_entry_ser_us);
    *t_blk = k.launch_us + (w_blk > crit_blk ? w_blk : crit_blk);
    double live = 64.0 * (double)in.n_full;
    if (in.n_partial > 0) {
        double rho = ((double)in.nnz - 4096.0 * (double)in.n_full) /
                     (4096.0 * (double)in.n_partial);
        rho = rho < 0.0 ? 0.0 : (rho > 1.0 ? 1.0 : rho);
        double miss = 1.0 - rho;   // (1 - rho)^8: no row of 8 sees the key
        miss = miss * miss;
        miss = miss * miss;
        miss = miss * miss;
        live += (double)in.n_partial * 64.0 * (1.0 - miss);
    }
    const double chunks = live / 64.0 + (double)in.rows;
    const double w_row =
        heads * (tiles * k.row_gather_us + 8.0 * chunks * k.row_chunk_us);
    const double live_max =
        tiles > 0.0 ? live / tiles * (double)in.max_row_tiles : 0.0;
    const double crit_row = (double)in.max_row_tiles / 8.0 * k.row_gather_ser_us +
                            (live_max / 64.0 + 1.0) * k.row_chunk_ser_us;
    *t_row = k.row_launch_us + (w_row > crit_row ? w_row : crit_row);
}

// Row-wise is taken when its predicted time is below this fraction of the
// block-wise one.  With the split critical path and per-kernel launch
// costs the plain comparison loses 0.16% (d = 64) and 0.03% (d = 128) of
// the calibration sweep's total time to wrong picks (every pick within 3%
// of the faster kernel on 170 and 172 of 180 points), so no margin is kept.
constexpr double kRowMargin = 1.0;

// 1 = row-wise, 2 = block-wise (the smh_kernel values).
SMH_HD inline int select_model(const SelectInput &in) {
    double tr, tb;
    select_costs_us(in, &tr, &tb);
    return tr < kRowMargin * tb ? 1 : 2;
}
#pragma clang fp contract(on)

// Device side: read the statistics the encoder wrote and decide.
__device__ inline int select_on_device(const int64_t *stats, int64_t heads,
                                       int64_t rows, int d, int bf16) {
    SelectInput in;
    in.nnz = stats[0];
    in.n_full = stats[1];
    in.n_partial = stats[2];
    in.max_row_tiles = stats[4];
    in.n_sparse = stats[5];
    in.entries = stats[6];
    in.heads = heads;
    in.rows = rows;
    in.d = d;
    in.bf16 = bf16;
    return select_model(in);
}

}  // namespace smh
