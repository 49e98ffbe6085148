/* smh.h -- sparse masked multi-head attention forward for AMD MI355X (gfx950).
 *
 * Method: the unified sparse MHA module of STOF, as described on the pages
 *   [ABS] "Accelerating Sparse Transformer Inference on GPU", arXiv
 *         catalogue record, abstract;
 *   [EXP] "Accelerating Sparse Transformer Inference on GPU", gist.science
 *         explainer, Technical summary > Methodology > 1. Unified MHA module.
 * An arbitrary boolean attention mask is encoded once into a two-level
 * format (BSR outer tiles split into full and partial lists, one uint64
 * bitmap per 8x8 inner tile of each partial tile, empty tiles absent); a
 * row-wise kernel or a block-wise kernel, picked by an analytical cost model,
 * then computes masked softmax(Q K^T * scale) V reading only that encoding.
 *
 * Conventions shared by every entry point
 *   - Device buffers are owned by the caller.  The library never allocates,
 *     frees or synchronises device memory, except smh_mask_stats_get, which
 *     synchronises `stream`.
 *   - `stream` is a hipStream_t passed as void*; NULL is the null stream.
 *     Device work is enqueued on it and the call returns at once.
 *   - Every argument is validated on the host before anything is enqueued;
 *     on an error status nothing is enqueued and no output is written.
 *   - No C++ exception crosses this interface.  A failed kernel launch is
 *     reported as SMH_EHIP.
 *   - The library keeps no mutable global state besides cached device
 *     properties; calls are thread-safe.  Calls that share a workspace or an
 *     output buffer must be ordered by the caller (same stream or events).
 */
#ifndef SMH_H_
#define SMH_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SMH_OK = 0,
    SMH_EINVAL = 1,        /* bad argument (null pointer, size mismatch, ...) */
    SMH_EUNSUPPORTED = 2,  /* valid request outside what is built (d, dtype, S % 64) */
    SMH_ENOSPACE = 3,      /* workspace smaller than smh_encode_workspace_bytes */
    SMH_EHIP = 4           /* a HIP runtime call or kernel launch failed */
} smh_status;

typedef enum { SMH_F16 = 0, SMH_BF16 = 1, SMH_F32 = 2 } smh_dtype;

typedef enum {
    SMH_AUTO = 0,       /* let smh_select_kernel decide (needs host stats) */
    SMH_ROWWISE = 1,    /* row-wise kernel ([EXP] row-wise kernel item)     */
    SMH_BLOCKWISE = 2   /* block-wise kernel ([EXP] block-wise kernel item) */
} smh_kernel;

/* Largest sequence length accepted (the encoding workspace grows as
 * (S/64)^2 * 1040 bytes: 4.4 GB at this limit). */
#define SMH_MAX_S 131072
/* Outer tile edge and inner tile edge, in elements. */
#define SMH_OT 64
#define SMH_IT 8

/* The two-level encoding of one S x S mask ([EXP] storage-format items).
 * A host struct of device pointers into the caller's workspace; it stays
 * valid while the workspace lives and may be reused by any number of
 * smh_sparse_mha_fwd calls (every batch, head and layer that shares the
 * mask).  n_ot = S / 64 outer tiles per side.  Outer tile (I, J) covers
 * rows 64I..64I+63 and columns 64J..64J+63.
 *   full_row_ptr[n_ot+1], full_col_idx[n_full]: CSR lists of the outer
 *       tiles whose 4096 elements are all valid, J ascending in each row.
 *   part_row_ptr[n_ot+1], part_col_idx[n_partial]: CSR lists of the outer
 *       tiles with some but not all elements valid, J ascending.
 *   part_bitmaps[n_partial * 64]: the p-th partial tile (global order, i.e.
 *       position p in part_col_idx) owns words 64p..64p+63; word 8*ir+ic is
 *       inner tile (ir, ic), covering tile rows 8ir..8ir+7 and columns
 *       8ic..8ic+7; bit 8*r+c of it is element (8ir+r, 8ic+c).
 *   Outer tiles with no valid element appear in neither list.
 *   stats[5] (device int64): nnz, n_full, n_partial, n_empty_rows (query
 *       rows with no valid key), max_row_tiles (stored tiles in the fullest
 *       outer-tile row).
 *   row_order[n_ot] (device int32): outer-tile rows sorted by their number
 *       of stored tiles, most first, ties by ascending row (a schedule).
 * Capacities reserved in the workspace: col_idx arrays n_ot^2, bitmaps
 * n_ot^2 * 64 words. */
typedef struct {
    int32_t S;
    int32_t n_ot;
    int32_t *full_row_ptr;
    int32_t *full_col_idx;
    int32_t *part_row_ptr;
    int32_t *part_col_idx;
    uint64_t *part_bitmaps;
    int64_t *stats;
    int32_t *row_order;
} smh_mask_enc;

/* Host copy of the encoding statistics. */
typedef struct {
    int64_t nnz;          /* valid (query, key) pairs of the mask */
    int32_t S;
    int32_t n_full;       /* full outer tiles */
    int32_t n_partial;    /* partial outer tiles */
    int32_t n_empty_rows; /* query rows with no valid key (their output is 0) */
    int32_t max_row_tiles; /* stored tiles in the fullest outer-tile row */
} smh_mask_stats;

/* Bytes of device workspace smh_encode_mask needs for sequence length S
 * (encoding arrays plus internal scratch).  Returns 0 when S is not
 * accepted (S < 0, S % 64 != 0 or S > SMH_MAX_S); S == 0 is accepted. */
size_t smh_encode_workspace_bytes(int32_t S);

/* Encode a dense mask ([EXP] storage-format items: BSR outer tiles split
 * into full and partial pointer arrays, empty tiles skipped, one uint64 per
 * 8x8 inner tile of a partial tile).  Two or three kernel launches:
 * a strip pass over segments of outer-tile rows, then the placement of
 * their tiles (with the prefix scan inside it, or before it for long S).
 *   mask: device uint8 [S][S], row-major, 16-byte aligned, element (i, j)
 *         nonzero means query i attends to key j.  Read only.  NULL allowed
 *         only when S == 0.
 *   S: sequence length, 0 <= S <= SMH_MAX_S and S % 64 == 0 (else
 *      SMH_EUNSUPPORTED for S % 64 != 0, SMH_EINVAL for the rest).
 *   workspace: device memory, 256-byte aligned, at least
 *      smh_encode_workspace_bytes(S) bytes (else SMH_ENOSPACE); it holds the
 *      encoding afterwards and must outlive every use of *enc_out.
 *   enc_out: host struct filled with pointers into workspace.
 * The result is deterministic and independent of the launch configuration.
 * Asynchronous on `stream`. */
smh_status smh_encode_mask(const uint8_t *mask, int32_t S, void *workspace,
                           size_t ws_bytes, smh_mask_enc *enc_out,
                           void *stream);

/* Copy the encoding statistics to the host.  Synchronises `stream`. */
smh_status smh_mask_stats_get(const smh_mask_enc *enc, smh_mask_stats *out,
                              void *stream);

/* Analytical kernel choice ([EXP] kernel-selection item: the choice between
 * the row-wise and the block-wise kernel follows from mask sparsity and
 * sequence length; [ABS]: "analytical modeling").  Pure host arithmetic on
 * the statistics and the problem shape; touches no device.
 *   st: statistics of the mask (smh_mask_stats_get).
 *   B, H >= 0; d in {64, 128}; dt in {SMH_F16, SMH_BF16}.
 *   *out receives SMH_ROWWISE or SMH_BLOCKWISE. */
smh_status smh_select_kernel(const smh_mask_stats *st, int32_t B, int32_t H,
                             int32_t d, smh_dtype dt, smh_kernel *out);

/* The same model's predicted times (microseconds) of both kernels, for
 * reporting and for checking the choice against measurements.  Same
 * arguments and errors as smh_select_kernel; either output may be NULL. */
smh_status smh_select_costs(const smh_mask_stats *st, int32_t B, int32_t H,
                            int32_t d, smh_dtype dt, double *t_rowwise_us,
                            double *t_blockwise_us);

/* Masked attention forward: for every b < B, h < H and query row i,
 *   O[b,h,i,:] = sum_j w_j V[b,h,j,:] / sum_j w_j over valid keys j of row i,
 *   w_j = exp(scale * <Q[b,h,i,:], K[b,h,j,:]> - max), and O = 0 for a row
 * with no valid key.  Outer tiles absent from the encoding are never read.
 *   q, k, v: device [B][H][S][d] contiguous, element type in_dt (SMH_F16 or
 *            SMH_BF16), 16-byte aligned.  Read only.
 *   o: device [B][H][S][d] contiguous, element type out_dt (in_dt or
 *      SMH_F32), 16-byte aligned, not overlapping q, k or v.
 *   B, H >= 0 (0 is a no-op); S == enc->S; d in {64, 128}.
 *   scale: score multiplier, finite and >= 0; 0 means 1/sqrt(d).
 *   enc: encoding of the [S][S] mask shared by every (b, h).
 *   which: SMH_ROWWISE, SMH_BLOCKWISE, or SMH_AUTO.  With SMH_AUTO and st
 *          non-NULL the host decides (smh_select_kernel).  With SMH_AUTO and
 *          st NULL the same model is evaluated on the device from the
 *          statistics the encoder wrote, inside one fused launch that then
 *          runs the chosen algorithm, so no host synchronisation is needed.
 * Arithmetic: fp32 scores, softmax statistics and accumulators.  The
 * block-wise kernel rounds the probabilities to in_dt for its matrix-core
 * probability-times-V product (the row sums use the rounded values); the
 * row-wise kernel keeps them in fp32.  Asynchronous on `stream`. */
smh_status smh_sparse_mha_fwd(const void *q, const void *k, const void *v,
                              void *o, int32_t B, int32_t H, int32_t S,
                              int32_t d, smh_dtype in_dt, smh_dtype out_dt,
                              float scale, const smh_mask_enc *enc,
                              smh_kernel which, const smh_mask_stats *st,
                              void *stream);

/* Static description of a status code. */
const char *smh_status_string(smh_status s);

/* Library version string. */
const char *smh_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SMH_H_ */
