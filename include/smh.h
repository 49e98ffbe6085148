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
 *     synchronises `stream`.  (smh_encode_masks_noalloc uses a fixed device
 *     array of the library's code object as scratch.)
 *   - `stream` is a hipStream_t passed as void*; NULL is the null stream.
 *     Device work is enqueued on it and the call returns at once.
 *   - Every argument is validated on the host before anything is enqueued;
 *     on an error status nothing is enqueued and no output is written.
 *   - No C++ exception crosses this interface.  A failed kernel launch is
 *     reported as SMH_EHIP.
 *   - The library keeps no mutable global state besides cached device
 *     properties and the static encoder scratch of
 *     smh_encode_masks_noalloc (see there); calls are thread-safe.  Calls that share a workspace or an
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
    SMH_EUNSUPPORTED = 2,  /* valid request outside what is built (d, dtype) */
    SMH_ENOSPACE = 3,      /* workspace smaller than smh_encode_workspace_bytes */
    SMH_EHIP = 4           /* a HIP runtime call or kernel launch failed */
} smh_status;

typedef enum { SMH_F16 = 0, SMH_BF16 = 1, SMH_F32 = 2 } smh_dtype;

typedef enum {
    SMH_AUTO = 0,       /* let smh_select_kernel decide (needs host stats) */
    SMH_ROWWISE = 1,    /* row-wise kernel ([EXP] row-wise kernel item)     */
    SMH_BLOCKWISE = 2,  /* block-wise kernel ([EXP] block-wise kernel item)
                           with per-tile dispatch: sparse partial tiles (at
                           most SMH_SPARSE_TILE_MAX valid elements) on its
                           gather path when S <= 65536                      */
    SMH_BLOCKWISE_DENSE = 3  /* block-wise kernel, every stored tile on the
                                matrix-core tile path                        */
} smh_kernel;

/* Largest sequence length accepted (the encoding workspace of one mask
 * grows as ceil(S/64)^2 * 1040 bytes: 4.4 GB at this limit). */
#define SMH_MAX_S 131072
/* Largest number of outer-tile rows of one encoding: masks in the stack
 * times ceil(S/64). */
#define SMH_MAX_ENC_ROWS 8192
/* Outer tile edge and inner tile edge, in elements. */
#define SMH_OT 64
#define SMH_IT 8
/* A partial outer tile with at most this many valid elements (2.7% of its
 * 4096) is "sparse": the block-wise kernel computes it on its gather path
 * (each wavefront gathers the keys its 16 query rows see) instead of as a
 * dense 64 x 64 tile, when the mask's length allows (S <= 65536).  The
 * gather path is the faster one below about 105 valid elements per tile on
 * MI355X (random masks of rising density, d = 64 and 128). */
#define SMH_SPARSE_TILE_MAX 112

/* The two-level encoding of a stack of S x S masks ([EXP] storage-format
 * items).  A host struct of device pointers into the caller's workspace; it
 * stays valid while the workspace lives and may be reused by any number of
 * smh_sparse_mha_fwd calls (every batch, head and layer that shares the
 * masks).
 *   The stack holds G = mask_b * mask_h masks, mask g = gb * mask_h + gh
 *   (gb < mask_b, gh < mask_h); one mask is the stack 1 x 1.  Batch b and
 *   head h of an attention call use mask (mask_b > 1 ? b : 0, mask_h > 1 ?
 *   h : 0), so mask_b is 1 or B and mask_h is 1 or H (broadcasting).
 *   n_ot = ceil(S / 64) outer tiles per side.  Outer tile (I, J) covers rows
 *   64I..64I+63 and columns 64J..64J+63; when S is not a multiple of 64 the
 *   last row and column of tiles are cut by S, and elements outside the
 *   S x S mask count as not valid (so a cut tile is never full).
 *   The encoding has R = G * n_ot rows: row g * n_ot + I is outer-tile row
 *   I of mask g.  Column indices J are in [0, n_ot).
 *   full_row_ptr[R+1], full_col_idx[n_full]: CSR lists of the outer
 *       tiles whose 4096 elements are all valid, J ascending in each row.
 *   part_row_ptr[R+1], part_col_idx[n_partial]: CSR lists of the outer
 *       tiles with some but not all elements valid, J ascending.
 *   part_bitmaps[n_partial * 64]: the p-th partial tile (global order, i.e.
 *       position p in part_col_idx) owns words 64p..64p+63; word 8*ir+ic is
 *       inner tile (ir, ic), covering tile rows 8ir..8ir+7 and columns
 *       8ic..8ic+7; bit 8*r+c of it is element (8ir+r, 8ic+c).
 *   Outer tiles with no valid element appear in neither list.
 *   stats[8] (device int64), summed over the stack: nnz, n_full,
 *       n_partial, n_empty_rows (query rows with no valid key),
 *       max_row_tiles (stored tiles in the fullest outer-tile row), n_sparse
 *       (partial tiles with at most SMH_SPARSE_TILE_MAX valid elements),
 *       sparse_nnz (their valid elements) and row_entries (the row-wise
 *       entries of those tiles, the sum of row_ent_cnt).
 *   part_pop[n_partial] (device int32): valid elements of each partial tile
 *       (the population count of its 64 words), in part_col_idx order.
 *   row_ent, row_ent_cnt (device uint32, int32): the row-wise format of
 *       the sparse partial tiles ([ABS]: the row-wise kernel reads a format
 *       of its own), built when S <= 65536 (else every count is 0).  For
 *       encoding row r (outer-tile row I) and group q < 4 of 16 query rows
 *       (rows 64I + 16q .. +15): the keys j of the row's sparse tiles that
 *       some query of the group attends to, ascending, each entry
 *       rows << 16 | j with bit 16 + k set iff query 64I + 16q + k attends
 *       to j; entry i < row_ent_cnt[4r + q] at
 *       row_ent[256 * part_row_ptr[r] + 64 * q * np + i], np = the row's
 *       partial-tile count.
 *   row_order[R] (device int32): the encoding's rows sorted by their number
 *       of stored tiles, most first, ties by ascending row (a schedule).
 *   row_info[R][16] (device int32): a summary of each row that a kernel
 *       reads in one load: [0] full_row_ptr[r], [1] its full-tile count,
 *       [2] part_row_ptr[r], [3] its partial-tile count, [4..7] the columns
 *       of the row's first four stored tiles in list order (full tiles,
 *       then partial tiles), -1 past the row's last tile, [8..15] the
 *       encoding's nnz (low, high 32 bits), n_full, n_partial,
 *       max_row_tiles, n_sparse and row_entries (low, high 32 bits).
 * Capacities reserved in the workspace: col_idx and part_pop arrays
 * R * n_ot, bitmaps R * n_ot * 64 words, row_ent R * n_ot * 256 entries
 * (S <= 65536). */
typedef struct {
    int32_t S;
    int32_t n_ot;
    int32_t mask_b;
    int32_t mask_h;
    int32_t *full_row_ptr;
    int32_t *full_col_idx;
    int32_t *part_row_ptr;
    int32_t *part_col_idx;
    uint64_t *part_bitmaps;
    int64_t *stats;
    int32_t *row_order;
    int32_t *row_info;
    int32_t *part_pop;
    uint32_t *row_ent;
    int32_t *row_ent_cnt;
} smh_mask_enc;

/* Host copy of the encoding statistics (totals over the masks of the
 * stack). */
typedef struct {
    int64_t nnz;          /* valid (query, key) pairs of the masks */
    int32_t S;
    int32_t n_full;       /* full outer tiles */
    int32_t n_partial;    /* partial outer tiles */
    int32_t n_empty_rows; /* query rows with no valid key (their output is 0) */
    int32_t max_row_tiles; /* stored tiles in the fullest outer-tile row */
    int32_t mask_b;       /* the stack's shape, as in smh_mask_enc */
    int32_t mask_h;
    int32_t n_sparse;     /* partial tiles of at most SMH_SPARSE_TILE_MAX valid elements */
    int64_t sparse_nnz;   /* valid pairs in those tiles */
    int64_t row_entries;  /* their row-wise entries (0 when S > 65536) */
} smh_mask_stats;

/* Bytes of device workspace smh_encode_mask needs for sequence length S
 * (encoding arrays plus internal scratch).  Returns 0 when S is not
 * accepted (S < 0 or S > SMH_MAX_S); S == 0 is accepted. */
size_t smh_encode_workspace_bytes(int32_t S);

/* The same for a stack of mask_b x mask_h masks (smh_encode_masks).
 * Returns 0 when the arguments are not accepted (mask_b or mask_h < 1,
 * S out of range, or mask_b * mask_h * ceil(S/64) > SMH_MAX_ENC_ROWS). */
size_t smh_encode_masks_workspace_bytes(int32_t mask_b, int32_t mask_h,
                                        int32_t S);

/* Encode a dense mask ([EXP] storage-format items: BSR outer tiles split
 * into full and partial pointer arrays, empty tiles skipped, one uint64 per
 * 8x8 inner tile of a partial tile).  Two or three kernel launches:
 * a strip pass over segments of outer-tile rows, then the placement of
 * their tiles (with the prefix scan inside it, or before it for long S).
 *   mask: device uint8 [S][S], row-major, 16-byte aligned, element (i, j)
 *         nonzero means query i attends to key j.  Read only.  NULL allowed
 *         only when S == 0.
 *   S: sequence length, 0 <= S <= SMH_MAX_S (else SMH_EINVAL); any S,
 *      the last outer tiles are cut when S % 64 != 0.
 *   workspace: device memory, 256-byte aligned, at least
 *      smh_encode_workspace_bytes(S) bytes (else SMH_ENOSPACE); it holds the
 *      encoding afterwards and must outlive every use of *enc_out.
 *   enc_out: host struct filled with pointers into workspace (mask_b =
 *      mask_h = 1).
 * The result is deterministic and independent of the launch configuration.
 * Asynchronous on `stream`. */
smh_status smh_encode_mask(const uint8_t *mask, int32_t S, void *workspace,
                           size_t ws_bytes, smh_mask_enc *enc_out,
                           void *stream);

/* Encode a stack of masks, one per batch and/or head ([EXP] problem
 * statement: the mask decides which pairs take part, and it may differ
 * from sequence to sequence).  One encoding holds them all (layout in
 * smh_mask_enc); the launches are those of smh_encode_mask, over every
 * mask at once.
 *   masks: device uint8 [mask_b][mask_h][S][S] contiguous, 16-byte
 *          aligned, nonzero = valid.  Read only.
 *   mask_b, mask_h >= 1, mask_b * mask_h * ceil(S/64) <= SMH_MAX_ENC_ROWS
 *          (else SMH_EINVAL).
 *   S, workspace (smh_encode_masks_workspace_bytes bytes), enc_out: as for
 *          smh_encode_mask.
 * Encoding a 1 x 1 stack is smh_encode_mask. */
smh_status smh_encode_masks(const uint8_t *masks, int32_t mask_b,
                            int32_t mask_h, int32_t S, void *workspace,
                            size_t ws_bytes, smh_mask_enc *enc_out,
                            void *stream);

/* Size of the static encoder scratch of smh_encode_masks_noalloc: 40 MiB,
 * enough for one mask of S = 16384 (33 MiB) or any stack with as many
 * outer tiles.  Every device the library runs on holds one copy of it in
 * the library's code object until the process ends. */
#define SMH_STATIC_SCRATCH_BYTES ((size_t)40 << 20)

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the
 * encoder of smh_encode_masks without a workspace argument.  The encoding
 * is written to the caller's `enc_buf`; the encoder's internal scratch is
 * the library's static device array (SMH_STATIC_SCRATCH_BYTES per device,
 * its address looked up once per device on the first call there).  The
 * call allocates nothing: no hipMalloc, hipFree or allocating library
 * routine.  Same launches, result and layout as smh_encode_masks.
 *   enc_bytes (in/out): with enc_buf == NULL the call only stores the
 *       number of bytes the encoding needs in *enc_bytes and returns
 *       SMH_OK (nothing enqueued, no device touched).  Otherwise *enc_bytes
 *       is the capacity of enc_buf (SMH_ENOSPACE when smaller than that
 *       number).
 *   enc_buf: device memory, 256-byte aligned, on the current device; it
 *       holds the encoding afterwards and must outlive every use of
 *       *enc_out.
 *   masks, mask_b, mask_h, S, enc_out, stream: as for smh_encode_masks;
 *       the stream must belong to the current device.
 * SMH_EUNSUPPORTED when the scratch the stack needs exceeds
 * SMH_STATIC_SCRATCH_BYTES (about ceil(S/64)^2 * masks * 530 bytes).
 * Every call on a device shares that device's scratch (no call needs it
 * cleared, and each call's result depends only on its own inputs): calls
 * that may overlap on one device (different streams, different host
 * threads) race and must be ordered by the caller. */
smh_status smh_encode_masks_noalloc(const uint8_t *masks, int32_t mask_b,
                                    int32_t mask_h, int32_t S, void *enc_buf,
                                    size_t *enc_bytes, smh_mask_enc *enc_out,
                                    void *stream);

/* A mask described by its pattern instead of stored ([EXP] storage-format
 * items: the encoding is built without the dense S x S mask).  Element
 * (i, j), i, j < S, is valid iff
 *     (causal == 0 or j <= i)  and  (
 *         |i - j| <= window                       (window >= 0; -1: no band)
 *      or i < global_rows  or  j < global_cols    (global tokens)
 *      or blocks[i/64][j/64] == 1                 (a listed 64x64 block)
 *      or blocks[i/64][j/64] not in {0, 1} and u(i, j) < keep16
 *      or blocks[i/64][j/64] == 0 (or no map) and u(i, j) < rand16 )
 * with keep16 = floor(block_keep * 65536), rand16 = floor(random_p * 65536)
 * (float arithmetic) and u(i, j) the element's 16-bit draw: with
 * e = i * S + j, bits 16 (e % 4) .. 16 (e % 4) + 15 of output number e / 4
 * (from 0) of SplitMix64 seeded with `seed` (Steele, Lea and Flood, OOPSLA
 * 2014: output k = mix(seed + (k + 1) * 0x9E3779B97F4A7C15)).  With
 * block_keep == 1 and random_p == 0 the pattern has no random part. */
typedef struct {
    int32_t causal;        /* nonzero: keys j <= i only */
    int32_t window;        /* band half-width, >= 0, or -1 for no band */
    int32_t global_rows;   /* >= 0 */
    int32_t global_cols;   /* >= 0 */
    const uint8_t *blocks; /* device [ceil(S/64)][ceil(S/64)] block map, or NULL */
    float block_keep;      /* in [0, 1] */
    float random_p;        /* in [0, 1] */
    uint64_t seed;
} smh_pattern;

/* Encode the mask a pattern describes.  Same launches, output, workspace
 * (smh_encode_workspace_bytes(S)) and errors as smh_encode_mask, with
 * the strip pass computing each inner-tile row from the pattern instead of
 * reading mask bytes; the result equals smh_encode_mask of the dense mask
 * the pattern describes.  SMH_EINVAL for a NULL pattern, window < -1,
 * negative global counts or probabilities outside [0, 1]. */
smh_status smh_encode_pattern(const smh_pattern *pattern, int32_t S,
                              void *workspace, size_t ws_bytes,
                              smh_mask_enc *enc_out, void *stream);

/* Copy the encoding statistics to the host.  Synchronises `stream`. */
smh_status smh_mask_stats_get(const smh_mask_enc *enc, smh_mask_stats *out,
                              void *stream);

/* Analytical kernel choice ([EXP] kernel-selection item: the choice between
 * the row-wise and the block-wise kernel follows from mask sparsity and
 * sequence length; [ABS]: "analytical modeling").  Pure host arithmetic on
 * the statistics and the problem shape; touches no device.
 *   st: statistics of the mask stack (smh_mask_stats_get).
 *   B, H >= 0, st->mask_b in {1, B}, st->mask_h in {1, H} (else
 *   SMH_EINVAL); d in {64, 128}; dt in {SMH_F16, SMH_BF16}.
 *   *out receives SMH_ROWWISE or SMH_BLOCKWISE. */
smh_status smh_select_kernel(const smh_mask_stats *st, int32_t B, int32_t H,
                             int32_t d, smh_dtype dt, smh_kernel *out);

/* The same model's predicted times (microseconds) of both kernels, for
 * reporting and for checking the choice against measurements.  Same
 * arguments and errors as smh_select_kernel; either output may be NULL. */
smh_status smh_select_costs(const smh_mask_stats *st, int32_t B, int32_t H,
                            int32_t d, smh_dtype dt, double *t_rowwise_us,
                            double *t_blockwise_us);

/* Masked attention forward ([EXP] Technical summary > Problem statement: a
 * mask decides which (query, key) pairs take part in softmax(Q K^T) V, and
 * a masked pair must not contribute; Methodology > 1. Unified MHA module:
 * the row-wise and block-wise kernels read only the two-level encoding,
 * skip absent outer tiles and mask partial ones bit by bit from their
 * inner-tile bitmaps, so the result is exact).  For every b < B, h < H and
 * query row i,
 *   O[b,h,i,:] = sum_j w_j V[b,h,j,:] / sum_j w_j over valid keys j of row i
 *   in the mask of (b, h),
 *   w_j = exp(scale * <Q[b,h,i,:], K[b,h,j,:]> - max), and O = 0 for a row
 * with no valid key.  Outer tiles absent from the encoding are never read.
 *   q, k, v: device [B][H][S][d] contiguous, element type in_dt (SMH_F16 or
 *            SMH_BF16), 16-byte aligned.  Read only.
 *   o: device [B][H][S][d] contiguous, element type out_dt (in_dt or
 *      SMH_F32), 16-byte aligned, not overlapping q, k or v.
 *   B, H >= 0 (0 is a no-op); S == enc->S (any S up to SMH_MAX_S);
 *   d in {64, 128}.
 *   scale: score multiplier, finite and >= 0; 0 means 1/sqrt(d).
 *   enc: encoding of the mask stack: enc->mask_b in {1, B} and enc->mask_h
 *        in {1, H} (else SMH_EINVAL); (b, h) uses the mask smh_mask_enc
 *        describes.
 *   which: SMH_ROWWISE, SMH_BLOCKWISE, or SMH_AUTO.  With SMH_AUTO and st
 *          non-NULL the host decides (smh_select_kernel).  With SMH_AUTO and
 *          st NULL the same model is evaluated on the device from the
 *          statistics the encoder wrote, inside one fused launch that then
 *          runs the chosen algorithm, so no host synchronisation is needed.
 * Arithmetic: fp32 scores, softmax statistics and accumulators.  Both
 * kernels round the probabilities to in_dt for their matrix-core
 * probability-times-V product, and the row sums use the rounded values.
 * Q, K and V must be finite: a
 * masked key's V row is multiplied by a zero probability.  Asynchronous on
 * `stream`. */
smh_status smh_sparse_mha_fwd(const void *q, const void *k, const void *v,
                              void *o, int32_t B, int32_t H, int32_t S,
                              int32_t d, smh_dtype in_dt, smh_dtype out_dt,
                              float scale, const smh_mask_enc *enc,
                              smh_kernel which, const smh_mask_stats *st,
                              void *stream);

/* Output projection of the attention result, with bias and residual added
 * in the same pass (the pages' operator-fusion module fuses MHA with the
 * operators that follow it: [EXP] Methodology > 2. operator fusion; this
 * is one such fused operator, written by hand):
 *   out[b, s, n] = sum_{h < H, k < d} O[b, h, s, k] * W[n, h*d + k]
 *                  + bias[n] + residual[b, s, n]
 *   o: device [B][H][S][d] (the layout smh_sparse_mha_fwd writes), dt.
 *   w: device [D][H*d] row-major (a linear layer's weight: out = x W^T), dt.
 *   bias: device [D] or NULL (no bias), dt.
 *   residual: device [B][S][D] or NULL (no residual), dt.
 *   out: device [B][S][D], dt, not overlapping o, w or bias; it may be
 *        residual itself (in place) but not overlap it otherwise.
 *   B, H, S >= 0 (an empty product is a no-op); d in {64, 128}; D > 0 and
 *   D % 64 == 0 (else SMH_EUNSUPPORTED); dt in {SMH_F16, SMH_BF16}.
 *   All pointers 16-byte aligned.
 * Products on the matrix cores with fp32 accumulation; bias and residual
 * are added in fp32 and the sum is rounded once to dt.  One launch,
 * asynchronous on `stream`. */
smh_status smh_out_proj(const void *o, const void *w, const void *bias,
                        const void *residual, void *out, int32_t B,
                        int32_t H, int32_t S, int32_t d, int32_t D,
                        smh_dtype dt, void *stream);

/* Static description of a status code. */
const char *smh_status_string(smh_status s);

/* Library version string. */
const char *smh_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SMH_H_ */
