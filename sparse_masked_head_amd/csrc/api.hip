// C interface of libsmh: argument validation and dispatch.  Every check
// happens before anything is enqueued; see include/smh.h for the contract.
#include <math.h>
#include <string.h>

#include "smh_internal.h"

using namespace smh;

namespace {

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Outer-tile rows of a stack of mask_b x mask_h masks of S x S, or -1 when
// the stack is not accepted.
int64_t stack_rows(int32_t mask_b, int32_t mask_h, int32_t S) {
    if (S < 0 || S > SMH_MAX_S || mask_b < 1 || mask_h < 1) return -1;
    const int64_t rows = (int64_t)mask_b * mask_h * (((int64_t)S + SMH_OT - 1) / SMH_OT);
    return rows > SMH_MAX_ENC_ROWS ? -1 : rows;
}

// A mask stack [mask_b][mask_h] serves B x H (batch, head) pairs when each
// side is 1 (broadcast) or equal.
bool broadcasts(int32_t mask_b, int32_t mask_h, int32_t B, int32_t H) {
    return (mask_b == 1 || mask_b == B) && (mask_h == 1 || mask_h == H);
}

smh_status check_stats(const smh_mask_stats *st) {
    if (!st) return SMH_EINVAL;
    const int64_t rows = stack_rows(st->mask_b, st->mask_h, st->S);
    if (rows < 0) return SMH_EINVAL;
    const int64_t n = ((int64_t)st->S + SMH_OT - 1) / SMH_OT;
    const int64_t G = (int64_t)st->mask_b * st->mask_h;
    if (st->n_full < 0 || st->n_partial < 0 || st->nnz < 0 ||
        st->max_row_tiles < 0 || st->n_empty_rows < 0 || st->n_sparse < 0 ||
        st->sparse_nnz < 0)
        return SMH_EINVAL;
    if (st->n_sparse > st->n_partial || st->row_entries < 0 ||
        st->sparse_nnz > (int64_t)st->n_sparse * SMH_SPARSE_TILE_MAX ||
        st->row_entries > st->sparse_nnz)
        return SMH_EINVAL;
    if ((int64_t)st->n_full + st->n_partial > rows * n ||
        st->nnz > G * st->S * st->S || st->max_row_tiles > n)
        return SMH_EINVAL;
    return SMH_OK;
}

smh_status check_select(const smh_mask_stats *st, int32_t B, int32_t H,
                        int32_t d, smh_dtype dt) {
    smh_status s = check_stats(st);
    if (s != SMH_OK) return s;
    if (B < 0 || H < 0) return SMH_EINVAL;
    if (B > 0 && H > 0 && !broadcasts(st->mask_b, st->mask_h, B, H))
        return SMH_EINVAL;
    if (d != 64 && d != 128) return SMH_EUNSUPPORTED;
    if (dt != SMH_F16 && dt != SMH_BF16) return SMH_EUNSUPPORTED;
    return SMH_OK;
}

// The encoding's pointers into workspace `ws` laid out as L.
void fill_enc(smh_mask_enc &e, char *ws, const EncLayout &L, int32_t S,
              int32_t mask_b, int32_t mask_h) {
    e.S = S;
    e.n_ot = (int32_t)L.n;
    e.mask_b = mask_b;
    e.mask_h = mask_h;
    e.full_row_ptr = (int32_t *)(ws + L.full_row_ptr);
    e.full_col_idx = (int32_t *)(ws + L.full_col_idx);
    e.part_row_ptr = (int32_t *)(ws + L.part_row_ptr);
    e.part_col_idx = (int32_t *)(ws + L.part_col_idx);
    e.part_bitmaps = (uint64_t *)(ws + L.part_bitmaps);
    e.stats = (int64_t *)(ws + L.stats);
    e.row_order = (int32_t *)(ws + L.row_order);
    e.row_info = (int32_t *)(ws + L.row_info);
    e.part_pop = (int32_t *)(ws + L.part_pop);
    e.row_ent = (uint32_t *)(ws + L.row_ent);
    e.row_ent_cnt = (int32_t *)(ws + L.row_ent_cnt);
}

// (batch, head) pairs that share each mask of the stack.
int64_t heads_per_mask(const smh_mask_stats *st, int32_t B, int32_t H) {
    return (int64_t)(st->mask_b > 1 ? 1 : B) * (st->mask_h > 1 ? 1 : H);
}

}  // namespace

extern "C" {

const char *smh_version(void) { return "smh 0.2 (gfx950)"; }

const char *smh_status_string(smh_status s) {
    switch (s) {
        case SMH_OK: return "ok";
        case SMH_EINVAL: return "invalid argument";
        case SMH_EUNSUPPORTED: return "unsupported configuration";
        case SMH_ENOSPACE: return "workspace too small";
        case SMH_EHIP: return "HIP runtime error";
    }
    return "unknown status";
}

size_t smh_encode_masks_workspace_bytes(int32_t mask_b, int32_t mask_h,
                                        int32_t S) {
    if (stack_rows(mask_b, mask_h, S) < 0) return 0;
    return enc_layout(S, (int64_t)mask_b * mask_h).total;
}

size_t smh_encode_workspace_bytes(int32_t S) {
    return smh_encode_masks_workspace_bytes(1, 1, S);
}

smh_status smh_encode_masks(const uint8_t *masks, int32_t mask_b,
                            int32_t mask_h, int32_t S, void *workspace,
                            size_t ws_bytes, smh_mask_enc *enc_out,
                            void *stream) {
    try {
        if (stack_rows(mask_b, mask_h, S) < 0) return SMH_EINVAL;
        if (!enc_out || !workspace) return SMH_EINVAL;
        if (S > 0 && (!masks || !aligned(masks, 16))) return SMH_EINVAL;
        if (!aligned(workspace, 256)) return SMH_EINVAL;
        const int64_t G = (int64_t)mask_b * mask_h;
        const EncLayout L = enc_layout(S, G);
        if (ws_bytes < L.total) return SMH_ENOSPACE;
        if (S > 0 && overlaps(masks, (size_t)G * S * S, workspace, L.total))
            return SMH_EINVAL;
        char *ws = (char *)workspace;
        smh_mask_enc e;
        fill_enc(e, ws, L, S, mask_b, mask_h);
        if (launch_encode(masks, S, L, e, ws + enc_output_bytes(L),
                          (hipStream_t)stream) !=
            hipSuccess)
            return SMH_EHIP;
        *enc_out = e;
        return SMH_OK;
    } catch (...) {
        return SMH_EHIP;
    }
}

smh_status smh_encode_pattern(const smh_pattern *pat, int32_t S,
                              void *workspace, size_t ws_bytes,
                              smh_mask_enc *enc_out, void *stream) {
    try {
        if (!pat || stack_rows(1, 1, S) < 0) return SMH_EINVAL;
        if (!enc_out || !workspace || !aligned(workspace, 256)) return SMH_EINVAL;
        if (pat->window < -1 || pat->global_rows < 0 || pat->global_cols < 0)
            return SMH_EINVAL;
        if (!(pat->block_keep >= 0.f && pat->block_keep <= 1.f) ||
            !(pat->random_p >= 0.f && pat->random_p <= 1.f))
            return SMH_EINVAL;
        const EncLayout L = enc_layout(S, 1);
        if (ws_bytes < L.total) return SMH_ENOSPACE;
        const size_t n = (size_t)L.n;
        if (pat->blocks && overlaps(pat->blocks, n * n, workspace, L.total))
            return SMH_EINVAL;
        char *ws = (char *)workspace;
        smh_mask_enc e;
        fill_enc(e, ws, L, S, 1, 1);
        if (launch_encode_pattern(*pat, S, L, e, ws + enc_output_bytes(L),
                                  (hipStream_t)stream) !=
            hipSuccess)
            return SMH_EHIP;
        *enc_out = e;
        return SMH_OK;
    } catch (...) {
        return SMH_EHIP;
    }
}

smh_status smh_encode_masks_noalloc(const uint8_t *masks, int32_t mask_b,
                                    int32_t mask_h, int32_t S, void *enc_buf,
                                    size_t *enc_bytes, smh_mask_enc *enc_out,
                                    void *stream) {
    try {
        if (stack_rows(mask_b, mask_h, S) < 0 || !enc_bytes) return SMH_EINVAL;
        const int64_t G = (int64_t)mask_b * mask_h;
        const EncLayout L = enc_layout(S, G);
        const size_t need = enc_output_bytes(L);
        if (!enc_buf) {  // size query: nothing enqueued, no device touched
            *enc_bytes = need;
            return SMH_OK;
        }
        if (!enc_out) return SMH_EINVAL;
        if (S > 0 && (!masks || !aligned(masks, 16))) return SMH_EINVAL;
        if (!aligned(enc_buf, 256)) return SMH_EINVAL;
        if (*enc_bytes < need) return SMH_ENOSPACE;
        if (enc_scratch_bytes(L) > SMH_STATIC_SCRATCH_BYTES) return SMH_EUNSUPPORTED;
        if (S > 0 && overlaps(masks, (size_t)G * S * S, enc_buf, need))
            return SMH_EINVAL;
        char *scratch = nullptr;
        if (static_scratch(&scratch) != hipSuccess) return SMH_EHIP;
        char *ws = (char *)enc_buf;
        smh_mask_enc e;
        fill_enc(e, ws, L, S, mask_b, mask_h);
        if (launch_encode(masks, S, L, e, scratch, (hipStream_t)stream) !=
            hipSuccess)
            return SMH_EHIP;
        *enc_out = e;
        return SMH_OK;
    } catch (...) {
        return SMH_EHIP;
    }
}

smh_status smh_encode_mask(const uint8_t *mask, int32_t S, void *workspace,
                           size_t ws_bytes, smh_mask_enc *enc_out,
                           void *stream) {
    return smh_encode_masks(mask, 1, 1, S, workspace, ws_bytes, enc_out,
                            stream);
}

smh_status smh_mask_stats_get(const smh_mask_enc *enc, smh_mask_stats *out,
                              void *stream) {
    try {
        if (!enc || !out || !enc->stats) return SMH_EINVAL;
        if (stack_rows(enc->mask_b, enc->mask_h, enc->S) < 0) return SMH_EINVAL;
        int64_t h[8];
        hipStream_t s = (hipStream_t)stream;
        if (hipMemcpyAsync(h, enc->stats, sizeof(h), hipMemcpyDeviceToHost,
                           s) != hipSuccess)
            return SMH_EHIP;
        if (hipStreamSynchronize(s) != hipSuccess) return SMH_EHIP;
        out->nnz = h[0];
        out->S = enc->S;
        out->n_full = (int32_t)h[1];
        out->n_partial = (int32_t)h[2];
        out->n_empty_rows = (int32_t)h[3];
        out->max_row_tiles = (int32_t)h[4];
        out->mask_b = enc->mask_b;
        out->mask_h = enc->mask_h;
        out->n_sparse = (int32_t)h[5];
        out->sparse_nnz = h[6];
        out->row_entries = h[7];
        return SMH_OK;
    } catch (...) {
        return SMH_EHIP;
    }
}

smh_status smh_select_costs(const smh_mask_stats *st, int32_t B, int32_t H,
                            int32_t d, smh_dtype dt, double *t_rowwise_us,
                            double *t_blockwise_us) {
    smh_status s = check_select(st, B, H, d, dt);
    if (s != SMH_OK) return s;
    select_kernel(*st, heads_per_mask(st, B, H), d, dt, t_rowwise_us,
                  t_blockwise_us);
    return SMH_OK;
}

smh_status smh_select_kernel(const smh_mask_stats *st, int32_t B, int32_t H,
                             int32_t d, smh_dtype dt, smh_kernel *out) {
    if (!out) return SMH_EINVAL;
    smh_status s = check_select(st, B, H, d, dt);
    if (s != SMH_OK) return s;
    *out = select_kernel(*st, heads_per_mask(st, B, H), d, dt, nullptr, nullptr);
    return SMH_OK;
}

smh_status smh_sparse_mha_fwd(const void *q, const void *k, const void *v,
                              void *o, int32_t B, int32_t H, int32_t S,
                              int32_t d, smh_dtype in_dt, smh_dtype out_dt,
                              float scale, const smh_mask_enc *enc,
                              smh_kernel which, const smh_mask_stats *st,
                              void *stream) {
    try {
        if (!enc) return SMH_EINVAL;
        if (B < 0 || H < 0 || S < 0 || S > SMH_MAX_S) return SMH_EINVAL;
        if (enc->S != S || enc->n_ot != (S + SMH_OT - 1) / SMH_OT) return SMH_EINVAL;
        if (stack_rows(enc->mask_b, enc->mask_h, S) < 0) return SMH_EINVAL;
        if (d != 64 && d != 128) return SMH_EUNSUPPORTED;
        if (in_dt != SMH_F16 && in_dt != SMH_BF16) return SMH_EUNSUPPORTED;
        if (out_dt != in_dt && out_dt != SMH_F32) return SMH_EUNSUPPORTED;
        if (!isfinite(scale) || scale < 0.f) return SMH_EINVAL;
        if (which != SMH_AUTO && which != SMH_ROWWISE && which != SMH_BLOCKWISE &&
            which != SMH_BLOCKWISE_DENSE)
            return SMH_EINVAL;
        const int64_t BH = (int64_t)B * H;
        if (BH > 0 && !broadcasts(enc->mask_b, enc->mask_h, B, H)) return SMH_EINVAL;
        // grid sizes: one workgroup per (head, outer-tile row) for the
        // block-wise kernel, one wavefront per (head, 8 query rows) for the
        // row-wise kernel
        if (BH * 8 * enc->n_ot > (int64_t)INT32_MAX) return SMH_EINVAL;
        if (which == SMH_AUTO && st) {
            smh_status s2 = check_select(st, B, H, d, in_dt);
            if (s2 != SMH_OK) return s2;
            if (st->S != S || st->mask_b != enc->mask_b ||
                st->mask_h != enc->mask_h)
                return SMH_EINVAL;
        }
        const size_t n_el = (size_t)BH * S * d;
        if (n_el == 0) return SMH_OK;  // nothing to compute
        if (!q || !k || !v || !o) return SMH_EINVAL;
        if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) ||
            !aligned(o, 16))
            return SMH_EINVAL;
        if (!enc->full_row_ptr || !enc->full_col_idx || !enc->part_row_ptr ||
            !enc->part_col_idx || !enc->part_bitmaps || !enc->row_order ||
            !enc->row_info || !enc->part_pop || !enc->row_ent || !enc->row_ent_cnt)
            return SMH_EINVAL;
        const size_t in_b = n_el * 2;
        const size_t out_b = n_el * (out_dt == SMH_F32 ? 4 : 2);
        if (overlaps(o, out_b, q, in_b) || overlaps(o, out_b, k, in_b) ||
            overlaps(o, out_b, v, in_b))
            return SMH_EINVAL;
        const float sc = scale == 0.f ? 1.0f / sqrtf((float)d) : scale;
        const hipStream_t hs = (hipStream_t)stream;
        hipError_t e;
        if (which == SMH_AUTO && !st)  // decided on the device, one launch
            e = launch_auto(q, k, v, o, B, H, S, d, in_dt, out_dt, sc, *enc, hs);
        else {
            if (which == SMH_AUTO)
                which = select_kernel(*st, heads_per_mask(st, B, H), d, in_dt,
                                      nullptr, nullptr);
            if (which == SMH_ROWWISE)
                e = launch_rowwise(q, k, v, o, B, H, S, d, in_dt, out_dt, sc,
                                   *enc, hs);
            else
                e = launch_blockwise(q, k, v, o, B, H, S, d, in_dt, out_dt, sc,
                                     *enc, which != SMH_BLOCKWISE_DENSE, hs);
        }
        return e == hipSuccess ? SMH_OK : SMH_EHIP;
    } catch (...) {
        return SMH_EHIP;
    }
}

smh_status smh_out_proj(const void *o, const void *w, const void *bias,
                        const void *residual, void *out, int32_t B,
                        int32_t H, int32_t S, int32_t d, int32_t D,
                        smh_dtype dt, void *stream) {
    try {
        if (B < 0 || H < 0 || S < 0 || S > SMH_MAX_S) return SMH_EINVAL;
        if (d != 64 && d != 128) return SMH_EUNSUPPORTED;
        if (D <= 0 || D % 64) return SMH_EUNSUPPORTED;
        if (dt != SMH_F16 && dt != SMH_BF16) return SMH_EUNSUPPORTED;
        const int64_t M = (int64_t)B * S, K = (int64_t)H * d;
        if (M > INT32_MAX / 2 || K > INT32_MAX / 2 || M * D > INT64_MAX / 4)
            return SMH_EINVAL;
        if ((M + 63) / 64 > 65535) return SMH_EINVAL;  // grid rows
        if (M == 0) return SMH_OK;
        if (K == 0) return SMH_EINVAL;  // no heads: nothing to project
        if (!o || !w || !out) return SMH_EINVAL;
        if (!aligned(o, 16) || !aligned(w, 16) || !aligned(out, 16) ||
            (bias && !aligned(bias, 16)) || (residual && !aligned(residual, 16)))
            return SMH_EINVAL;
        const size_t ob = (size_t)M * D * 2;
        if (overlaps(out, ob, o, (size_t)M * K * 2) ||
            overlaps(out, ob, w, (size_t)D * K * 2) ||
            (bias && overlaps(out, ob, bias, (size_t)D * 2)) ||
            (residual && residual != out && overlaps(out, ob, residual, ob)))
            return SMH_EINVAL;
        return launch_out_proj(o, w, bias, residual, out, B, H, S, d, D, dt,
                               (hipStream_t)stream) == hipSuccess
                   ? SMH_OK
                   : SMH_EHIP;
    } catch (...) {
        return SMH_EHIP;
    }
}

}  // extern "C"
