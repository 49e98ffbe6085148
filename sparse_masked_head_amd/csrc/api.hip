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

smh_status check_stats(const smh_mask_stats *st) {
    if (!st) return SMH_EINVAL;
    if (st->S < 0 || st->S > SMH_MAX_S) return SMH_EINVAL;
    if (st->S % SMH_OT) return SMH_EUNSUPPORTED;
    const int64_t n = st->S / SMH_OT;
    if (st->n_full < 0 || st->n_partial < 0 || st->nnz < 0 ||
        st->max_row_tiles < 0 || st->n_empty_rows < 0)
        return SMH_EINVAL;
    if ((int64_t)st->n_full + st->n_partial > n * n ||
        st->nnz > (int64_t)st->S * st->S || st->max_row_tiles > n)
        return SMH_EINVAL;
    return SMH_OK;
}

smh_status check_select(const smh_mask_stats *st, int32_t B, int32_t H,
                        int32_t d, smh_dtype dt) {
    smh_status s = check_stats(st);
    if (s != SMH_OK) return s;
    if (B < 0 || H < 0) return SMH_EINVAL;
    if (d != 64 && d != 128) return SMH_EUNSUPPORTED;
    if (dt != SMH_F16 && dt != SMH_BF16) return SMH_EUNSUPPORTED;
    return SMH_OK;
}

}  // namespace

extern "C" {

const char *smh_version(void) { return "smh 0.1 (gfx950)"; }

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

size_t smh_encode_workspace_bytes(int32_t S) {
    if (S < 0 || S > SMH_MAX_S || S % SMH_OT) return 0;
    return enc_layout(S).total;
}

smh_status smh_encode_mask(const uint8_t *mask, int32_t S, void *workspace,
                           size_t ws_bytes, smh_mask_enc *enc_out,
                           void *stream) {
    try {
        if (S < 0 || S > SMH_MAX_S) return SMH_EINVAL;
        if (S % SMH_OT) return SMH_EUNSUPPORTED;
        if (!enc_out || !workspace) return SMH_EINVAL;
        if (S > 0 && (!mask || !aligned(mask, 16))) return SMH_EINVAL;
        if (!aligned(workspace, 256)) return SMH_EINVAL;
        const EncLayout L = enc_layout(S);
        if (ws_bytes < L.total) return SMH_ENOSPACE;
        if (S > 0 && overlaps(mask, (size_t)S * S, workspace, L.total))
            return SMH_EINVAL;
        char *ws = (char *)workspace;
        smh_mask_enc e;
        e.S = S;
        e.n_ot = (int32_t)L.n;
        e.full_row_ptr = (int32_t *)(ws + L.full_row_ptr);
        e.full_col_idx = (int32_t *)(ws + L.full_col_idx);
        e.part_row_ptr = (int32_t *)(ws + L.part_row_ptr);
        e.part_col_idx = (int32_t *)(ws + L.part_col_idx);
        e.part_bitmaps = (uint64_t *)(ws + L.part_bitmaps);
        e.stats = (int64_t *)(ws + L.stats);
        e.row_order = (int32_t *)(ws + L.row_order);
        if (launch_encode(mask, S, ws, L, e, (hipStream_t)stream) !=
            hipSuccess)
            return SMH_EHIP;
        *enc_out = e;
        return SMH_OK;
    } catch (...) {
        return SMH_EHIP;
    }
}

smh_status smh_mask_stats_get(const smh_mask_enc *enc, smh_mask_stats *out,
                              void *stream) {
    try {
        if (!enc || !out || !enc->stats) return SMH_EINVAL;
        int64_t h[5];
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
    select_kernel(*st, (int64_t)B * H, d, dt, t_rowwise_us, t_blockwise_us);
    return SMH_OK;
}

smh_status smh_select_kernel(const smh_mask_stats *st, int32_t B, int32_t H,
                             int32_t d, smh_dtype dt, smh_kernel *out) {
    if (!out) return SMH_EINVAL;
    smh_status s = check_select(st, B, H, d, dt);
    if (s != SMH_OK) return s;
    *out = select_kernel(*st, (int64_t)B * H, d, dt, nullptr, nullptr);
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
        if (S % SMH_OT) return SMH_EUNSUPPORTED;
        if (enc->S != S || enc->n_ot != S / SMH_OT) return SMH_EINVAL;
        if (d != 64 && d != 128) return SMH_EUNSUPPORTED;
        if (in_dt != SMH_F16 && in_dt != SMH_BF16) return SMH_EUNSUPPORTED;
        if (out_dt != in_dt && out_dt != SMH_F32) return SMH_EUNSUPPORTED;
        if (!isfinite(scale) || scale < 0.f) return SMH_EINVAL;
        if (which != SMH_AUTO && which != SMH_ROWWISE && which != SMH_BLOCKWISE)
            return SMH_EINVAL;
        const int64_t BH = (int64_t)B * H;
        // grid sizes: one workgroup per (head, outer-tile row) for the
        // block-wise kernel, one wavefront per (head, 8 query rows) for the
        // row-wise kernel
        if (BH * (S / 8) > (int64_t)INT32_MAX) return SMH_EINVAL;
        if (which == SMH_AUTO && st) {
            smh_status s2 = check_select(st, B, H, d, in_dt);
            if (s2 != SMH_OK) return s2;
            if (st->S != S) return SMH_EINVAL;
        }
        const size_t n_el = (size_t)BH * S * d;
        if (n_el == 0) return SMH_OK;  // nothing to compute
        if (!q || !k || !v || !o) return SMH_EINVAL;
        if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) ||
            !aligned(o, 16))
            return SMH_EINVAL;
        if (!enc->full_row_ptr || !enc->full_col_idx || !enc->part_row_ptr ||
            !enc->part_col_idx || !enc->part_bitmaps || !enc->row_order)
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
                which = select_kernel(*st, BH, d, in_dt, nullptr, nullptr);
            if (which == SMH_ROWWISE)
                e = launch_rowwise(q, k, v, o, B, H, S, d, in_dt, out_dt, sc,
                                   *enc, hs);
            else
                e = launch_blockwise(q, k, v, o, B, H, S, d, in_dt, out_dt, sc,
                                     *enc, hs);
        }
        return e == hipSuccess ? SMH_OK : SMH_EHIP;
    } catch (...) {
        return SMH_EHIP;
    }
}

}  // extern "C"
