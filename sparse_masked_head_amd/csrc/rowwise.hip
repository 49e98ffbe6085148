// Row-wise kernel: one wavefront per (head, 8 query rows); four independent
// wavefronts per workgroup only for packing.  The work of a wavefront is
// rowwise_group() in rowwise_body.h.
#include "rowwise_body.h"

namespace smh {
namespace {

template <int D, typename TIn, typename TOut>
__global__ __launch_bounds__(256, D == 64 ? 4 : 3) void rowwise_fwd(
    FwdArgs<TIn, TOut> a, long long n_groups) {
    __shared__ __attribute__((aligned(16))) char lds[4 * RowLds<D>::BYTES];
    const int w = threadIdx.x >> 6;
    const long long gw = (long long)blockIdx.x * 4 + w;
    if (gw >= n_groups) return;  // the whole wavefront leaves; no barriers
    // heavy encoding rows first, then the row's heads (slot_of), then
    // inner-tile row
    const long long per_oi = (long long)a.U * 8;
    const int oi = (int)(gw / per_oi);
    const int rem = (int)(gw - (long long)oi * per_oi);
    const Slot sl = slot_of(a, oi, rem >> 3);
    rowwise_group<D, TIn, TOut>(a, lds + w * RowLds<D>::BYTES, sl.I, rem & 7,
                                sl.bh, load_row_info(a, sl.row));
}

template <int D, typename TIn, typename TOut>
hipError_t launch_d(const void *q, const void *k, const void *v, void *o,
                    int B, int H, int S, float scale, const smh_mask_enc &enc,
                    hipStream_t stream) {
    FwdArgs<TIn, TOut> a = make_args<TIn, TOut>(q, k, v, o, B, H, S, scale, enc);
    const long long n_groups = (long long)a.R * a.U * 8;  // = 8 n B H
    hipLaunchKernelGGL((rowwise_fwd<D, TIn, TOut>),
                       dim3((unsigned)((n_groups + 3) / 4)), dim3(256), 0,
                       stream, a, n_groups);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_rowwise(const void *q, const void *k, const void *v,
                          void *o, int B, int H, int S, int d, int in_dt,
                          int out_dt, float scale, const smh_mask_enc &enc,
                          hipStream_t stream) {
#define SMH_CASE(D_, TI, TO)                                                  \
    return launch_d<D_, TI, TO>(q, k, v, o, B, H, S, scale, enc, stream)
    if (d == 64) {
        if (in_dt == SMH_F16) {
            if (out_dt == SMH_F32) SMH_CASE(64, _Float16, float);
            SMH_CASE(64, _Float16, _Float16);
        }
        if (out_dt == SMH_F32) SMH_CASE(64, __bf16, float);
        SMH_CASE(64, __bf16, __bf16);
    }
    if (in_dt == SMH_F16) {
        if (out_dt == SMH_F32) SMH_CASE(128, _Float16, float);
        SMH_CASE(128, _Float16, _Float16);
    }
    if (out_dt == SMH_F32) SMH_CASE(128, __bf16, float);
    SMH_CASE(128, __bf16, __bf16);
#undef SMH_CASE
}

}  // namespace smh
