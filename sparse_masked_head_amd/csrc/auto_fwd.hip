// Fused kernel for SMH_AUTO without host statistics: one launch whose
// workgroups first evaluate the kernel-choice cost model on the statistics
// the encoder wrote (the same function as smh_select_kernel) and then run
// either algorithm.  Grid and workgroup shape are the block-wise kernel's
// (one workgroup per (head, outer-tile row): slot_of), 256 threads; under
// the row-wise choice each of the 4 wavefronts takes inner-tile rows w and
// w+4 of that outer-tile row, independently and without barriers.
#include "blockwise_body.h"
#include "rowwise_body.h"

namespace smh {
namespace {

template <int D, typename TIn, typename TOut>
__global__ __launch_bounds__(256, D == 64 ? 4 : 2) void auto_fwd(FwdArgs<TIn, TOut> a) {
    __shared__ __attribute__((aligned(16))) char k0[Lds<D>::KBUF], k1[Lds<D>::KBUF];
    __shared__ __attribute__((aligned(16))) char v0[Lds<D>::VBUF], v1[Lds<D>::VBUF];
    __shared__ HybLds hl;
    __shared__ __attribute__((aligned(16))) uint32_t e0[4 * 64], e1[4 * 64];
    const Slot sl = slot_at(a, (int)blockIdx.x);
    // the block-wise path's Q rows, requested before the row summary so that
    // they arrive during its round trip (under the row-wise choice the
    // row-wise path reads the same rows again, from the caches)
    typename Frag<TIn>::type qf[D / 32];
    load_q_frags<D>(a, sl.I, sl.bh, qf);
    // the row summary carries the statistics the choice reads (both paths
    // need the summary)
    const RowInfo ri = load_row_info(a, sl.row);
    if (device_choice<D>(a, ri) == 2) {
        const TileBufs<D> bufs{{k0, k1}, {v0, v1}, {e0, e1}};
        blockwise_row<D, TIn, TOut>(a, bufs, sl.row, sl.I, sl.bh, ri, qf, hl);
    } else {
        // each wavefront's slice is one of the tile buffers
        const int w = threadIdx.x >> 6;
        char *slice = w == 0 ? k0 : w == 1 ? k1 : w == 2 ? v0 : v1;
        rowwise_group<D, TIn, TOut>(a, slice, sl.I, w, sl.bh, ri);
        rowwise_group<D, TIn, TOut>(a, slice, sl.I, w + 4, sl.bh, ri);
    }
}

template <int D, typename TIn, typename TOut>
hipError_t launch_d(const void *q, const void *k, const void *v, void *o,
                    int B, int H, int S, float scale, const smh_mask_enc &enc,
                    hipStream_t stream) {
    static_assert(RowLds<D>::BYTES <= Lds<D>::KBUF, "LDS slices");
    auto kern = auto_fwd<D, TIn, TOut>;
    FwdArgs<TIn, TOut> a = make_args<TIn, TOut>(q, k, v, o, B, H, S, scale, enc);
    a.hybrid = hybrid_allowed(S, enc.n_ot);
    const long long slots = (long long)a.R * a.U;  // = n * B * H
    a.use_order = slots > resident_workgroups<auto_fwd<D, TIn, TOut>>(0);
    hipLaunchKernelGGL(kern, dim3((unsigned)slots), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_auto(const void *q, const void *k, const void *v, void *o,
                       int B, int H, int S, int d, int in_dt, int out_dt,
                       float scale, const smh_mask_enc &enc,
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
