// Block-wise kernel: one workgroup per (head, outer-tile row).  The work of
// a workgroup is blockwise_row() in blockwise_body.h.
#include "blockwise_body.h"

namespace smh {
namespace {

template <int D, typename TIn, typename TOut>
__global__ __launch_bounds__(256, D == 64 ? 4 : 2) void blockwise_fwd(FwdArgs<TIn, TOut> a) {
    __shared__ __attribute__((aligned(16))) char k0[Lds<D>::KBUF], k1[Lds<D>::KBUF];
    __shared__ __attribute__((aligned(16))) char v0[Lds<D>::VBUF], v1[Lds<D>::VBUF];
    __shared__ HybLds hl;
    __shared__ __attribute__((aligned(16))) uint32_t e0[4 * 64], e1[4 * 64];
    const TileBufs<D> bufs{{k0, k1}, {v0, v1}, {e0, e1}};
    // heavy rows first, heads in sequence per XCD (slot_at)
    const Slot sl = slot_at(a, (int)blockIdx.x);
    typename Frag<TIn>::type qf[D / 32];
    load_q_frags<D>(a, sl.I, sl.bh, qf);  // before the row summary's round trip
    blockwise_row<D, TIn, TOut>(a, bufs, sl.row, sl.I, sl.bh, load_row_info(a, sl.row), qf, hl);
}

template <int D, typename TIn, typename TOut>
hipError_t launch_d(const void *q, const void *k, const void *v, void *o,
                    int B, int H, int S, float scale, const smh_mask_enc &enc,
                    int hybrid, hipStream_t stream) {
    auto kern = blockwise_fwd<D, TIn, TOut>;
    FwdArgs<TIn, TOut> a = make_args<TIn, TOut>(q, k, v, o, B, H, S, scale, enc);
    a.hybrid = hybrid && hybrid_allowed(S, enc.n_ot);
    const long long slots = (long long)a.R * a.U;  // = n * B * H
    a.use_order = slots > resident_workgroups<blockwise_fwd<D, TIn, TOut>>(0);
    hipLaunchKernelGGL(kern, dim3((unsigned)slots), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_blockwise(const void *q, const void *k, const void *v,
                            void *o, int B, int H, int S, int d, int in_dt,
                            int out_dt, float scale, const smh_mask_enc &enc,
                            int hybrid, hipStream_t stream) {
#define SMH_CASE(D_, TI, TO)                                                  \
    return launch_d<D_, TI, TO>(q, k, v, o, B, H, S, scale, enc, hybrid, stream)
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
