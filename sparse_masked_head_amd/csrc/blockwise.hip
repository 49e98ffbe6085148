// Block-wise sparse attention kernel for gfx950 (MFMA).
//
// The general kernel of STOF ("Accelerating Sparse Transformer Inference on
// GPU", gist.science explainer, Technical summary > Methodology > 1. Unified
// MHA module, block-wise kernel item: Q, K and V cut into blocks, staged
// through on-chip memory with copies overlapping compute).  Skipping follows
// the outer-tile item of the same section (tiles absent from the encoding
// are never loaded) and exact masking the inner-tile item (partial tiles are
// masked bit by bit from their 8x8 bitmaps).
//
// One workgroup (4 wavefronts, 256 threads) owns the 64 query rows of one
// outer-tile row I of one (batch, head).  It walks the full tiles of row I,
// then its partial tiles.  Per tile J:
//   * the K tile (row-major) and the V tile (transposed, keys contiguous)
//     sit in LDS, double-buffered: while tile t is computed the global loads
//     of tile t+1 are already in flight into registers and are written to
//     the other LDS buffer afterwards, one barrier per tile;
//   * wavefront w owns queries 16w..16w+15 and computes S^T = K Q^T with
//     v_mfma_f32_16x16x32 (A = K rows from LDS, B = its Q rows held in
//     registers for the whole loop).  In this accumulator layout lane l
//     holds the scores of query l%16 against keys 16t + 4(l/16) + i;
//   * partial tiles reset masked scores to -inf from the tile's bitmaps
//     (staged into LDS as one 64-bit key mask per query row);
//   * online softmax in base 2 (running max m and running sum l per query);
//     only the 4 lanes that share a query exchange values (2 shuffles);
//   * O^T += V^T P^T with the same MFMA: P^T is the B operand straight from
//     the score registers (rounded to the input type), V^T the A operand
//     from LDS, so no probability ever goes through LDS, and the O rows a
//     lane holds belong to the same query as its softmax state.
// Epilogue: O / l (0 for a row with no valid key), stored in the output type.
#include "smh_internal.h"

namespace smh {
namespace {

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef __bf16 b8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));

template <typename T> struct Frag;
template <> struct Frag<_Float16> {
    typedef h8_t type;
    static __device__ inline f4_t mfma(h8_t a, h8_t b, f4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
};
template <> struct Frag<__bf16> {
    typedef b8_t type;
    static __device__ inline f4_t mfma(b8_t a, b8_t b, f4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};

template <typename T> __device__ inline void store4(T *p, f4_t x);
template <> __device__ inline void store4<float>(float *p, f4_t x) {
    *reinterpret_cast<f4_t *>(p) = x;
}
template <> __device__ inline void store4<_Float16>(_Float16 *p, f4_t x) {
    typedef _Float16 h4 __attribute__((ext_vector_type(4)));
    h4 y = {(_Float16)x[0], (_Float16)x[1], (_Float16)x[2], (_Float16)x[3]};
    *reinterpret_cast<h4 *>(p) = y;
}
template <> __device__ inline void store4<__bf16>(__bf16 *p, f4_t x) {
    typedef __bf16 b4 __attribute__((ext_vector_type(4)));
    b4 y = {(__bf16)x[0], (__bf16)x[1], (__bf16)x[2], (__bf16)x[3]};
    *reinterpret_cast<b4 *>(p) = y;
}

constexpr float kLog2e = 1.4426950408889634f;

template <int D> struct Lds {
    static constexpr int KLD = D + 8;     // K row stride (elements)
    static constexpr int VLD = 64 + 4;    // V^T row stride (elements)
    static constexpr int K_ELEMS = 64 * KLD;
    static constexpr int V_ELEMS = D * VLD;
    static constexpr int STAGE_BYTES = 2 * (K_ELEMS + V_ELEMS) + 64 * 8;
};

template <int D, typename TIn, typename TOut>
__global__ __launch_bounds__(256, 2) void blockwise_fwd(
    const TIn *__restrict__ Q, const TIn *__restrict__ K,
    const TIn *__restrict__ V, TOut *__restrict__ O, int S, int BH, float c,
    const int32_t *__restrict__ frp, const int32_t *__restrict__ fci,
    const int32_t *__restrict__ prp, const int32_t *__restrict__ pci,
    const uint64_t *__restrict__ bm, const int32_t *__restrict__ row_order) {
    using F = Frag<TIn>;
    using frag = typename F::type;
    using L = Lds<D>;
    constexpr int KCH = 64 * D / 8 / 256;   // 16-byte K chunks per thread
    constexpr int VT = 32 * (D / 8) / 256;  // V transpose tasks per thread
    extern __shared__ __attribute__((aligned(16))) char smem[];

    // heavy rows first across all heads; one head's rows are BH apart, so
    // with BH % 8 == 0 every workgroup of a head lands on the same XCD.
    const int oi = blockIdx.x / BH;
    const int bh = blockIdx.x - oi * BH;
    const int I = row_order[oi];
    const size_t head = (size_t)bh * S * D;
    const TIn *Qh = Q + head, *Kh = K + head, *Vh = V + head;

    const int t = threadIdx.x, w = t >> 6, l = t & 63;
    const int lq = l & 15, g = l >> 4;

    const int f0 = frp[I], nF = frp[I + 1] - f0;
    const int p0 = prp[I], nP = prp[I + 1] - p0;
    const int nT = nF + nP;

    // this lane's Q rows as the B operand: query lq, d = 32s + 8g + 0..7
    frag qf[D / 32];
    {
        const TIn *qrow = Qh + (size_t)(64 * I + 16 * w + lq) * D;
#pragma unroll
        for (int s = 0; s < D / 32; ++s)
            qf[s] = *reinterpret_cast<const frag *>(qrow + 32 * s + 8 * g);
    }

    f4_t acc[D / 16];
#pragma unroll
    for (int i = 0; i < D / 16; ++i) acc[i] = f4_t{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;

    uint4 kr[KCH], va[VT], vb[VT];
    uint64_t bw = 0;

    auto tile_col = [&](int idx) {
        return idx < nF ? fci[f0 + idx] : pci[p0 + idx - nF];
    };
    auto fetch = [&](int idx) {
        const int J = tile_col(idx);
        const TIn *kt = Kh + (size_t)J * 64 * D;
        const TIn *vt = Vh + (size_t)J * 64 * D;
#pragma unroll
        for (int i = 0; i < KCH; ++i)
            kr[i] = *reinterpret_cast<const uint4 *>(kt + (t + 256 * i) * 8);
#pragma unroll
        for (int i = 0; i < VT; ++i) {
            const int e = t + 256 * i;
            const int dc = e % (D / 8), kp = e / (D / 8);
            va[i] = *reinterpret_cast<const uint4 *>(vt + (2 * kp) * D + 8 * dc);
            vb[i] =
                *reinterpret_cast<const uint4 *>(vt + (2 * kp + 1) * D + 8 * dc);
        }
        if (idx >= nF && t < 64) bw = bm[(size_t)(p0 + idx - nF) * 64 + t];
    };
    auto stage = [&](int buf, bool partial) {
        char *base = smem + buf * L::STAGE_BYTES;
        TIn *ks = reinterpret_cast<TIn *>(base);
        TIn *vs = ks + L::K_ELEMS;
        uint8_t *rm = reinterpret_cast<uint8_t *>(vs + L::V_ELEMS);
#pragma unroll
        for (int i = 0; i < KCH; ++i) {
            const int e = t + 256 * i;
            const int row = e / (D / 8), col = (e % (D / 8)) * 8;
            *reinterpret_cast<uint4 *>(ks + row * L::KLD + col) = kr[i];
        }
#pragma unroll
        for (int i = 0; i < VT; ++i) {
            const int e = t + 256 * i;
            const int dc = e % (D / 8), kp = e / (D / 8);
            const uint32_t a[4] = {va[i].x, va[i].y, va[i].z, va[i].w};
            const uint32_t b[4] = {vb[i].x, vb[i].y, vb[i].z, vb[i].w};
            uint32_t *dst = reinterpret_cast<uint32_t *>(vs);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                // element 2k and 2k+1 of keys 2kp (low half) and 2kp+1
                dst[((8 * dc + 2 * k) * L::VLD + 2 * kp) / 2] =
                    (a[k] & 0xFFFFu) | (b[k] << 16);
                dst[((8 * dc + 2 * k + 1) * L::VLD + 2 * kp) / 2] =
                    (a[k] >> 16) | (b[k] & 0xFFFF0000u);
            }
        }
        if (partial && t < 64) {
            // inner tile ir*8+ic -> byte ic of the key mask of row 8ir+r
            const int ir = t >> 3, ic = t & 7;
#pragma unroll
            for (int r = 0; r < 8; ++r)
                rm[(8 * ir + r) * 8 + ic] = (uint8_t)(bw >> (8 * r));
        }
    };

    if (nT > 0) {
        fetch(0);
        stage(0, nF == 0);
    }
    __syncthreads();

    for (int it = 0; it < nT; ++it) {
        const int buf = it & 1;
        const bool partial = it >= nF;
        if (it + 1 < nT) fetch(it + 1);

        const char *base = smem + buf * L::STAGE_BYTES;
        const TIn *ks = reinterpret_cast<const TIn *>(base);
        const TIn *vs = ks + L::K_ELEMS;
        const uint64_t *rm = reinterpret_cast<const uint64_t *>(vs + L::V_ELEMS);

        // S^T = K Q^T: four 16-key sub-tiles
        f4_t sc[4];
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            sc[st] = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < D / 32; ++s) {
                const frag a = *reinterpret_cast<const frag *>(
                    ks + (16 * st + lq) * L::KLD + 32 * s + 8 * g);
                sc[st] = F::mfma(a, qf[s], sc[st]);
            }
        }
        if (partial) {
            const uint64_t keys = rm[16 * w + lq];
#pragma unroll
            for (int st = 0; st < 4; ++st)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (!((keys >> (16 * st + 4 * g + i)) & 1))
                        sc[st][i] = -INFINITY;
        }
        float mx = sc[0][0];
#pragma unroll
        for (int st = 0; st < 4; ++st)
#pragma unroll
            for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sc[st][i]);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = exp2f((m_run - m_use) * c);
        const float mc = m_use * c;
        m_run = m_new;

        // P^T as B operand: keys 32u + 4g + j (j < 4), 32u + 16 + 4g + j - 4
        frag pf[2];
        float lsum = 0.f;
#pragma unroll
        for (int st = 0; st < 4; ++st)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const TIn p = (TIn)exp2f(fmaf(sc[st][i], c, -mc));
                pf[st >> 1][(st & 1) * 4 + i] = p;
                lsum += (float)p;
            }
        l_run = l_run * alpha + lsum;
#pragma unroll
        for (int i = 0; i < D / 16; ++i) acc[i] *= alpha;

        // O^T += V^T P^T
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
            const TIn *vrow = vs + (16 * dt + lq) * L::VLD;
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                typedef uint32_t u2 __attribute__((ext_vector_type(2)));
                const u2 lo =
                    *reinterpret_cast<const u2 *>(vrow + 32 * u + 4 * g);
                const u2 hi =
                    *reinterpret_cast<const u2 *>(vrow + 32 * u + 16 + 4 * g);
                typedef uint32_t u4 __attribute__((ext_vector_type(4)));
                const u4 packed = {lo[0], lo[1], hi[0], hi[1]};
                frag a;
                __builtin_memcpy(&a, &packed, sizeof(a));
                acc[dt] = F::mfma(a, pf[u], acc[dt]);
            }
        }

        if (it + 1 < nT) stage(buf ^ 1, it + 1 >= nF);
        __syncthreads();
    }

    // epilogue: total l over the 4 lanes of this query
    float lt = l_run;
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    TOut *orow = O + head + (size_t)(64 * I + 16 * w + lq) * D;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
        store4<TOut>(orow + 16 * dt + 4 * g, acc[dt] * inv);
}

template <int D, typename TIn, typename TOut>
hipError_t launch_t(const void *q, const void *k, const void *v, void *o,
                    int BH, int S, float scale, const smh_mask_enc &enc,
                    hipStream_t stream) {
    const int n = enc.n_ot;
    const size_t smem = 2 * Lds<D>::STAGE_BYTES;
    auto kern = blockwise_fwd<D, TIn, TOut>;
    static bool attr_set = false;  // idempotent; races are harmless
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(
            reinterpret_cast<const void *>(kern),
            hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)((size_t)n * BH)), dim3(256), smem,
                       stream, (const TIn *)q, (const TIn *)k, (const TIn *)v,
                       (TOut *)o, S, BH, scale * kLog2e, enc.full_row_ptr,
                       enc.full_col_idx, enc.part_row_ptr, enc.part_col_idx,
                       enc.part_bitmaps, enc.row_order);
    return hipGetLastError();
}

template <int D, typename TIn>
hipError_t dispatch_out(int out_dt, const void *q, const void *k,
                        const void *v, void *o, int BH, int S, float scale,
                        const smh_mask_enc &enc, hipStream_t stream) {
    if (out_dt == SMH_F32)
        return launch_t<D, TIn, float>(q, k, v, o, BH, S, scale, enc, stream);
    return launch_t<D, TIn, TIn>(q, k, v, o, BH, S, scale, enc, stream);
}

template <int D>
hipError_t dispatch_in(int in_dt, int out_dt, const void *q, const void *k,
                       const void *v, void *o, int BH, int S, float scale,
                       const smh_mask_enc &enc, hipStream_t stream) {
    if (in_dt == SMH_F16)
        return dispatch_out<D, _Float16>(out_dt, q, k, v, o, BH, S, scale, enc,
                                         stream);
    return dispatch_out<D, __bf16>(out_dt, q, k, v, o, BH, S, scale, enc,
                                   stream);
}

}  // namespace

hipError_t launch_blockwise(const void *q, const void *k, const void *v,
                            void *o, int B, int H, int S, int d, int in_dt,
                            int out_dt, float scale, const smh_mask_enc &enc,
                            hipStream_t stream) {
    const int BH = B * H;
    if (d == 64)
        return dispatch_in<64>(in_dt, out_dt, q, k, v, o, BH, S, scale, enc,
                               stream);
    return dispatch_in<128>(in_dt, out_dt, q, k, v, o, BH, S, scale, enc,
                            stream);
}

}  // namespace smh
