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
//   * partial tiles reset masked scores to -inf from the tile's bitmaps,
//     staged into LDS with the tile; each lane reads the four bytes (one
//     per 16-key sub-tile) that hold its query row's bits;
//   * online softmax in base 2 (running max m and running sum l per query);
//     only the 4 lanes that share a query exchange values (2 shuffles);
//   * O^T += V^T P^T with the same MFMA: P^T is the B operand straight from
//     the score registers (rounded to the input type), V^T the A operand
//     from LDS, so no probability ever goes through LDS, and the O rows a
//     lane holds belong to the same query as its softmax state.
// Epilogue: O / l (0 for a row with no valid key), stored in the output type.
#include "select_model.h"
#include "smh_internal.h"

namespace smh {
namespace {

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef __bf16 b8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));

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

// Row sum of two probabilities already rounded to the input type, exact
// products with 1 accumulated in fp32 (v_dot2).
template <typename T> __device__ inline float sum2(uint32_t pair, float acc);
template <> __device__ inline float sum2<_Float16>(uint32_t pair, float acc) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    h2 x, one = {(_Float16)1.0f, (_Float16)1.0f};
    __builtin_memcpy(&x, &pair, 4);
    return __builtin_amdgcn_fdot2(x, one, acc, false);
}
template <> __device__ inline float sum2<__bf16>(uint32_t pair, float acc) {
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    b2 x, one = {(__bf16)1.0f, (__bf16)1.0f};
    __builtin_memcpy(&x, &pair, 4);
    return __builtin_amdgcn_fdot2_f32_bf16(x, one, acc, false);
}

// Registers that carry one K/V tile (and a partial tile's 64 words) from
// global memory to LDS.
template <int D> struct Staging {
    static constexpr int KCH = 64 * D / 8 / 256;   // 16-byte K chunks/thread
    static constexpr int VT = 32 * (D / 8) / 256;  // V transpose tasks/thread
    u4_t kr[KCH], va[VT], vb[VT];
    uint64_t bw;
};

// Issue the global loads of tile J (K rows contiguous: thread t takes
// 16-byte chunks t, t+256, ...; V: thread t takes keys 2kp, 2kp+1 of
// 8-column chunk dc for the transpose).
template <int D, typename TIn>
__device__ __attribute__((always_inline)) inline void fetch_tile(
    Staging<D> &st, const TIn *__restrict__ Kh, const TIn *__restrict__ Vh,
    int J, const uint64_t *__restrict__ words, int t) {
    const TIn *kt = Kh + (size_t)J * 64 * D;
    const TIn *vt = Vh + (size_t)J * 64 * D;
#pragma unroll
    for (int i = 0; i < Staging<D>::KCH; ++i)
        st.kr[i] = *reinterpret_cast<const u4_t *>(kt + (t + 256 * i) * 8);
#pragma unroll
    for (int i = 0; i < Staging<D>::VT; ++i) {
        const int e = t + 256 * i;
        const int dc = e % (D / 8), kp = e / (D / 8);
        st.va[i] = *reinterpret_cast<const u4_t *>(vt + (2 * kp) * D + 8 * dc);
        st.vb[i] = *reinterpret_cast<const u4_t *>(vt + (2 * kp + 1) * D + 8 * dc);
    }
    if (words && t < 64) st.bw = words[t];
}

// Write a fetched tile into one LDS stage: K row-major (padded rows), V
// transposed (row = output column, keys contiguous), the 64 words raw.
template <int D, typename TIn>
__device__ __attribute__((always_inline)) inline void stage_tile(
    const Staging<D> &st, char *base, bool partial, int t) {
    using L = Lds<D>;
    TIn *ks = reinterpret_cast<TIn *>(base);
    uint32_t *vs = reinterpret_cast<uint32_t *>(ks + L::K_ELEMS);
    uint64_t *wd = reinterpret_cast<uint64_t *>(base + 2 * (L::K_ELEMS + L::V_ELEMS));
#pragma unroll
    for (int i = 0; i < Staging<D>::KCH; ++i) {
        const int e = t + 256 * i;
        const int row = e / (D / 8), col = (e % (D / 8)) * 8;
        *reinterpret_cast<u4_t *>(ks + row * L::KLD + col) = st.kr[i];
    }
#pragma unroll
    for (int i = 0; i < Staging<D>::VT; ++i) {
        const int e = t + 256 * i;
        const int dc = e % (D / 8), kp = e / (D / 8);
        const u4_t a = st.va[i], b = st.vb[i];
        uint32_t *dst = vs + (8 * dc * L::VLD + 2 * kp) / 2;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            // elements 2k, 2k+1 of keys 2kp (low half) and 2kp+1 (high)
            dst[(2 * k) * L::VLD / 2] = (a[k] & 0xFFFFu) | (b[k] << 16);
            dst[(2 * k + 1) * L::VLD / 2] = (a[k] >> 16) | (b[k] & 0xFFFF0000u);
        }
    }
    if (partial && t < 64) wd[t] = st.bw;
}

template <int D, typename TIn, typename TOut>
__global__ __launch_bounds__(256, 2) void blockwise_fwd(
    const TIn *__restrict__ Q, const TIn *__restrict__ K,
    const TIn *__restrict__ V, TOut *__restrict__ O, int S, int BH, float c,
    const int32_t *__restrict__ frp, const int32_t *__restrict__ fci,
    const int32_t *__restrict__ prp, const int32_t *__restrict__ pci,
    const uint64_t *__restrict__ bm, const int32_t *__restrict__ row_order,
    const int64_t *__restrict__ stats, int auto_select) {
    using F = Frag<TIn>;
    using frag = typename F::type;
    using L = Lds<D>;
    extern __shared__ __attribute__((aligned(16))) char smem[];

    // SMH_AUTO without host statistics: run only if the cost model picks
    // this kernel (every workgroup of both launches reaches the same answer)
    if (auto_select &&
        select_on_device(stats, BH, D, __is_same(TIn, __bf16) ? 1 : 0) != 2)
        return;

    // heavy rows first across all heads; one head's rows are BH apart, so
    // with BH % 8 == 0 every workgroup of a head lands on the same XCD.
    const int oi = blockIdx.x / BH;
    const int bh = blockIdx.x - oi * BH;
    const int I = row_order[oi];
    const size_t head = (size_t)bh * S * D;
    const TIn *Qh = Q + head, *Kh = K + head, *Vh = V + head;

    const int t = threadIdx.x, w = t >> 6, l = t & 63;
    const int lq = l & 15, g = l >> 4;
    const int r = 16 * w + lq;  // this lane's query row inside the tile

    const int f0 = frp[I], nF = frp[I + 1] - f0;
    const int p0 = prp[I], nP = prp[I + 1] - p0;
    const int nT = nF + nP;

    // this lane's Q rows as the B operand: query r, d = 32s + 8g + 0..7
    frag qf[D / 32];
    {
        const TIn *qrow = Qh + (size_t)(64 * I + r) * D;
#pragma unroll
        for (int s = 0; s < D / 32; ++s)
            qf[s] = *reinterpret_cast<const frag *>(qrow + 32 * s + 8 * g);
    }

    f4_t acc[D / 16];
#pragma unroll
    for (int i = 0; i < D / 16; ++i) acc[i] = f4_t{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;

    Staging<D> stg;
    stg.bw = 0;
    auto tile_words = [&](int idx) -> const uint64_t * {
        return idx < nF ? nullptr : bm + (size_t)(p0 + idx - nF) * 64;
    };
    auto tile_col = [&](int idx) {
        return idx < nF ? fci[f0 + idx] : pci[p0 + idx - nF];
    };

    if (nT > 0) {
        fetch_tile<D, TIn>(stg, Kh, Vh, tile_col(0), tile_words(0), t);
        stage_tile<D, TIn>(stg, smem, nF == 0, t);
    }
    __syncthreads();

    // per-lane LDS offsets (elements / bytes) shared by both buffers
    const int k_off = lq * L::KLD + 8 * g;
    const int v_off = lq * L::VLD + 4 * g;
    const int b_off = ((r >> 3) * 8 + (g >> 1)) * 8 + (r & 7);
    const int nib = 4 * (g & 1);

    for (int it = 0; it < nT; ++it) {
        const int buf = it & 1;
        const bool partial = it >= nF;
        if (it + 1 < nT)
            fetch_tile<D, TIn>(stg, Kh, Vh, tile_col(it + 1),
                               tile_words(it + 1), t);

        const char *base = smem + buf * L::STAGE_BYTES;
        const TIn *ks = reinterpret_cast<const TIn *>(base) + k_off;
        const TIn *vs = reinterpret_cast<const TIn *>(base) + L::K_ELEMS + v_off;
        const uint8_t *wbytes =
            reinterpret_cast<const uint8_t *>(base + 2 * (L::K_ELEMS + L::V_ELEMS)) + b_off;

        // S^T = K Q^T: four 16-key sub-tiles
        f4_t sc[4];
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            sc[st] = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < D / 32; ++s) {
                const frag a = *reinterpret_cast<const frag *>(
                    ks + 16 * st * L::KLD + 32 * s);
                sc[st] = F::mfma(a, qf[s], sc[st]);
            }
        }
        if (partial) {
            // keys 16st + 4g + i of row r: bits 4(g&1)+i of byte r&7 of
            // inner tile (r>>3, 2st + (g>>1))
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                const uint32_t bits = (uint32_t)wbytes[16 * st] >> nib;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (!((bits >> i) & 1u)) sc[st][i] = -INFINITY;
            }
        }
        float mx = fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3]));
#pragma unroll
        for (int st = 1; st < 4; ++st)
            mx = fmaxf(mx, fmaxf(fmaxf(sc[st][0], sc[st][1]),
                                 fmaxf(sc[st][2], sc[st][3])));
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f((m_run - m_use) * c);
        const float mc = m_use * c;
        m_run = m_new;

        // P^T as B operand: keys 32u + 4g + j (j < 4), 32u + 16 + 4g + j - 4
        frag pf[2];
#pragma unroll
        for (int st = 0; st < 4; ++st)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                pf[st >> 1][(st & 1) * 4 + i] =
                    (TIn)__builtin_amdgcn_exp2f(fmaf(sc[st][i], c, -mc));
        float lsum = 0.f;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            uint32_t pw[4];
            __builtin_memcpy(pw, &pf[u], 16);
#pragma unroll
            for (int j = 0; j < 4; ++j) lsum = sum2<TIn>(pw[j], lsum);
        }
        l_run = l_run * alpha + lsum;
        if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
            for (int i = 0; i < D / 16; ++i) acc[i] *= alpha;
        }

        // O^T += V^T P^T
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                typedef uint32_t u2 __attribute__((ext_vector_type(2)));
                const TIn *vp = vs + 16 * dt * L::VLD + 32 * u;
                const u2 lo = *reinterpret_cast<const u2 *>(vp);
                const u2 hi = *reinterpret_cast<const u2 *>(vp + 16);
                typedef uint32_t u4 __attribute__((ext_vector_type(4)));
                const u4 packed = {lo[0], lo[1], hi[0], hi[1]};
                frag a;
                __builtin_memcpy(&a, &packed, sizeof(a));
                acc[dt] = F::mfma(a, pf[u], acc[dt]);
            }
        }

        if (it + 1 < nT)
            stage_tile<D, TIn>(stg, smem + (buf ^ 1) * L::STAGE_BYTES,
                               it + 1 >= nF, t);
        __syncthreads();
    }

    // epilogue: total l over the 4 lanes of this query
    float lt = l_run;
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    TOut *orow = O + head + (size_t)(64 * I + r) * D;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
        store4<TOut>(orow + 16 * dt + 4 * g, acc[dt] * inv);
}

template <int D, typename TIn, typename TOut>
hipError_t launch_t(const void *q, const void *k, const void *v, void *o,
                    int BH, int S, float scale, const smh_mask_enc &enc,
                    int auto_select, hipStream_t stream) {
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
                       enc.part_bitmaps, enc.row_order, enc.stats, auto_select);
    return hipGetLastError();
}

template <int D, typename TIn>
hipError_t dispatch_out(int out_dt, const void *q, const void *k,
                        const void *v, void *o, int BH, int S, float scale,
                        const smh_mask_enc &enc, int auto_select,
                        hipStream_t stream) {
    if (out_dt == SMH_F32)
        return launch_t<D, TIn, float>(q, k, v, o, BH, S, scale, enc,
                                       auto_select, stream);
    return launch_t<D, TIn, TIn>(q, k, v, o, BH, S, scale, enc, auto_select,
                                 stream);
}

template <int D>
hipError_t dispatch_in(int in_dt, int out_dt, const void *q, const void *k,
                       const void *v, void *o, int BH, int S, float scale,
                       const smh_mask_enc &enc, int auto_select,
                       hipStream_t stream) {
    if (in_dt == SMH_F16)
        return dispatch_out<D, _Float16>(out_dt, q, k, v, o, BH, S, scale, enc,
                                         auto_select, stream);
    return dispatch_out<D, __bf16>(out_dt, q, k, v, o, BH, S, scale, enc,
                                   auto_select, stream);
}

}  // namespace

hipError_t launch_blockwise(const void *q, const void *k, const void *v,
                            void *o, int B, int H, int S, int d, int in_dt,
                            int out_dt, float scale, const smh_mask_enc &enc,
                            int auto_select, hipStream_t stream) {
    const int BH = B * H;
    if (d == 64)
        return dispatch_in<64>(in_dt, out_dt, q, k, v, o, BH, S, scale, enc,
                               auto_select, stream);
    return dispatch_in<128>(in_dt, out_dt, q, k, v, o, BH, S, scale, enc,
                            auto_select, stream);
}

}  // namespace smh
