// Row-wise sparse attention kernel for gfx950.
//
// STOF's kernel for highly sparse, short sequences ("Accelerating Sparse
// Transformer Inference on GPU", gist.science explainer, Technical summary >
// Methodology > 1. Unified MHA module, row-wise kernel item: Q is cut into
// rows, each row is handled with intra-warp exchanges only, and there is no
// synchronisation between warps).
//
// Here the unit is one wavefront (64 lanes) and 8 query rows: the 8 rows of
// one inner-tile row, so that for a partial outer tile the 8 inner-tile
// words (ir, 0..7) hold exactly this row group's mask.  Four independent
// wavefronts share a workgroup only for packing; no s_barrier is ever
// executed and each wavefront uses its own slice of LDS.
// Per outer tile J of the row group's outer-tile row (full tiles, then
// partial tiles):
//   * lane j owns key 64J + j and builds the 8-bit set of rows that may see
//     it (all rows for a full tile, one bit per row from the bitmaps for a
//     partial tile); a lane whose set is empty loads nothing;
//   * scores: lane j reads its K row and dots it with the 8 query rows
//     (fp16/bf16 pairs, fp32 accumulation, v_dot2); masked pairs get -inf;
//   * online softmax per row with a 64-lane max reduction;
//   * P V with lane = output column: the probabilities go through the
//     wavefront's LDS slice, then the wavefront walks only the keys some
//     row can see (the ballot of non-empty lanes) and accumulates p * V.
// Probabilities stay in fp32 in this kernel.
#include "select_model.h"
#include "smh_internal.h"

namespace smh {
namespace {

constexpr int R = 8;  // query rows per wavefront

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef __bf16 b2_t __attribute__((ext_vector_type(2)));

template <typename T> __device__ inline float dot2(uint32_t a, uint32_t b, float c);
template <> __device__ inline float dot2<_Float16>(uint32_t a, uint32_t b, float c) {
    h2_t x, y;
    __builtin_memcpy(&x, &a, 4);
    __builtin_memcpy(&y, &b, 4);
    return __builtin_amdgcn_fdot2(x, y, c, false);
}
template <> __device__ inline float dot2<__bf16>(uint32_t a, uint32_t b, float c) {
    b2_t x, y;
    __builtin_memcpy(&x, &a, 4);
    __builtin_memcpy(&y, &b, 4);
    return __builtin_amdgcn_fdot2_f32_bf16(x, y, c, false);
}

template <typename T> __device__ inline float to_f32(T x) { return (float)x; }

// Orders this wavefront's LDS accesses across lanes: the compiler may not
// move memory operations across it and it waits for outstanding LDS work.
__device__ inline void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ inline float wave_max(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
    return x;
}
__device__ inline float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
    return x;
}

template <typename T, int E> struct Out;
template <int E> struct Out<float, E> {
    static __device__ inline void store(float *p, const float *v) {
#pragma unroll
        for (int e = 0; e < E; ++e) p[e] = v[e];
    }
};
template <int E> struct Out<_Float16, E> {
    static __device__ inline void store(_Float16 *p, const float *v) {
#pragma unroll
        for (int e = 0; e < E; ++e) p[e] = (_Float16)v[e];
    }
};
template <int E> struct Out<__bf16, E> {
    static __device__ inline void store(__bf16 *p, const float *v) {
#pragma unroll
        for (int e = 0; e < E; ++e) p[e] = (__bf16)v[e];
    }
};

template <int D, typename TIn, typename TOut>
__global__ __launch_bounds__(256) void rowwise_fwd(
    const TIn *__restrict__ Q, const TIn *__restrict__ K,
    const TIn *__restrict__ V, TOut *__restrict__ O, int S, int BH,
    long long n_groups, float c, const int32_t *__restrict__ frp,
    const int32_t *__restrict__ fci, const int32_t *__restrict__ prp,
    const int32_t *__restrict__ pci, const uint64_t *__restrict__ bm,
    const int32_t *__restrict__ row_order, const int64_t *__restrict__ stats,
    int auto_select) {
    constexpr int E = D / 64;  // output columns per lane
    __shared__ __attribute__((aligned(16))) float pbuf[4][64][R];
    __shared__ __attribute__((aligned(16))) uint32_t qbuf[4][R][D / 2];

    // SMH_AUTO without host statistics: run only if the cost model picks
    // this kernel (every workgroup of both launches reaches the same answer)
    if (auto_select &&
        select_on_device(stats, BH, D, __is_same(TIn, __bf16) ? 1 : 0) != 1)
        return;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const long long gw = (long long)blockIdx.x * 4 + w;
    if (gw >= n_groups) return;  // whole wavefront leaves; no barriers follow
    // heavy outer-tile rows first, then head, then inner-tile row
    const long long per_oi = (long long)BH * 8;
    const int oi = (int)(gw / per_oi);
    const int rem = (int)(gw - (long long)oi * per_oi);
    const int bh = rem >> 3, ir = rem & 7;
    const int I = row_order[oi];
    const int row0 = 64 * I + 8 * ir;
    const size_t head = (size_t)bh * S * D;
    const TIn *Kh = K + head, *Vh = V + head;

    {  // stage the 8 query rows (contiguous) into this wavefront's slice
        const uint4 *src = reinterpret_cast<const uint4 *>(Q + head + (size_t)row0 * D);
        uint4 *dst = reinterpret_cast<uint4 *>(&qbuf[w][0][0]);
        for (int e = lane; e < R * D / 8; e += 64) dst[e] = src[e];
    }
    wave_lds_sync();

    const int f0 = frp[I], nF = frp[I + 1] - f0;
    const int p0 = prp[I], nP = prp[I + 1] - p0;
    const int nT = nF + nP;

    float m[R], lp[R], o[R][E];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        m[r] = -INFINITY;
        lp[r] = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) o[r][e] = 0.f;
    }

    for (int it = 0; it < nT; ++it) {
        const bool partial = it >= nF;
        const int J = partial ? pci[p0 + it - nF] : fci[f0 + it];
        uint32_t rb = 0xFFu;  // rows that may see key 64J + lane
        if (partial) {
            const uint64_t wd = bm[(size_t)(p0 + it - nF) * 64 + ir * 8 + (lane >> 3)];
            // bit 8r + (lane&7) of the word -> bit r (byte-LSB gather)
            const uint64_t x = (wd >> (lane & 7)) & 0x0101010101010101ull;
            rb = (uint32_t)((x * 0x0102040810204080ull) >> 56);
        }

        float s[R];
#pragma unroll
        for (int r = 0; r < R; ++r) s[r] = 0.f;
        if (rb) {
            const uint4 *krow = reinterpret_cast<const uint4 *>(
                Kh + (size_t)(64 * J + lane) * D);
#pragma unroll 4
            for (int cc = 0; cc < D / 8; ++cc) {
                const uint4 kc = krow[cc];
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const uint4 qc = *reinterpret_cast<const uint4 *>(&qbuf[w][r][4 * cc]);
                    float a = s[r];
                    a = dot2<TIn>(qc.x, kc.x, a);
                    a = dot2<TIn>(qc.y, kc.y, a);
                    a = dot2<TIn>(qc.z, kc.z, a);
                    a = dot2<TIn>(qc.w, kc.w, a);
                    s[r] = a;
                }
            }
        }
        float p[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float sr = (rb >> r) & 1 ? s[r] : -INFINITY;
            const float mx = wave_max(sr);
            const float m_new = fmaxf(m[r], mx);
            const float m_use = m_new == -INFINITY ? 0.f : m_new;
            const float alpha = __builtin_amdgcn_exp2f((m[r] - m_use) * c);
            m[r] = m_new;
            p[r] = __builtin_amdgcn_exp2f(fmaf(sr, c, -m_use * c));
            lp[r] = lp[r] * alpha + p[r];
#pragma unroll
            for (int e = 0; e < E; ++e) o[r][e] *= alpha;
        }
        wave_lds_sync();  // previous tile's readers of pbuf are done
        {
            float4 *dst = reinterpret_cast<float4 *>(&pbuf[w][lane][0]);
            dst[0] = make_float4(p[0], p[1], p[2], p[3]);
            dst[1] = make_float4(p[4], p[5], p[6], p[7]);
        }
        wave_lds_sync();

        uint64_t live = __ballot(rb != 0);
        const TIn *vt = Vh + (size_t)64 * J * D + lane * E;
        while (live) {
            // up to 4 keys per step so their V loads overlap
            int js[4];
            float vv[4][E];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                js[u] = live ? __builtin_ctzll(live) : -1;
                if (live) live &= live - 1;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int e = 0; e < E; ++e)
                    vv[u][e] = js[u] >= 0 ? to_f32(vt[(size_t)js[u] * D + e]) : 0.f;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (js[u] < 0) break;
                const float4 pa = *reinterpret_cast<const float4 *>(&pbuf[w][js[u]][0]);
                const float4 pb = *reinterpret_cast<const float4 *>(&pbuf[w][js[u]][4]);
                const float pr[R] = {pa.x, pa.y, pa.z, pa.w, pb.x, pb.y, pb.z, pb.w};
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int e = 0; e < E; ++e) o[r][e] = fmaf(pr[r], vv[u][e], o[r][e]);
            }
        }
    }

#pragma unroll
    for (int r = 0; r < R; ++r) {
        const float lt = wave_sum(lp[r]);
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
        float out[E];
#pragma unroll
        for (int e = 0; e < E; ++e) out[e] = o[r][e] * inv;
        Out<TOut, E>::store(O + head + (size_t)(row0 + r) * D + lane * E, out);
    }
}

template <int D, typename TIn, typename TOut>
hipError_t launch_t(const void *q, const void *k, const void *v, void *o,
                    int BH, int S, float scale, const smh_mask_enc &enc,
                    int auto_select, hipStream_t stream) {
    const long long n_groups = (long long)BH * (S / 8);
    const unsigned blocks = (unsigned)((n_groups + 3) / 4);
    hipLaunchKernelGGL((rowwise_fwd<D, TIn, TOut>), dim3(blocks), dim3(256), 0,
                       stream, (const TIn *)q, (const TIn *)k, (const TIn *)v,
                       (TOut *)o, S, BH, n_groups, scale * 1.4426950408889634f,
                       enc.full_row_ptr, enc.full_col_idx, enc.part_row_ptr,
                       enc.part_col_idx, enc.part_bitmaps, enc.row_order,
                       enc.stats, auto_select);
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

hipError_t launch_rowwise(const void *q, const void *k, const void *v,
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
