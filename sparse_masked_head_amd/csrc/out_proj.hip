// Output projection of the attention result with bias and residual fused
// into its epilogue:
//   out[b, s, n] = sum_{h, k} O[b, h, s, k] W[n, h*d + k] + bias[n]
//                  + residual[b, s, n]
// The first of the fusion templates that follow MHA in the pages' model
// ("Accelerating Sparse Transformer Inference on GPU", gist.science
// explainer, Technical summary > Methodology > 2. operator fusion: MHA
// output feeding the next dense operator), written by hand here.
//
// A dense contraction, so it runs on the matrix cores: C^T = W A^T with
// v_mfma_f32_16x16x32 (A operand = W rows n, B operand = rows m = (b, s) of
// the head-merged attention output, both contiguous in k), so each lane's
// four accumulators are four consecutive output columns of one row and the
// epilogue reads the residual and writes the output as 8-byte pieces.  The
// head merge is in the loads: a 64-wide k block lies inside one head (d is
// 64 or 128), so row m of the block is 64 contiguous elements of O.
//
// Workgroup: BT x BT outputs (BT = 128, or 64 when the bigger tile would
// leave the chip short of workgroups), 4 wavefronts in 2 x 2, each
// BT/2 x BT/2 (BT/32 x BT/32 MFMA tiles: at BT = 128 one LDS fragment per
// two MFMAs, which LDS bandwidth sustains at the matrix cores' rate); k in
// blocks of 64 staged through two LDS buffers from a ring of P blocks of
// global loads in flight (P = 1: deeper rings measured slower, the extra
// registers costing occupancy).
#include "fwd_common.h"

namespace smh {
namespace {

constexpr int kPK = 64;          // k block
constexpr int kPLD = kPK + 16;   // LDS row stride (elements): 32-byte row shift

template <typename T> struct ProjArgs {
    const T *O, *W, *bias, *res;
    T *out;
    int M, S, H, d, K, N;
};

template <int BT> constexpr int proj_lds_bytes() { return 2 * 2 * BT * kPLD * 2; }

// Address of 16-byte chunk c of the O block (rows m0 .., k0 .. k0+63):
// row c / 8, elements 8 (c % 8); rows past M read row M-1.
template <typename T>
__device__ __attribute__((always_inline)) inline const T *o_chunk(
    const ProjArgs<T> &a, int m0, int k0, int c) {
    const int m = min(m0 + (c >> 3), a.M - 1);
    const int b = m / a.S, s = m - b * a.S;
    const int h = k0 / a.d, kk = k0 - h * a.d + 8 * (c & 7);
    return a.O + (((size_t)b * a.H + h) * a.S + s) * a.d + kk;
}

template <int BT, int P, typename T>
__global__ __launch_bounds__(256) void out_proj(ProjArgs<T> a) {
    using F = Frag<T>;
    using frag = typename F::type;
    constexpr int TW = BT / 32;            // MFMA tiles per wave and side
    constexpr int NC = BT * 8 / 256;       // chunks per thread per operand
    extern __shared__ __attribute__((aligned(16))) char proj_smem[];
    T *lds = reinterpret_cast<T *>(proj_smem);   // [buf][W|O][BT][kPLD]
    auto buf = [&](int b, int op) { return lds + (2 * b + op) * BT * kPLD; };
    const int t = threadIdx.x, w = t >> 6, l = t & 63;
    const int lq = l & 15, g = l >> 4;
    const int n0 = blockIdx.x * BT, m0 = blockIdx.y * BT;
    const int wn = (w & 1) * (BT / 2), wm = (w >> 1) * (BT / 2);

    // register ring: k block j is loaded into slot j % P, P blocks ahead
    u4_t wr[P][NC], orr[P][NC];
    auto load = [&](int slot, int k0) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            const int c = t + 256 * i;
            wr[slot][i] = *reinterpret_cast<const u4_t *>(
                a.W + (size_t)(n0 + (c >> 3)) * a.K + k0 + 8 * (c & 7));
            orr[slot][i] = *reinterpret_cast<const u4_t *>(o_chunk(a, m0, k0, c));
        }
    };
    auto stage = [&](int slot, int b) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            const int c = t + 256 * i;
            const int off = (c >> 3) * kPLD + 8 * (c & 7);
            *reinterpret_cast<u4_t *>(buf(b, 0) + off) = wr[slot][i];
            *reinterpret_cast<u4_t *>(buf(b, 1) + off) = orr[slot][i];
        }
    };

    f4_t acc[TW][TW];
#pragma unroll
    for (int i = 0; i < TW; ++i)
#pragma unroll
        for (int j = 0; j < TW; ++j) acc[i][j] = f4_t{0.f, 0.f, 0.f, 0.f};

    const int nk = a.K / kPK;
#pragma unroll
    for (int j = 0; j < P; ++j)
        if (j < nk) load(j, j * kPK);
    stage(0, 0);
    if (P < nk) load(0, P * kPK);
    __syncthreads();
    // iteration kb: product of block kb (LDS buffer kb & 1), then block
    // kb+1 staged from its slot, which then takes block kb+1+P
    auto iter = [&](int kb, int u) __attribute__((always_inline)) {
        const int cur = kb & 1;
        const T *ws = buf(cur, 0);
        const T *os = buf(cur, 1);
#pragma unroll
        for (int ks = 0; ks < kPK / 32; ++ks) {
            frag fw[TW], fo[TW];
#pragma unroll
            for (int i = 0; i < TW; ++i) {
                fw[i] = *reinterpret_cast<const frag *>(
                    ws + (wn + 16 * i + lq) * kPLD + 32 * ks + 8 * g);
                fo[i] = *reinterpret_cast<const frag *>(
                    os + (wm + 16 * i + lq) * kPLD + 32 * ks + 8 * g);
            }
#pragma unroll
            for (int i = 0; i < TW; ++i)
#pragma unroll
                for (int j = 0; j < TW; ++j)
                    acc[i][j] = F::mfma(fw[i], fo[j], acc[i][j]);
        }
        if (kb + 1 < nk) {
            stage((u + 1) % P, cur ^ 1);  // its buffer was last read at kb-1
            if (kb + 1 + P < nk) load((u + 1) % P, (kb + 1 + P) * kPK);
        }
        __syncthreads();
    };
    for (int kb = 0; kb < nk; kb += P) {
#pragma unroll
        for (int u = 0; u < P; ++u)
            if (kb + u < nk) iter(kb + u, u);
    }

    // epilogue: lane holds out[m][n .. n+3], m = wm + 16j + lq,
    // n = wn + 16i + 4g
#pragma unroll
    for (int j = 0; j < TW; ++j) {
        const int m = m0 + wm + 16 * j + lq;
        if (m >= a.M) continue;
#pragma unroll
        for (int i = 0; i < TW; ++i) {
            const int n = n0 + wn + 16 * i + 4 * g;
            f4_t v = acc[i][j];
            if (a.bias) {
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] += (float)a.bias[n + e];
            }
            if (a.res) {
                const T *r = a.res + (size_t)m * a.N + n;
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] += (float)r[e];
            }
            store4<T>(a.out + (size_t)m * a.N + n, v);
        }
    }
}

template <int BT, int P, typename T>
hipError_t launch_bt(const ProjArgs<T> &a, hipStream_t stream) {
    auto kern = out_proj<BT, P, T>;
    const int lds = proj_lds_bytes<BT>();
    hipError_t e = ensure_lds_limit(kern, lds);
    if (e != hipSuccess) return e;
    dim3 grid((unsigned)(a.N / BT), (unsigned)((a.M + BT - 1) / BT));
    hipLaunchKernelGGL(kern, grid, dim3(256), lds, stream, a);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const void *o, const void *w, const void *bias,
                    const void *res, void *out, int B, int H, int S, int d,
                    int D, hipStream_t stream) {
    ProjArgs<T> a;
    a.O = (const T *)o;
    a.W = (const T *)w;
    a.bias = (const T *)bias;
    a.res = (const T *)res;
    a.out = (T *)out;
    a.M = B * S;
    a.S = S;
    a.H = H;
    a.d = d;
    a.K = H * d;
    a.N = D;
    // the bigger tile when it divides N and still gives every CU a
    // workgroup (measured at M = 4096, N = K = 768: 768 workgroups of
    // 64 x 64 take 15.5 us, 192 of 128 x 128 take 22.4 us)
    const long long big = (long long)((a.M + 127) / 128) * (D / 128);
    if (D % 128 == 0 && big >= 256) return launch_bt<128, 1, T>(a, stream);
    return launch_bt<64, 1, T>(a, stream);
}

}  // namespace

hipError_t launch_out_proj(const void *o, const void *w, const void *bias,
                           const void *res, void *out, int B, int H, int S,
                           int d, int D, int dt, hipStream_t stream) {
    if (dt == SMH_F16)
        return launch_t<_Float16>(o, w, bias, res, out, B, H, S, d, D, stream);
    return launch_t<__bf16>(o, w, bias, res, out, B, H, S, d, D, stream);
}

}  // namespace smh
