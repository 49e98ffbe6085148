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
#include <type_traits>

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

// Load-to-LDS ring kernel: BT x BT outputs per workgroup of NW wavefronts
// (BT = 256: 16 wavefronts in 4 x 4, each 64 x 64; BT = 128: 4 in 2 x 2,
// 64 x 64; BT = 64: 4 in 2 x 2, 32 x 32), k in blocks of 32 through a ring
// of four LDS stages filled straight from global memory
// (global_load_lds_dwordx4, no staging registers), three blocks ahead.  The
// bigger the tile, the fewer bytes per flop: at the matrix cores' rate a
// 256 x 256 tile needs 32 bytes per clock into the CU, a 128 x 128 one 64,
// which is all a CU's load path gives.  A stage holds the W block (rows n)
// then the O block (rows m), 64 bytes per row; the 16-byte chunk c of row r
// sits at chunk c ^ ((r >> 2) & 3), so the 16 rows of an operand read fall
// on 16 distinct bank slots.  The four stages are separate LDS objects and
// the k loop is unrolled by four so that each is picked at compile time:
// the loads into one stage then never hold up the reads of another.
constexpr int kGK = 32;

// 32-bit LDS address of a pointer into a __shared__ array.
typedef __attribute__((address_space(3))) const char lds_char_t;
__device__ __attribute__((always_inline)) inline uint32_t lds_addr(const char *p) {
    return (uint32_t)(uintptr_t)(lds_char_t *)p;
}

// 16-byte LDS read written out: the compiler does not see it as a read of
// the stage, so it adds no wait of its own for the stage's loads (it cannot
// count them across the k loop and would wait for all of them); the caller
// waits for the results before using them.
template <int off, typename F>
__device__ __attribute__((always_inline)) inline void lds_read16(F &f, uint32_t addr) {
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(f) : "v"(addr), "i"(off));
}

// Wait until at most n of this wave's LDS reads are outstanding.
template <int n> __device__ __attribute__((always_inline)) inline void lds_wait_asm();
#define SMH_LGKM(n)                                                      \
    template <> __device__ __attribute__((always_inline)) inline void   \
    lds_wait_asm<n>() { asm volatile("s_waitcnt lgkmcnt(" #n ")" ::: "memory"); }
SMH_LGKM(0) SMH_LGKM(1) SMH_LGKM(2) SMH_LGKM(3)
#undef SMH_LGKM

template <int BT, int NW> struct Ring {
    static constexpr int OP = BT * kGK * 2;           // bytes of one operand block
    static constexpr int STAGE = 2 * OP;              // W block, then O block
    static constexpr int LPW = BT / 16 / NW;          // 1 KB loads per wave and operand
    static constexpr int WSIDE = NW == 16 ? 4 : 2;    // wavefronts per side
    static constexpr int WT = BT / WSIDE;             // wavefront tile side
    static constexpr int TW = WT / 16;                // MFMA tiles per side
};

template <int BT, int NW, int D, typename T>
__global__ __launch_bounds__(NW * 64) void out_proj_ring(ProjArgs<T> a) {
    using F = Frag<T>;
    using frag = typename F::type;
    using R = Ring<BT, NW>;
    constexpr int TW = R::TW, LPW = R::LPW;
    __shared__ __attribute__((aligned(16))) char st0[R::STAGE], st1[R::STAGE];
    __shared__ __attribute__((aligned(16))) char st2[R::STAGE], st3[R::STAGE];
    const int t = threadIdx.x, l = t & 63;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);
    const int lq = l & 15, g = l >> 4;
    // Tile of this workgroup.  Launch slots go round-robin over the 8 XCDs,
    // each with its own L2: slot i runs on XCD i % 8.  Each XCD gets a
    // contiguous range of tiles in row-grouped order (4 row blocks, then
    // every column block), so that its concurrent workgroups share their O
    // rows and W columns in its L2 instead of every XCD streaming all of O.
    const int mt = (a.M + BT - 1) / BT, nt = a.N / BT;
    int tm, tn;
    {
        const int nt_all = mt * nt, i = blockIdx.x;
        const int v = nt_all % 8 == 0 ? (i % 8) * (nt_all / 8) + i / 8 : i;
        constexpr int kGroup = 4;
        const int per = kGroup * nt, first = (v / per) * kGroup;
        const int gs = min(mt - first, kGroup), r = v - (v / per) * per;
        tm = first + r % gs;
        tn = r / gs;
    }
    const int n0 = tn * BT, m0 = tm * BT;
    const int wn = R::WT * (w % R::WSIDE), wm = R::WT * (w / R::WSIDE);

    // loads: wave w's instruction i fills rows 16 (LPW w + i) .. +15 of both
    // operand blocks, lane l row 16 (LPW w + i) + l / 4, chunk position l % 4
    uint32_t wo[LPW], oo[LPW];
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
        const int row = 16 * (LPW * w + i) + (l >> 2);
        const int cs = (l & 3) ^ ((row >> 2) & 3);  // the chunk stored there
        wo[i] = 2u * (uint32_t)((size_t)(n0 + row) * a.K + 8 * cs);
        const int m = min(m0 + row, a.M - 1);  // rows past M read row M-1
        const int b = m / a.S, s = m - b * a.S;
        oo[i] = 2u * (uint32_t)(((size_t)b * a.H * a.S + s) * D + 8 * cs);
    }
    const char *Wb = reinterpret_cast<const char *>(a.W);
    const char *Ob = reinterpret_cast<const char *>(a.O);
    // k block kb: W columns k0 .. k0+31, O head h = k0 / d, columns k0 - h d
    auto wk = [&](int kb) { return uniform_ptr(Wb + 2 * (size_t)kb * kGK); };
    auto ok = [&](int kb) {
        const int k0 = kb * kGK, h = k0 / D;
        return uniform_ptr(Ob + 2 * ((size_t)h * a.S * D + (k0 - h * D)));
    };
    auto load = [&](char *stage, int kb) __attribute__((always_inline)) {
        const char *wp = wk(kb), *op = ok(kb);
#pragma unroll
        for (int i = 0; i < LPW; ++i) {
            __builtin_amdgcn_global_load_lds((gbl_void_t *)(wp + wo[i]),
                                             (lds_void_t *)(stage + 1024 * (LPW * w + i)),
                                             16, 0, 0);
            __builtin_amdgcn_global_load_lds((gbl_void_t *)(op + oo[i]),
                                             (lds_void_t *)(stage + R::OP + 1024 * (LPW * w + i)),
                                             16, 0, 0);
        }
    };

    // operand reads: rows wn + 16 i + lq (W) and wm + 16 j + lq (O), chunk
    // g (k = 8g .. 8g+7); the swizzle depends on lq only
    const int sx = (g ^ ((lq >> 2) & 3)) * 16;
    const int rw = (wn + lq) * 64 + sx, ro = R::OP + (wm + lq) * 64 + sx;

    f4_t acc[TW][TW];
#pragma unroll
    for (int i = 0; i < TW; ++i)
#pragma unroll
        for (int j = 0; j < TW; ++j) acc[i][j] = f4_t{0.f, 0.f, 0.f, 0.f};

    const int nk = a.K / kGK;
    // stage i's buffer, i a compile-time constant
    auto stage = [&](auto ic) -> char * {
        constexpr int i = decltype(ic)::value & 3;
        return i == 0 ? st0 : i == 1 ? st1 : i == 2 ? st2 : st3;
    };
    // nk is a multiple of 4 (launch condition).  Every step issues the same
    // loads, so that the count of each wait is fixed: past the last block a
    // step reloads the last block into the stage it frees, which nothing
    // reads again.
    load(st0, 0);
    load(st1, 1);
    load(st2, 2);

    auto step = [&](int kb, auto sc) __attribute__((always_inline)) {
        constexpr int S_ = decltype(sc)::value;
        // keep each block's reads and products inside its step (the
        // scheduler would otherwise hoist later blocks' operands)
        __builtin_amdgcn_sched_barrier(0);
        // this wave's loads of block kb are in; the two later blocks'
        // loads (2 LPW each) stay in flight
        if constexpr (LPW == 1)
            asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
        else
            asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
        // every wave's block kb is in, and every wave is done with block
        // kb - 1, whose stage block kb + 3 takes.  A bare s_barrier: the
        // workgroup fence of __syncthreads would wait for the later blocks'
        // loads too.  (Each wave waited above for its own loads of block
        // kb, and its reads of block kb - 1 have returned: its products of
        // that block used them.)
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        load(stage(std::integral_constant<int, S_ + 3>()), min(kb + 3, nk - 1));
        const uint32_t aw = lds_addr(stage(std::integral_constant<int, S_>())) + rw;
        const uint32_t ao = aw - rw + ro;
        frag fw[TW], fo[TW];
        lds_read16<0>(fw[0], aw);
        lds_read16<1024>(fw[1], aw);
        if constexpr (TW == 4) {
            lds_read16<2048>(fw[2], aw);
            lds_read16<3072>(fw[3], aw);
        }
        lds_read16<0>(fo[0], ao);
        lds_read16<1024>(fo[1], ao);
        if constexpr (TW == 4) {
            lds_read16<2048>(fo[2], ao);
            lds_read16<3072>(fo[3], ao);
        }
        // LDS reads return in order: the products of O fragment j start as
        // soon as it is in (after the W fragments), while the later reads
        // are still on their way.  The "+v" operands tie each fragment's
        // products to its wait.
#pragma unroll
        for (int j = 0; j < TW; ++j) {
            if (j == 0) {
                lds_wait_asm<TW - 1>();
#pragma unroll
                for (int i = 0; i < TW; ++i) asm volatile("" : "+v"(fw[i]));
            } else if (j == 1) {
                lds_wait_asm<TW - 2>();
            } else if (j == 2) {
                lds_wait_asm<(TW > 2 ? TW - 3 : 0)>();
            } else {
                lds_wait_asm<0>();
            }
            asm volatile("" : "+v"(fo[j]));
#pragma unroll
            for (int i = 0; i < TW; ++i) acc[i][j] = F::mfma(fw[i], fo[j], acc[i][j]);
            __builtin_amdgcn_sched_barrier(0);  // these products before the next wait
        }
    };
    for (int kb = 0; kb < nk; kb += 4) {  // nk % 4 == 0 (launch condition)
        step(kb, std::integral_constant<int, 0>());
        step(kb + 1, std::integral_constant<int, 1>());
        step(kb + 2, std::integral_constant<int, 2>());
        step(kb + 3, std::integral_constant<int, 3>());
    }
    // the last steps' loads (re-reads of the last block) land before the
    // workgroup's LDS is released
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

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

template <int BT, int NW, typename T>
hipError_t launch_ring(const ProjArgs<T> &a, hipStream_t stream) {
    dim3 grid((unsigned)((a.N / BT) * ((a.M + BT - 1) / BT)));
    if (a.d == 64)
        hipLaunchKernelGGL((out_proj_ring<BT, NW, 64, T>), grid, dim3(NW * 64), 0, stream, a);
    else
        hipLaunchKernelGGL((out_proj_ring<BT, NW, 128, T>), grid, dim3(NW * 64), 0, stream, a);
    return hipGetLastError();
}

template <int BT, int P, typename T>
hipError_t launch_bt(const ProjArgs<T> &a, hipStream_t stream) {
    auto kern = out_proj<BT, P, T>;
    const int lds = proj_lds_bytes<BT>();
    hipError_t e = ensure_lds_limit<out_proj<BT, P, T>>(lds);
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
    // The ring kernel when K is a multiple of four k blocks and every byte
    // offset of a lane fits 32 bits: 256 x 256 tiles when they divide N and
    // still give every CU a workgroup, else 128 x 128 on the same terms,
    // else 64 x 64.
    if (a.K % (4 * kGK) == 0 && (size_t)a.M * a.K * 2 < (1ull << 32) &&
        (size_t)D * a.K * 2 < (1ull << 32)) {
        const long long t256 = (long long)((a.M + 255) / 256) * (D / 256);
        const long long t128 = (long long)((a.M + 127) / 128) * (D / 128);
        if (D % 256 == 0 && t256 >= 256) return launch_ring<256, 16, T>(a, stream);
        if (D % 128 == 0 && t128 >= 256) return launch_ring<128, 4, T>(a, stream);
        return launch_ring<64, 4, T>(a, stream);
    }
    // else the register-staged kernel: the bigger tile when it divides N and
    // still gives every CU a workgroup (measured at M = 4096, N = K = 768:
    // 768 workgroups of 64 x 64 take 15.5 us, 192 of 128 x 128 take 22.4 us)
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
