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

// Large shapes: 256 x 256 outputs per workgroup of 1024 threads (16
// wavefronts, 4 along n x 4 along m, each 64 x 64: 16 MFMA tiles), k in
// blocks of 32 through a ring of four LDS stages filled straight from global
// memory (global_load_lds_dwordx4, no staging registers), three blocks
// ahead.  A 256 x 256 tile needs half the bytes per flop of a 128 x 128 one:
// at the matrix cores' rate 32 bytes per clock into the CU instead of 64,
// which is all a CU's load path gives.  A stage holds the W block (rows n)
// then the O block (rows m), 64 bytes per row; the 16-byte chunk c of row r
// sits at chunk c ^ ((r >> 2) & 3), so the 16 rows of an operand read fall
// on 16 distinct bank slots.  The four stages are separate LDS objects and
// the k loop is unrolled by four so that each is picked at compile time:
// the loads into one stage then never hold up the reads of another.
constexpr int kGB = 256, kGK = 32;
constexpr int kGOp = kGB * kGK * 2;  // bytes of one operand block
constexpr int kGStage = 2 * kGOp;    // W block, then O block

// p as a wave-uniform value (two v_readfirstlane): the compiler then keeps
// a k block's base in scalar registers and adds each lane's fixed 32-bit
// offset in the load itself, instead of carrying a 64-bit address per lane
// and k block.
__device__ __attribute__((always_inline)) inline const char *uniform_ptr(const char *p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<const char *>(((uint64_t)hi << 32) | lo);
}

// 32-bit LDS address of a pointer into a __shared__ array.
typedef __attribute__((address_space(3))) const char lds_char_t;
__device__ __attribute__((always_inline)) inline uint32_t lds_addr(const char *p) {
    return (uint32_t)(uintptr_t)(lds_char_t *)p;
}

// 16-byte LDS read written out: the compiler does not see it as a read of
// the stage, so it adds no wait of its own for the stage's loads (it cannot
// count them across the k loop and would wait for all of them); the caller
// waits for the results (lds_wait) before using them.
template <int off, typename F>
__device__ __attribute__((always_inline)) inline void lds_read16(F &f, uint32_t addr) {
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(f) : "v"(addr), "i"(off));
}

template <typename T>
__device__ __attribute__((always_inline)) inline void big_load(
    char *stage, const char *wk, const char *ok, uint32_t wo, uint32_t oo, int w) {
    __builtin_amdgcn_global_load_lds((gbl_void_t *)(wk + wo),
                                     (lds_void_t *)(stage + 1024 * w), 16, 0, 0);
    __builtin_amdgcn_global_load_lds((gbl_void_t *)(ok + oo),
                                     (lds_void_t *)(stage + kGOp + 1024 * w), 16, 0, 0);
}

template <int D, typename T>
__global__ __launch_bounds__(1024) void out_proj_big(ProjArgs<T> a) {
    using F = Frag<T>;
    using frag = typename F::type;
    __shared__ __attribute__((aligned(16))) char st0[kGStage], st1[kGStage];
    __shared__ __attribute__((aligned(16))) char st2[kGStage], st3[kGStage];
    const int t = threadIdx.x, l = t & 63;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);
    const int lq = l & 15, g = l >> 4;
    // Tile of this workgroup.  Launch slots go round-robin over the 8 XCDs,
    // each with its own L2: slot i runs on XCD i % 8.  Each XCD gets a
    // contiguous range of tiles in row-grouped order (4 row blocks, then
    // every column block), so that its concurrent workgroups share their O
    // rows and W columns in its L2 instead of every XCD streaming all of O.
    const int mt = (a.M + kGB - 1) / kGB, nt = a.N / kGB;
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
    const int n0 = tn * kGB, m0 = tm * kGB;
    const int wn = 64 * (w & 3), wm = 64 * (w >> 2);

    // loads: wave w fills rows 16w .. 16w+15 of both operand blocks, lane l
    // row 16w + l / 4, chunk position l % 4
    const int row = 16 * w + (l >> 2);
    const int cs = (l & 3) ^ ((row >> 2) & 3);  // the chunk stored there
    const uint32_t wo = 2u * (uint32_t)((size_t)(n0 + row) * a.K + 8 * cs);
    uint32_t oo;
    {
        const int m = min(m0 + row, a.M - 1);  // rows past M read row M-1
        const int b = m / a.S, s = m - b * a.S;
        oo = 2u * (uint32_t)(((size_t)b * a.H * a.S + s) * D + 8 * cs);
    }
    const char *Wb = reinterpret_cast<const char *>(a.W);
    const char *Ob = reinterpret_cast<const char *>(a.O);
    // k block kb: W columns k0 .. k0+31, O head h = k0 / d, columns k0 - h d
    auto wk = [&](int kb) { return uniform_ptr(Wb + 2 * (size_t)kb * kGK); };
    auto ok = [&](int kb) {
        const int k0 = kb * kGK, h = k0 / D;
        return uniform_ptr(Ob + 2 * ((size_t)h * a.S * D + (k0 - h * D)));
    };

    // operand reads: rows wn + 16 i + lq (W) and wm + 16 j + lq (O), chunk
    // g (k = 8g .. 8g+7); the swizzle depends on lq only
    const int sx = (g ^ ((lq >> 2) & 3)) * 16;
    const int rw = (wn + lq) * 64 + sx, ro = kGOp + (wm + lq) * 64 + sx;

    f4_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f4_t{0.f, 0.f, 0.f, 0.f};

    const int nk = a.K / kGK;
    // stage i's buffer, i a compile-time constant
    auto stage = [&](auto ic) -> char * {
        constexpr int i = decltype(ic)::value & 3;
        return i == 0 ? st0 : i == 1 ? st1 : i == 2 ? st2 : st3;
    };
    // nk >= 4 (launch condition).  Every step issues the same two loads, so
    // that the compiler's own wait before the operand reads can count them:
    // past the last block a step reloads the last block into the stage it
    // frees, which nothing reads again.
    big_load<T>(st0, wk(0), ok(0), wo, oo, w);
    big_load<T>(st1, wk(1), ok(1), wo, oo, w);
    big_load<T>(st2, wk(2), ok(2), wo, oo, w);

    auto step = [&](int kb, auto sc) __attribute__((always_inline)) {
        constexpr int S_ = decltype(sc)::value;
        // keep each block's reads and products inside its step (the
        // scheduler would otherwise hoist later blocks' operands and run
        // out of registers)
        __builtin_amdgcn_sched_barrier(0);
        // this wave's loads of block kb are in; the two later blocks'
        // loads stay in flight
        asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
        // every wave's block kb is in, and every wave is done with block
        // kb - 1, whose stage block kb + 3 takes.  A bare s_barrier: the
        // workgroup fence of __syncthreads would wait for the later blocks'
        // loads too.  (Each wave waited above for its own loads of block
        // kb, and its reads of block kb - 1 have returned: its products of
        // that block used them.)
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        const int kn = min(kb + 3, nk - 1);
        big_load<T>(stage(std::integral_constant<int, S_ + 3>()), wk(kn), ok(kn), wo, oo, w);
        const uint32_t aw = lds_addr(stage(std::integral_constant<int, S_>())) + rw;
        const uint32_t ao = aw - rw + ro;
        frag fw[4], fo[4];
        lds_read16<0>(fw[0], aw);
        lds_read16<1024>(fw[1], aw);
        lds_read16<2048>(fw[2], aw);
        lds_read16<3072>(fw[3], aw);
        lds_read16<0>(fo[0], ao);
        lds_read16<1024>(fo[1], ao);
        lds_read16<2048>(fo[2], ao);
        lds_read16<3072>(fo[3], ao);
        // LDS reads return in order: the products of O fragment j start as
        // soon as it is in (after the W fragments), while the later reads
        // are still on their way.  Each wait names the fragments it makes
        // ready, which ties their products to it.
        asm volatile("s_waitcnt lgkmcnt(3)"
                     : "+v"(fw[0]), "+v"(fw[1]), "+v"(fw[2]), "+v"(fw[3]), "+v"(fo[0]));
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i][0] = F::mfma(fw[i], fo[0], acc[i][0]);
        __builtin_amdgcn_sched_barrier(0);  // these products before the next wait
        asm volatile("s_waitcnt lgkmcnt(2)" : "+v"(fo[1]));
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i][1] = F::mfma(fw[i], fo[1], acc[i][1]);
        __builtin_amdgcn_sched_barrier(0);  // these products before the next wait
        asm volatile("s_waitcnt lgkmcnt(1)" : "+v"(fo[2]));
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i][2] = F::mfma(fw[i], fo[2], acc[i][2]);
        __builtin_amdgcn_sched_barrier(0);  // these products before the next wait
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(fo[3]));
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i][3] = F::mfma(fw[i], fo[3], acc[i][3]);
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
    for (int j = 0; j < 4; ++j) {
        const int m = m0 + wm + 16 * j + lq;
        if (m >= a.M) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
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
    // 256 x 256 tiles when they divide N, still give every CU a workgroup,
    // K is a multiple of four k blocks and every byte offset of a lane fits
    // 32 bits
    const long long huge = (long long)((a.M + 255) / 256) * (D / 256);
    if (D % 256 == 0 && huge >= 256 && a.K % (4 * kGK) == 0 &&
        (size_t)a.M * a.K * 2 < (1ull << 32) &&
        (size_t)D * a.K * 2 < (1ull << 32)) {
        dim3 grid((unsigned)((D / 256) * ((a.M + 255) / 256)));
        if (d == 64)
            hipLaunchKernelGGL((out_proj_big<64, T>), grid, dim3(1024), 0, stream, a);
        else
            hipLaunchKernelGGL((out_proj_big<128, T>), grid, dim3(1024), 0, stream, a);
        return hipGetLastError();
    }
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
