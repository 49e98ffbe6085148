// Types and helpers shared by the attention kernels of libsmh (gfx950).
#pragma once

#include <atomic>

#include "bits.h"
#include "select_model.h"
#include "smh_internal.h"

namespace smh {

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef __bf16 b8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u2_t __attribute__((ext_vector_type(2)));
typedef short s4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s4_t lds_s4_t;
// p as a wave-uniform value (two v_readfirstlane; p must be the same in
// every lane): the compiler then keeps such a base in scalar registers and
// adds each lane's fixed 32-bit offset in the load itself, instead of
// carrying a 64-bit address per lane and load.
template <typename P>
__device__ __attribute__((always_inline)) inline P *uniform_ptr(P *p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<P *>(((uint64_t)hi << 32) | lo);
}

// pointer types of the load-to-LDS builtin (global source, LDS destination)
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void gbl_void_t;

constexpr float kLog2e = 1.4426950408889634f;

// Everything an attention kernel reads: the tensors of one call and the
// encoding of its mask stack.  c = scale * log2(e) (scores are
// exponentiated in base 2).
template <typename TIn, typename TOut> struct FwdArgs {
    const TIn *Q, *K, *V;
    TOut *O;
    int S, BH, H;
    int n;       // outer tiles per side, ceil(S / 64)
    int R;       // rows of the encoding: masks * n
    int U;       // (batch, head) pairs per mask: BH / masks
    int mask_b, mask_h;
    float c;
    // 1: visit the encoding's rows in row_order (heavy first); 0: in index
    // order, used when every workgroup of the launch is resident at once
    // and the order cannot matter (saves a dependent load per workgroup)
    int use_order;
    // 1: launch slots go to XCDs head by head (slot_at); needs U % 8 == 0
    int xcd_seq;
    const int32_t *frp, *fci, *prp, *pci;
    const uint64_t *bm;
    const int32_t *row_order;
    const int32_t *info;  // row_info [R][16]
    const int64_t *stats;
    const int32_t *pop;   // part_pop: valid elements of each partial tile
    const uint32_t *rent; // row-wise entries of the sparse tiles (row_ent)
    const int32_t *rcnt;  // their counts per (row, 16-row group)
    // 1: the block-wise algorithm computes sparse partial tiles (at most
    // SMH_SPARSE_TILE_MAX valid elements) on its gather path; set only when
    // every key fits 16 bits (S <= 65536)
    int hybrid;
};

// A row's summary (row_info): where its full and partial lists start, their
// lengths, the columns of its first four stored tiles (full, then partial)
// and the encoding's statistics.  One scalar load, so that a kernel has its
// kernel choice and the K and V addresses of its first tiles one memory
// round trip after it starts.
struct RowInfo {
    int f0, nF, p0, nP;
    int c[4];
    // nnz, n_full, n_partial, (unused), max_row_tiles, n_sparse, row_entries
    int64_t stats[7];
};
template <typename TIn, typename TOut>
__device__ inline RowInfo load_row_info(const FwdArgs<TIn, TOut> &a, int row) {
    const int4 *p = reinterpret_cast<const int4 *>(a.info + 16 * (size_t)row);
    const int4 h = p[0], c = p[1], s = p[2], m = p[3];
    return RowInfo{h.x, h.y, h.z, h.w, {c.x, c.y, c.z, c.w},
                   {(int64_t)(((uint64_t)(uint32_t)s.y << 32) | (uint32_t)s.x),
                    s.z, s.w, 0, m.x, m.y,
                    (int64_t)(((uint64_t)(uint32_t)m.w << 32) | (uint32_t)m.z)}};
}

template <typename TIn, typename TOut>
inline FwdArgs<TIn, TOut> make_args(const void *q, const void *k,
                                    const void *v, void *o, int B, int H,
                                    int S, float scale,
                                    const smh_mask_enc &enc) {
    FwdArgs<TIn, TOut> a;
    a.Q = (const TIn *)q;
    a.K = (const TIn *)k;
    a.V = (const TIn *)v;
    a.O = (TOut *)o;
    a.S = S;
    a.BH = B * H;
    a.H = H;
    a.n = enc.n_ot;
    a.mask_b = enc.mask_b;
    a.mask_h = enc.mask_h;
    a.R = enc.mask_b * enc.mask_h * enc.n_ot;
    a.U = (enc.mask_b > 1 ? 1 : B) * (enc.mask_h > 1 ? 1 : H);
    a.c = scale * kLog2e;
    a.use_order = 1;
    a.xcd_seq = a.U % 8 == 0;
    a.frp = enc.full_row_ptr;
    a.fci = enc.full_col_idx;
    a.prp = enc.part_row_ptr;
    a.pci = enc.part_col_idx;
    a.bm = enc.part_bitmaps;
    a.row_order = enc.row_order;
    a.info = enc.row_info;
    a.stats = enc.stats;
    a.pop = enc.part_pop;
    a.rent = enc.row_ent;
    a.rcnt = enc.row_ent_cnt;
    a.hybrid = 0;
    return a;
}

// What one launch slot works on.  Slots are (encoding row, user) pairs,
// slot = oi * U + user: oi walks the encoding's rows (heavy first when
// use_order), user walks the U (batch, head) pairs that share the row's
// mask.  A head's slots are U apart, so with U % 8 == 0 they all land on
// one XCD (slots go round-robin over the 8 XCDs).
struct Slot {
    int row;  // row of the encoding: mask g, outer-tile row I
    int I;    // outer-tile row inside the mask
    int bh;   // b * H + h
};
template <typename TIn, typename TOut>
__device__ inline Slot slot_of(const FwdArgs<TIn, TOut> &a, int oi, int user) {
    Slot sl;
    sl.row = a.use_order ? a.row_order[oi] : oi;
    const int g = sl.row / a.n;
    sl.I = sl.row - g * a.n;
    // mask g = gb * mask_h + gh; users of g: b in {gb} or all B, h in {gh}
    // or all H (a broadcast side of size 1 spans every index)
    const int Hu = a.mask_h > 1 ? 1 : a.H;
    const int b = a.mask_b > 1 ? g / a.mask_h : user / Hu;
    const int h = a.mask_h > 1 ? g - (g / a.mask_h) * a.mask_h : user - (user / Hu) * Hu;
    sl.bh = b * a.H + h;
    return sl;
}

// The slot of launch index b.  Workgroups go round-robin over the 8 XCDs
// (b % 8), each XCD with its own L2.  Plain order (slot b = oi * U + user)
// keeps a head on one XCD when U % 8 == 0 but runs U / 8 heads on it at
// once; with xcd_seq the k-th workgroup of XCD x (b = 8k + x) takes head
// slot hs = k / R and row position oi = k % R, user = x + 8 hs, so an XCD
// works through its heads one after another (heavy rows first within each)
// and its L2 holds one head's K and V at a time.
template <typename TIn, typename TOut>
__device__ inline Slot slot_at(const FwdArgs<TIn, TOut> &a, int b) {
    if (a.xcd_seq) {
        const int k = b >> 3, x = b & 7;
        const int hs = k / a.R;
        return slot_of(a, k - hs * a.R, x + 8 * hs);
    }
    const int oi = b / a.U;
    return slot_of(a, oi, b - oi * a.U);
}

template <typename T> constexpr int is_bf16() { return __is_same(T, __bf16) ? 1 : 0; }

// MFMA 16x16x32 with fp32 accumulation for the two input types.
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

// Packed pair dot product with fp32 accumulation (v_dot2).
template <typename T> __device__ inline float dot2(uint32_t a, uint32_t b, float c);
template <> __device__ inline float dot2<_Float16>(uint32_t a, uint32_t b, float c) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    h2 x, y;
    __builtin_memcpy(&x, &a, 4);
    __builtin_memcpy(&y, &b, 4);
    return __builtin_amdgcn_fdot2(x, y, c, false);
}
template <> __device__ inline float dot2<__bf16>(uint32_t a, uint32_t b, float c) {
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    b2 x, y;
    __builtin_memcpy(&x, &a, 4);
    __builtin_memcpy(&y, &b, 4);
    return __builtin_amdgcn_fdot2_f32_bf16(x, y, c, false);
}
// Sum of a pair already in the input type: exact products with 1, fp32 sum.
template <typename T> __device__ inline uint32_t ones2();
template <> __device__ inline uint32_t ones2<_Float16>() { return 0x3C003C00u; }
template <> __device__ inline uint32_t ones2<__bf16>() { return 0x3F803F80u; }
template <typename T> __device__ inline float sum2(uint32_t pair, float acc) {
    return dot2<T>(pair, ones2<T>(), acc);
}

// Two fp32 values rounded (to nearest even) to T, packed (a in the low
// half): one packed conversion instruction.
template <typename T> __device__ inline uint32_t pack2(float a, float b) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef T t2 __attribute__((ext_vector_type(2)));
    const t2 v = __builtin_convertvector(f2{a, b}, t2);
    uint32_t r;
    __builtin_memcpy(&r, &v, 4);
    return r;
}

// Four fp32 values to the output type, one store.
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

// Max / sum of x over lanes l and l^16 (then l^32) with the gfx950 row
// swaps: swapping odd rows of one copy with even rows of the other leaves
// the two partners' values side by side in every lane.
// (The max is v_max_f32 written out: fmaxf on values from a lane swap
// makes the compiler quiet possible signalling NaNs first, two more
// instructions; no such NaN occurs here.)
__device__ inline float vmax(float a, float b) {
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}
__device__ inline float max_xor16(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float max_xor32(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float sum_xor16(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ inline float sum_xor32(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Orders one wavefront's LDS accesses across its lanes: no memory operation
// moves across it and outstanding LDS work is waited for.
__device__ inline void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Raise kernel Kern's dynamic-LDS limit once per device (the attribute is
// per device; repeated calls are cheap but are kept out of the launch path
// so that launches can be captured into graphs).  The kernel is a template
// argument so that each kernel has a cache of its own (instances of one
// kernel template share a function type).
template <auto Kern>
inline hipError_t ensure_lds_limit(int bytes) {
    static std::atomic<int> done[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < 64 && done[dev].load(std::memory_order_acquire) >= bytes)
        return hipSuccess;
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(Kern),
                            hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess && dev >= 0 && dev < 64)
        done[dev].store(bytes, std::memory_order_release);
    return e;
}

// Workgroups of kernel Kern (256 threads, `lds` bytes of dynamic LDS) that
// the current device holds at once; cached per kernel and device (a
// template argument, as for ensure_lds_limit).
template <auto Kern>
inline long long resident_workgroups(int lds) {
    static std::atomic<long long> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    long long v = cache[dev].load(std::memory_order_acquire);
    if (v > 0) return v;
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, reinterpret_cast<const void *>(Kern), 256, lds) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
            hipSuccess)
        return 0;
    v = (long long)per_cu * cus;
    cache[dev].store(v, std::memory_order_release);
    return v;
}

// The launch's kernel choice when decided on the device: 1 row-wise,
// 2 block-wise (same function as smh_select_kernel on the host).
template <int D, typename TIn, typename TOut>
__device__ inline int device_choice(const FwdArgs<TIn, TOut> &a, const RowInfo &ri) {
    return select_on_device(ri.stats, a.U, a.R, D, is_bf16<TIn>());
}

}  // namespace smh
