// Block-wise sparse attention: the work of one workgroup (256 threads, one
// outer-tile row of one head), used by the block-wise kernel and by the
// fused kernel that decides on the device.
//
// The general kernel of STOF ("Accelerating Sparse Transformer Inference on
// GPU", gist.science explainer, Technical summary > Methodology > 1. Unified
// MHA module, block-wise kernel item: Q, K and V cut into blocks, staged
// through on-chip memory with copies overlapping compute).  Skipping follows
// the outer-tile item of the same section (tiles absent from the encoding
// are never loaded) and exact masking the inner-tile item (partial tiles are
// masked bit by bit from their 8x8 bitmaps).
//
// The workgroup owns the 64 query rows of outer-tile row I of head bh and
// walks the full tiles of the row, then its partial tiles.  Per tile J:
//   * K and V sit row-major in separate LDS double buffers, 16-byte chunks
//     XOR-swizzled within each row (no padding), filled straight from
//     global memory by global_load_lds_dwordx4 (no staging registers, no
//     LDS write instructions); the transpose that V^T needs is done by
//     ds_read_b64_tr_b16 when the P V operand is read.  K is loaded two
//     tiles ahead of its use and V one, each into the buffer the previous
//     barrier freed, so iteration t issues the QK^T MFMAs of tile t+1
//     before the softmax of tile t and the matrix cores work while the VALU
//     does the softmax; one barrier per tile, before which every wave waits
//     for its own loads;
//   * wavefront w owns queries 16w..16w+15 and computes S^T = K Q^T with
//     v_mfma_f32_16x16x32 (A = K rows from LDS, B = its Q rows held in
//     registers for the whole row).  In this accumulator layout lane l holds
//     query l%16's scores against keys 16st + 4(l/16) + i;
//   * partial tiles get -inf for masked scores: each lane loads from the
//     tile's 64 words the four bytes (one per 16-key sub-tile) that hold
//     its query row's bits, together with the K tile, carries them in a
//     register, and starts the tile's QK^T accumulators at 0 / -inf from
//     them, so the masking costs two VALU operations per score;
//   * online softmax in base 2 (running max and sum per query) with lazy
//     rescaling (the reference max moves only when passed by more than 8
//     in exponent units); only the 4 lanes sharing a query exchange values
//     (two gfx950 row swaps);
//   * O^T += V^T P^T with the same MFMA: P^T is the B operand straight from
//     the score registers rounded to the input type, V^T the A operand from
//     LDS; the O rows a lane holds belong to the query whose softmax state
//     it holds, so rescaling is lane-local.
// Epilogue: O / l (0 for a row with no valid key), stored in the output type.
#pragma once

#include <type_traits>

#include "fwd_common.h"

namespace smh {

template <int D> struct Lds {
    // A tile is 64 rows of D elements = CPR 16-byte chunks per row, no
    // padding.  Chunk c of row r sits at chunk position c ^ sw(r) of the
    // row.  The 64 banks span 256 bytes: one row at d = 128, two at d = 64.
    // sw puts both read patterns on distinct 16-byte bank slots: a K
    // operand read (16 consecutive rows, one chunk: sw distinct over them,
    // within each row parity at d = 64) and the V^T reads of two lane
    // groups (8 consecutive rows, chunks 2dt and 2dt+1: sw >> 1 distinct
    // over them, within each row parity at d = 64).  sw depends on row % 16
    // only.
    static constexpr int CPR = D / 8;
    static constexpr int KBUF = 64 * D * 2;
    static constexpr int VBUF = 64 * D * 2;
    static __device__ int sw(int row) {
        return CPR == 16 ? (((row & 7) << 1) | ((row >> 3) & 1))
                         : ((((row >> 1) & 3) << 1) | ((row >> 3) & 1));
    }
    // byte offset of chunk c of row r inside a tile buffer
    static __device__ int chunk_off(int r, int c) {
        return (r * CPR + (c ^ sw(r))) * 16;
    }
};

// One tile (K or V) of 64 rows from global memory into a tile buffer with
// global_load_lds_dwordx4: wave w's instruction i fills chunk positions
// 64 (4i + w) .. +63 (1 KB, lane l the position 64 (4i + w) + l) and each
// lane reads the global chunk that belongs there.  The lane's byte offsets
// inside a tile are fixed (TileOffs); a tile adds only its base address,
// which is the same for the whole wave.  A chunk at a byte offset above
// `lim` is read from `lim` instead, so that the rows of a tile cut by S come
// from inside the tensor: they are masked (K) or multiplied by a zero
// probability (V), and any finite value serves.  The data lands
// asynchronously: the loads count in vmcnt.
template <int D> struct TileOffs {
    uint32_t off[D / 32];  // byte offset of this lane's chunk i in the tile
};
template <int D> __device__ inline TileOffs<D> tile_offsets(int w, int l) {
    using L = Lds<D>;
    TileOffs<D> o;
#pragma unroll
    for (int i = 0; i < L::CPR / 4; ++i) {
        const int pos = 64 * (4 * i + w) + l;  // chunk position in the buffer
        const int r = pos / L::CPR, c = (pos % L::CPR) ^ L::sw(r);
        o.off[i] = 2u * (uint32_t)(r * D + 8 * c);
    }
    return o;
}
template <int D>
__device__ __attribute__((always_inline)) inline void load_tile(
    char *buf, const char *tile, uint32_t lim, const TileOffs<D> &to, int w) {
    using L = Lds<D>;
#pragma unroll
    for (int i = 0; i < L::CPR / 4; ++i)
        __builtin_amdgcn_global_load_lds((gbl_void_t *)(tile + min(to.off[i], lim)),
                                         (lds_void_t *)(buf + 1024 * (4 * i + w)),
                                         16, 0, 0);
}

// The chunks load_tile would bring in for this lane, into registers
// instead (ordinary global loads, which the compiler waits for before the
// registers are used), and their later store to the chunk positions
// load_tile fills.
template <int D> struct TileRegs {
    u4_t c[D / 32];
};
template <int D>
__device__ __attribute__((always_inline)) inline void load_tile_regs(
    TileRegs<D> &rg, const char *tile, uint32_t lim, const TileOffs<D> &to) {
    typedef __attribute__((address_space(1))) const u4_t gbl_u4_t;
#pragma unroll
    for (int i = 0; i < D / 32; ++i)
        rg.c[i] = *(gbl_u4_t *)(tile + min(to.off[i], lim));
}
template <int D>
__device__ __attribute__((always_inline)) inline void store_tile_regs(
    char *buf, const TileRegs<D> &rg, int w, int l) {
#pragma unroll
    for (int i = 0; i < D / 32; ++i)
        *reinterpret_cast<u4_t *>(buf + 1024 * (4 * i + w) + 16 * l) = rg.c[i];
}

// This lane's mask bytes of a partial tile (global loads into registers):
// keys 16st + 4g + i of query row r are bits 4(g&1)+i of byte r&7 of inner
// tile (r>>3, 2st + (g>>1)); b_off is that byte's offset for st = 0, each
// further st is two words (16 bytes) on.
struct MaskRegs {
    uint32_t mb[4];
};
__device__ __attribute__((always_inline)) inline void load_mask(
    MaskRegs &m, const uint64_t *__restrict__ words, int b_off) {
    if (words) {
        const uint8_t *wb = reinterpret_cast<const uint8_t *>(words) + b_off;
#pragma unroll
        for (int st = 0; st < 4; ++st) m.mb[st] = wb[16 * st];
    }
}

// The same four loads from `src` (the lane's first mask byte, or any
// readable address when the bytes are not used), issued unconditionally.
__device__ __attribute__((always_inline)) inline void load_mask_at(
    MaskRegs &m, const uint8_t *src) {
#pragma unroll
    for (int st = 0; st < 4; ++st) m.mb[st] = src[16 * st];
}

// The lane's mask bits of a partial tile: bit 8st + i (i < 4) = key
// 16st + 4g + i of its query row (nib = 4(g&1)); the other bits are not
// used.
__device__ __attribute__((always_inline)) inline uint32_t mask_bits(
    const MaskRegs &m, int nib) {
    return (m.mb[0] | (m.mb[1] << 8) | (m.mb[2] << 16) | (m.mb[3] << 24)) >> nib;
}

// Bit `off` of x as 0 or -1 (v_bfe_i32; written out so that the compiler
// keeps this one-instruction form instead of a compare and a select).
template <int off> __device__ __attribute__((always_inline)) inline int bit_mask(int x) {
    int r;
    asm("v_bfe_i32 %0, %1, %2, 1" : "=v"(r) : "v"(x), "i"(off));
    return r;
}

// Wait for this wave's outstanding global loads (the tile loads into LDS
// among them), before the barrier that hands their buffers to every wave.
__device__ __attribute__((always_inline)) inline void wait_loads() {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}
// Wait until at most N (< 64) of this wave's global loads are outstanding.
// The builtin rather than inline assembly, so that the compiler knows those
// loads are complete and adds no wait of its own before their data is used.
// Encoding: vmcnt bits 3:0 and 15:14; expcnt (6:4) and lgkmcnt (11:8) at
// their maxima, i.e. not waited for.
template <int N> __device__ __attribute__((always_inline)) inline void wait_loads_but() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// s_barrier without the workgroup fence of __syncthreads (which would also
// wait for every global load still in flight).
__device__ __attribute__((always_inline)) inline void bare_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Running state of one lane: O^T accumulators of its query (d = 16dt +
// 4(l/16) + i), running max (raw score units) and its part of the sum.
template <int D> struct RowState {
    f4_t acc[D / 16];
    float m, l;
    float mc;  // m * c, or 0 while m is -inf (the exponent offset)
};

// S^T = K Q^T for one tile (four 16-key sub-tiles), raw scores.  For a
// partial tile the accumulators start at 0 for a valid key and -inf for a
// masked one (mbits: bit 8st + i = key 16st + 4g + i is valid), so masked
// scores leave the matrix cores as -inf and the softmax needs no masking.
// The two cases are separate code so that a full tile's first products
// take the constant zero accumulator.
// This lane's byte offsets into a K buffer for the A operand of S^T = K Q^T:
// row 16st + lq (st added by the caller), chunk 4s + g, s < D/32.
template <int D> struct KOff {
    int base;          // row lq
    int x[D / 32];     // swizzled chunk position of chunk 4s + g, times 16
};
template <int D> __device__ inline KOff<D> k_offsets(int lq, int g) {
    using L = Lds<D>;
    KOff<D> o;
    o.base = lq * L::CPR * 16;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) o.x[s] = ((4 * s + g) ^ L::sw(lq)) * 16;
    return o;
}

template <int D, typename TIn, bool kPartial>
__device__ __attribute__((always_inline)) inline void qk_tile_k(
    f4_t (&sc)[4], const typename Frag<TIn>::type (&qf)[D / 32],
    const char *kb, const KOff<D> &ko, uint32_t mbits) {
    using F = Frag<TIn>;
    using frag = typename F::type;
    const char *ks = kb + ko.base;
    const int inv = (int)~mbits;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
        f4_t c0 = f4_t{0.f, 0.f, 0.f, 0.f};
        if (kPartial)  // all ones where masked -> the bits of -inf
            c0 = f4_t{__int_as_float(bit_mask<0>(inv >> (8 * st)) & (int)0xFF800000u),
                      __int_as_float(bit_mask<1>(inv >> (8 * st)) & (int)0xFF800000u),
                      __int_as_float(bit_mask<2>(inv >> (8 * st)) & (int)0xFF800000u),
                      __int_as_float(bit_mask<3>(inv >> (8 * st)) & (int)0xFF800000u)};
        const char *row = ks + 16 * st * Lds<D>::CPR * 16;
        const frag a0 = *reinterpret_cast<const frag *>(row + ko.x[0]);
        sc[st] = F::mfma(a0, qf[0], c0);
#pragma unroll
        for (int s = 1; s < D / 32; ++s) {
            const frag a = *reinterpret_cast<const frag *>(row + ko.x[s]);
            sc[st] = F::mfma(a, qf[s], sc[st]);
        }
    }
}

template <int D, typename TIn>
__device__ __attribute__((always_inline)) inline void qk_tile(
    f4_t (&sc)[4], const typename Frag<TIn>::type (&qf)[D / 32],
    const char *kb, const KOff<D> &ko, bool partial, uint32_t mbits) {
    if (partial)
        qk_tile_k<D, TIn, true>(sc, qf, kb, ko, mbits);
    else
        qk_tile_k<D, TIn, false>(sc, qf, kb, ko, mbits);
}

// This lane's byte offsets into a V buffer for the transposing reads of
// V^T: key row 32u + 4g + (lq >> 2) (+16 for the upper slots; u added by
// the caller), elements 16dt + 4 (lq & 3) .. +3, i.e. half (lq & 1) of
// chunk 2dt + ((lq & 3) >> 1).  The swizzle of those rows does not depend
// on u or the +16.
template <int D> struct VOff {
    // byte offset of row 4g + (lq >> 2), half-chunk lq & 1, swizzled
    // chunk 2dt + ((lq & 3) >> 1); a buffer address plus a constant row
    // offset completes the address
    int x[D / 16];
};
template <int D> __device__ inline VOff<D> v_offsets(int lq, int g) {
    using L = Lds<D>;
    VOff<D> o;
    const int r = 4 * g + (lq >> 2);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
        o.x[dt] = r * L::CPR * 16 + 8 * (lq & 1) +
                  ((2 * dt + ((lq & 3) >> 1)) ^ L::sw(r)) * 16;
    return o;
}

// Softmax of the scores of NST 16-key sub-tiles (masked ones already -inf;
// NST = 4 for an outer tile, 2 for a gathered chunk of 32 keys) and
// O^T += V^T P^T with V's rows in a tile-buffer layout.  c = scale *
// log2(e) > 0.  kWaitV: wait for this wave's outstanding loads (the V rows
// it staged itself) before the first V read.
template <int D, typename TIn, int NST = 4, bool kWaitV = false>
__device__ __attribute__((always_inline)) inline void softmax_pv(
    RowState<D> &rs, f4_t (&sc)[NST], const char *vb, float c, const VOff<D> &vo) {
    using F = Frag<TIn>;
    using frag = typename F::type;
    using L = Lds<D>;
    float mx = -INFINITY;
#pragma unroll
    for (int st = 0; st < NST; ++st) {
        mx = fmaxf(fmaxf(mx, sc[st][0]), sc[st][1]);
        mx = fmaxf(fmaxf(mx, sc[st][2]), sc[st][3]);
    }
    mx = max_xor32(max_xor16(mx));
    // Lazy rescaling: the reference max rs.m moves only when a score passes
    // it by more than 8 in base-2 exponent units, so most tiles skip the
    // rescale; the probabilities then stay below 2^8 (well inside the input
    // type's range) and the final division by l cancels the reference.
    // (mx - m) * c is NaN (no move) when both are -inf, +inf when only m is.
    const bool grow = (mx - rs.m) * c > 8.f;
    if (__builtin_amdgcn_ballot_w64(grow)) {
        const float m_new = grow ? mx : rs.m;
        const float alpha = grow ? __builtin_amdgcn_exp2f((rs.m - m_new) * c) : 1.f;
        rs.m = m_new;
        rs.mc = grow ? mx * c : rs.mc;  // a growing max is finite
        rs.l *= alpha;
#pragma unroll
        for (int i = 0; i < D / 16; ++i) rs.acc[i] *= alpha;
    }
    const float mc = rs.mc;

    // P^T as B operand: keys 32u + 4g + j (j < 4), 32u + 16 + 4g + j - 4
    constexpr int NU = NST / 2;
    frag pf[NU];
#pragma unroll
    for (int st = 0; st < NST; ++st)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            pf[st >> 1][(st & 1) * 4 + i] =
                (TIn)__builtin_amdgcn_exp2f(fmaf(sc[st][i], c, -mc));
    float lsum = rs.l;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        uint32_t pw[4];
        __builtin_memcpy(pw, &pf[u], 16);
#pragma unroll
        for (int j = 0; j < 4; ++j) lsum = sum2<TIn>(pw[j], lsum);
    }
    rs.l = lsum;

    // A operand V^T (rows = output columns 16dt + l%16, slots = keys of
    // the P^T slots) read with ds_read_b64_tr_b16 from row-major V: within
    // each 16-lane group, lane j = a + 4q points at V[key0 + q][d0 + 4a]
    // and lane i receives V[key0 .. key0+3][d0 + i]; key0 = 32u + 4g for
    // slots 0..3 and 32u + 16 + 4g for slots 4..7.  vo holds the lane's
    // (q, a) offsets in the swizzled buffer.
    if (kWaitV) wait_loads();
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const char *p0 = vb + vo.x[dt] + 32 * u * L::CPR * 16;
            const char *p1 = p0 + 16 * L::CPR * 16;
            const s4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s4_t *)(p0));
            const s4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s4_t *)(p1));
            frag a;
            __builtin_memcpy(&a, &lo, 8);
            __builtin_memcpy(reinterpret_cast<char *>(&a) + 8, &hi, 8);
            rs.acc[dt] = F::mfma(a, pf[u], rs.acc[dt]);
        }
    }
}

// The stored tiles of one outer-tile row: full tiles first, then partial.
// Columns are clamped to [0, n): an encoding that is not this library's
// then gives wrong numbers, never an access outside K and V.  The columns
// of the first four tiles come with the row summary; the tile loop reads
// each later column one step before it needs it (a column read in the step
// that uses it would put a memory round trip in front of every tile load).
// With `dl` set (a row split by split_partials), the partial tiles the
// loop visits are the dense ones of the LDS list instead of the row's
// whole partial list.
struct TileList {
    const int32_t *fci, *pci;
    const uint64_t *bm;
    const uint32_t *dl;  // LDS: column << 16 | index in the row's partial list
    int f0, nF, p0, nT, nmax, S;
    __device__ int clamp(int J) const { return (int)min((unsigned)J, (unsigned)nmax); }
    // column of stored tile idx (full tiles first); a load from memory
    // (or LDS) that the caller issues a step before it needs the value
    __device__ int col_of(int idx) const {
        if (idx < nF) return fci[f0 + idx];
        return dl ? (int)(dl[idx - nF] >> 16) : pci[p0 + idx - nF];
    }
    // last in-bounds 16-byte chunk offset (bytes) of tile J (S cuts the last tile)
    template <int D> __device__ uint32_t lim(int J) const {
        return 2u * (uint32_t)(min(64, S - 64 * J) * D - 8);
    }
    __device__ const uint64_t *words(int idx) const {
        if (idx < nF) return nullptr;
        const int k = dl ? (int)(dl[idx - nF] & 0xFFFFu) : idx - nF;
        return bm + (size_t)(p0 + k) * 64;
    }
};

// Most outer tiles per side for which the block-wise algorithm splits rows
// into dense and sparse partial tiles (S <= 65536: keys fit 16 bits).
constexpr int kHybMaxN = 1024;

// LDS of the split: the row's partial tiles, dense ones first, each
// column << 16 | index in the row's partial list, and per-wavefront counts.
struct HybLds {
    uint32_t list[kHybMaxN];
    int wcnt[16];
};

// The split of an outer-tile row's partial tiles (whole workgroup, two
// barriers): list[0 .. nD) the dense ones (more than SMH_SPARSE_TILE_MAX
// valid elements), list[nD .. nP) the sparse ones, each in ascending column
// order.  Returns nD.  Requires nP <= kHybMaxN.
template <typename TIn, typename TOut>
__device__ inline int split_partials(const FwdArgs<TIn, TOut> &a, const RowInfo &ri,
                                     HybLds &hl) {
    constexpr int kPer = kHybMaxN / 256;
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int nP = ri.nP, nk = (nP + 255) >> 8;
    int popv[kPer], colv[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {  // every load in flight at once
        const int idx = 256 * k + t;
        const bool v = k < nk && idx < nP;
        popv[k] = v ? a.pop[ri.p0 + idx] : SMH_SPARSE_TILE_MAX + 1;
        colv[k] = v ? a.pci[ri.p0 + idx] : 0;
    }
    uint64_t dmask[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const bool dense = 256 * k + t < nP && popv[k] > SMH_SPARSE_TILE_MAX;
        dmask[k] = __builtin_amdgcn_ballot_w64(dense);
        if (lane == 0) hl.wcnt[4 * k + w] = __popcll(dmask[k]);
    }
    __syncthreads();
    int nD = 0, before[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        before[k] = nD;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int x = hl.wcnt[4 * k + q];
            before[k] += q < w ? x : 0;
            nD += x;
        }
    }
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int idx = 256 * k + t;
        if (idx < nP) {
            const int drank = before[k] +
                (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(dmask[k] >> 32),
                                               __builtin_amdgcn_mbcnt_lo((uint32_t)dmask[k], 0u));
            const bool dense = (dmask[k] >> lane) & 1ull;
            const int at = dense ? drank : nD + idx - drank;
            hl.list[at] = ((uint32_t)colv[k] << 16) | (uint32_t)idx;
        }
    }
    __syncthreads();
    return nD;
}

// Workgroup work: encoding row `row` (outer-tile row I of its mask, summary
// ri) of head bh.
// The four tile buffers (K0, K1, V0, V1) are separate LDS objects, and
// the tile loop picks them at compile time, so that the compiler can tell
// the loads filling one buffer from the reads of another and does not make
// those reads wait for the loads.
template <int D> struct TileBufs {
    char *k[2], *v[2];
};

// This lane's Q rows as the B operand of S^T = K Q^T for outer-tile row I
// of head bh: query 64I + 16w + l%16, d = 32s + 8(l/16) + 0..7 (a query
// past S, in a tile cut by S, reads query S-1 and is not stored).  Needs
// only the slot, not the row summary, so a kernel issues these loads before
// it reads the summary and they overlap its round trip.
template <int D, typename TIn, typename TOut>
__device__ __attribute__((always_inline)) inline void load_q_frags(
    const FwdArgs<TIn, TOut> &a, int I, int bh,
    typename Frag<TIn>::type (&qf)[D / 32]) {
    using frag = typename Frag<TIn>::type;
    const int t = threadIdx.x, l = t & 63;
    const int qi = 64 * I + 16 * (t >> 6) + (l & 15);
    const TIn *qrow = a.Q + (size_t)bh * a.S * D + (size_t)min(qi, a.S - 1) * D;
#pragma unroll
    for (int s = 0; s < D / 32; ++s)
        qf[s] = *reinterpret_cast<const frag *>(qrow + 32 * s + 8 * (l >> 4));
}

// ---- gather path of sparse partial tiles (per wavefront, no barrier) ----
//
// The row-wise side of the per-tile dispatch: a partial tile with few valid
// elements would cost a dense tile's work on the matrix cores, so each
// wavefront instead streams the row-wise entries of its 16 query rows (the
// keys some of them see in the row's sparse tiles, with their row sets;
// built once per mask by the encoder) and computes them in chunks of 32
// keys with the same MFMA layout and online-softmax state as the tile path.
// Pipeline, at chunk c: the entries of chunk c + 2 are requested (one
// register: lane l holds entry l % 32); chunk c + 1's K rows go into one of
// two register sets and its V rows (global_load_lds) into one of two V
// slots, chunk-swizzled like a tile buffer so that the tile path's V^T
// reads serve, its keys and row sets taken from its entry register with
// ds_bpermute; then chunk c is computed.  The V slots of chunks c and c + 1
// lie in different LDS objects (the K tile buffers, the V tile buffers),
// so the V^T reads of one do not wait for the loads landing in the other.
// Loads past the list re-read its last entry (or key 0), so every wait
// counts the same loads.

// One chunk in registers: K rows as A operands (entries 16st + lq, st =
// 0, 1; d = 32s + 8g .. +7) and the lane's score slots that are valid (bit
// 4st + i: entry 16st + 4g + i is in the chunk and its row set holds the
// lane's query row).
template <int D, typename TIn> struct ChunkK {
    typename Frag<TIn>::type k[2][D / 32];
    uint32_t ok;
};

template <int D, typename TIn>
__device__ __attribute__((always_inline)) inline void gather_stream(
    RowState<D> &rs, char *vslot0, char *vslot1, const uint32_t *__restrict__ ents,
    int ne, const typename Frag<TIn>::type (&qf)[D / 32], const TIn *__restrict__ Kh,
    const TIn *__restrict__ Vh, float c, int S, const VOff<D> &vo) {
    using F = Frag<TIn>;
    using L = Lds<D>;
    const int lane = threadIdx.x & 63, lq = lane & 15, g = lane >> 4;
    constexpr int RPI = 1024 / (2 * D);  // V rows per 1 KB load instruction
    constexpr int NV = 32 / RPI;         // V instructions per chunk
    constexpr int NK = 2 * (D / 32);     // K loads per chunk
    const int nch = (ne + 31) >> 5;
    // the key of entry ei of a chunk of n entries, clamped into the head's
    // rows; past the chunk: key 0
    auto key_of = [&](int ei, int n, uint32_t e) __attribute__((always_inline)) {
        return ei < n ? min((int)(e & 0xFFFFu), S - 1) : 0;
    };
    auto load_e = [&](int ci) __attribute__((always_inline)) {
        return ents[min(32 * ci + (lane & 31), ne - 1)];
    };
    auto issue = [&](int ci, uint32_t e, char *vs, ChunkK<D, TIn> &ck)
        __attribute__((always_inline)) {
        // entry idx of the chunk, from lane idx of the entry register
        auto ent = [&](int idx) __attribute__((always_inline)) {
            return (uint32_t)__builtin_amdgcn_ds_bpermute(idx << 2, (int)e);
        };
        const int n = min(32, ne - 32 * ci);
        uint32_t ok = 0;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int rr = RPI * i + lane / L::CPR, cp = lane % L::CPR;
            const int key = key_of(rr, n, ent(rr));
            __builtin_amdgcn_global_load_lds(
                (gbl_void_t *)(Vh + (size_t)key * D + 8 * (cp ^ L::sw(rr))),
                (lds_void_t *)(vs + 1024 * i), 16, 0, 0);
        }
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            const typename F::type *krow = reinterpret_cast<const typename F::type *>(
                Kh + (size_t)key_of(16 * st + lq, n, ent(16 * st + lq)) * D);
#pragma unroll
            for (int s2 = 0; s2 < D / 32; ++s2) ck.k[st][s2] = krow[4 * s2 + g];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t e2 = ent(16 * st + 4 * g + i);
                ok |= (uint32_t)(16 * st + 4 * g + i < n && ((e2 >> (16 + lq)) & 1u))
                      << (4 * st + i);
            }
        }
        ck.ok = ok;
    };
    auto compute = [&](const char *vs, const ChunkK<D, TIn> &ck)
        __attribute__((always_inline)) {
        f4_t sc[2];
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            f4_t c0;
#pragma unroll
            for (int i = 0; i < 4; ++i) c0[i] = (ck.ok >> (4 * st + i)) & 1u ? 0.f : -INFINITY;
            sc[st] = F::mfma(ck.k[st][0], qf[0], c0);
#pragma unroll
            for (int s2 = 1; s2 < D / 32; ++s2) sc[st] = F::mfma(ck.k[st][s2], qf[s2], sc[st]);
        }
        softmax_pv<D, TIn, 2>(rs, sc, vs, c, vo);
    };
    if (nch == 0) return;
    ChunkK<D, TIn> ka, kb;
    uint32_t ea = load_e(0), eb = load_e(1);
    issue(0, ea, vslot0, ka);
    // chunk ci: registers `cur`, V slot vc; chunk ci + 1: entries in `en`,
    // goes to `nxt` and vn; the entries of ci + 2 replace those of ci in
    // `ef`.  Loads issued after chunk ci's: the entries of ci + 2 (one) and
    // chunk ci + 1's (NV + NK).
    auto iter = [&](int ci, uint32_t &ef, const uint32_t en, char *vc, char *vn,
                    ChunkK<D, TIn> &cur, ChunkK<D, TIn> &nxt) __attribute__((always_inline)) {
        ef = load_e(ci + 2);
        issue(ci + 1, en, vn, nxt);
        wait_loads_but<NV + NK + 1>();
        asm volatile("" ::: "memory");
        compute(vc, cur);
    };
    for (int ci = 0; ci < nch; ci += 2) {
        iter(ci, ea, eb, vslot0, vslot1, ka, kb);
        if (ci + 1 >= nch) break;
        iter(ci + 1, eb, ea, vslot1, vslot0, kb, ka);
    }
    wait_loads();  // the loads past the list land before the slots are left
}

template <int D, typename TIn, typename TOut>
__device__ __attribute__((always_inline)) inline void blockwise_row(
    const FwdArgs<TIn, TOut> &a, const TileBufs<D> &bufs, int row, int I, int bh,
    const RowInfo &ri, const typename Frag<TIn>::type (&qf)[D / 32], HybLds &hl) {
    using frag = typename Frag<TIn>::type;
    using L = Lds<D>;
    const size_t head = (size_t)bh * a.S * D;
    const TIn *Kh = a.K + head, *Vh = a.V + head;

    const int t = threadIdx.x, w = t >> 6, l = t & 63;
    const int lq = l & 15, g = l >> 4;
    const int r = 16 * w + lq;  // this lane's query row inside the tile

    TileList tl;
    tl.fci = a.fci;
    tl.pci = a.pci;
    tl.bm = a.bm;
    tl.nmax = a.n - 1;
    tl.S = a.S;
    tl.f0 = ri.f0;
    tl.nF = ri.nF;
    tl.p0 = ri.p0;
    tl.dl = nullptr;
    // per-tile dispatch: with sparse partial tiles in the encoding, the row's
    // partial tiles are split; the dense ones stay on the tile path below,
    // the sparse ones go to the gather path after it
    const bool hyb = a.hybrid && ri.stats[5] > 0 && ri.nP > 0;
    int nD = ri.nP;
    if (hyb) {
        nD = split_partials(a, ri, hl);
        tl.dl = hl.list;
    }
    tl.nT = ri.nF + nD;
    const int nT = tl.nT, nF = tl.nF;
    // columns of the first four tiles the tile path visits (-1 past them)
    int cc[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
        cc[k] = !hyb || k < nF ? ri.c[k] : k < nT ? (int)(hl.list[k - nF] >> 16) : -1;

    const int qi = 64 * I + r;

    RowState<D> rs;
#pragma unroll
    for (int i = 0; i < D / 16; ++i) rs.acc[i] = f4_t{0.f, 0.f, 0.f, 0.f};
    rs.m = -INFINITY;
    rs.mc = 0.f;
    rs.l = 0.f;

    // per-lane LDS offsets, the same in every buffer
    const KOff<D> ko = k_offsets<D>(lq, g);
    const VOff<D> vo = v_offsets<D>(lq, g);
    const int b_off = ((r >> 3) * 8 + (g >> 1)) * 8 + (r & 7);
    const int nib = 4 * (g & 1);

    // Pipeline: K is loaded two tiles ahead of its use and V one tile
    // ahead, each straight into the buffer the previous barrier freed, so
    // that tile step `it` can issue QK^T of tile it+1 before the softmax of
    // tile it (matrix cores busy during the VALU work).  Buffers: K(it) in
    // bufs.k[it&1], V(it) in bufs.v[it&1].  The mask bytes of a partial tile
    // come into registers with its K load.  The loop is unrolled by two so
    // that the buffers are picked at compile time and the two score buffers
    // and mask slots swap roles instead of being copied.
    const int wu = __builtin_amdgcn_readfirstlane(w);  // w, known uniform
    const TileOffs<D> to = tile_offsets<D>(wu, l);
    // the K and V bases in scalar registers, whatever else in the kernel
    // uses the same values per lane (the tile addresses are then scalar
    // arithmetic and the loads take the scalar-base form)
    const char *Kb = reinterpret_cast<const char *>(uniform_ptr(Kh));
    const char *Vb = reinterpret_cast<const char *>(uniform_ptr(Vh));
    MaskRegs mk0, mk1;
    f4_t s_a[4], s_b[4];
    uint32_t m_a = 0, m_b = 0;
    // loads of stored tile idx (column J): K (with its mask bytes) or V
    auto load_k = [&](char *buf, MaskRegs &mk, int idx, int J) __attribute__((always_inline)) {
        load_tile<D>(buf, Kb + (size_t)J * 64 * D * 2, tl.lim<D>(J), to, wu);
        load_mask(mk, tl.words(idx), b_off);
    };
    auto load_v = [&](char *buf, int J) __attribute__((always_inline)) {
        load_tile<D>(buf, Vb + (size_t)J * 64 * D * 2, tl.lim<D>(J), to, wu);
    };
    if (nT >= 1 && nT <= 3) {
        // A row of at most three tiles requests all of them at once: tiles
        // 0 and 1 into the four buffers, tile 2 into registers, stored into
        // the buffers of tile 0 once every wave is done with them.  The row
        // then waits for memory once instead of once per tile (such rows
        // are common at small S, where all workgroups of a launch start
        // together and each wait is a full memory round trip).  Every load
        // is issued whatever nT and the tile kinds are (a missing tile
        // re-reads tile 0; a full tile's mask bytes come from the row
        // summary and go unused), so the loads are one fixed sequence and a
        // constant count waits for exactly those of tiles 0 and 1.  Tiles
        // go through the softmax in the loop's order (same results).
        const int c0 = tl.clamp(cc[0]);
        const int c1 = nT > 1 ? tl.clamp(cc[1]) : c0;
        const int c2 = nT > 2 ? tl.clamp(cc[2]) : c0;
        const uint8_t *any_src = reinterpret_cast<const uint8_t *>(a.info);
        auto mask_src = [&](int idx) __attribute__((always_inline)) {
            return idx < nT && idx >= nF
                       ? reinterpret_cast<const uint8_t *>(tl.words(idx)) + b_off
                       : any_src;
        };
        TileRegs<D> k2, v2;
        MaskRegs mk2;
        load_tile<D>(bufs.k[0], Kb + (size_t)c0 * 64 * D * 2, tl.lim<D>(c0), to, wu);
        load_mask_at(mk0, mask_src(0));
        load_tile<D>(bufs.v[0], Vb + (size_t)c0 * 64 * D * 2, tl.lim<D>(c0), to, wu);
        load_tile<D>(bufs.k[1], Kb + (size_t)c1 * 64 * D * 2, tl.lim<D>(c1), to, wu);
        load_mask_at(mk1, mask_src(1));
        load_tile<D>(bufs.v[1], Vb + (size_t)c1 * 64 * D * 2, tl.lim<D>(c1), to, wu);
        // tile 2's loads after all of those (the wait below counts on it)
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        load_tile_regs<D>(k2, Kb + (size_t)c2 * 64 * D * 2, tl.lim<D>(c2), to);
        load_mask_at(mk2, mask_src(2));
        load_tile_regs<D>(v2, Vb + (size_t)c2 * 64 * D * 2, tl.lim<D>(c2), to);
        __builtin_amdgcn_sched_barrier(0);
        // tiles 0 and 1 are in; tile 2's 2 * D/32 chunk loads and 4 mask
        // byte loads stay in flight
        wait_loads_but<2 * (D / 32) + 4>();
        m_a = nF == 0 ? mask_bits(mk0, nib) : 0u;
        m_b = nT > 1 && nF <= 1 ? mask_bits(mk1, nib) : 0u;
        bare_barrier();
        qk_tile<D, TIn>(s_a, qf, bufs.k[0], ko, nF == 0, m_a);
        if (nT > 1) qk_tile<D, TIn>(s_b, qf, bufs.k[1], ko, nF <= 1, m_b);
        softmax_pv<D, TIn>(rs, s_a, bufs.v[0], a.c, vo);
        if (nT > 2) {
            const uint32_t m_c = nF <= 2 ? mask_bits(mk2, nib) : 0u;
            bare_barrier();  // every wave is done with K(0) and V(0)
            store_tile_regs<D>(bufs.k[0], k2, wu, l);
            store_tile_regs<D>(bufs.v[0], v2, wu, l);
            __syncthreads();
            qk_tile<D, TIn>(s_a, qf, bufs.k[0], ko, nF <= 2, m_c);
        }
        if (nT > 1) softmax_pv<D, TIn>(rs, s_b, bufs.v[1], a.c, vo);
        if (nT > 2) softmax_pv<D, TIn>(rs, s_a, bufs.v[0], a.c, vo);
    } else {
        // columns of the K tile (jk, tile it+2) and V tile (jv, tile it+1) that
        // tile step it loads
        int jv = tl.clamp(cc[1]), jk = tl.clamp(cc[2]);
        if (nT > 0) {
            load_k(bufs.k[0], mk0, 0, tl.clamp(cc[0]));
            load_v(bufs.v[0], tl.clamp(cc[0]));
            if (nT > 1) load_k(bufs.k[1], mk1, 1, jv);
        }
        wait_loads();
        if (nT > 0 && nF == 0) m_a = mask_bits(mk0, nib);
        if (nT > 1 && 1 >= nF) m_b = mask_bits(mk1, nib);
        __syncthreads();
        if (nT > 0) qk_tile<D, TIn>(s_a, qf, bufs.k[0], ko, nF == 0, m_a);
        // every wave has read K(0) before tile step 0 loads into its buffer
        __syncthreads();

        // One tile step (cb = it & 1, a compile-time constant): scores of tile
        // it in `cur` (mask mc), of tile it+1 go to `nxt` (mask mn); mc is then
        // reused for tile it+2's mask.
        auto step = [&](int it, auto cbc, f4_t(&cur)[4], f4_t(&nxt)[4], uint32_t &mc,
                        const uint32_t mn) __attribute__((always_inline)) {
            constexpr int cb = decltype(cbc)::value, nb = cb ^ 1;
            // column of tile it+3 (tile step it+1 loads its K); from memory past
            // the four of the row summary
            int jn_raw = cc[3];
            if (it + 3 < nT && it + 3 >= 4) jn_raw = tl.col_of(it + 3);
            // K(it+2) replaces K(it) (read in the previous step); V(it+1)
            // replaces V(it-1) (read in the previous step)
            if (it + 2 < nT) load_k(bufs.k[cb], mk0, it + 2, jk);
            if (it + 1 < nT) load_v(bufs.v[nb], jv);
            if (it + 1 < nT)
                qk_tile<D, TIn>(nxt, qf, bufs.k[nb], ko, it + 1 >= nF, mn);
            softmax_pv<D, TIn>(rs, cur, bufs.v[cb], a.c, vo);
            wait_loads();
            mc = it + 2 < nT && it + 2 >= nF ? mask_bits(mk0, nib) : 0u;
            jv = jk;
            jk = tl.clamp(__builtin_amdgcn_readfirstlane(jn_raw));
            __syncthreads();
        };
        for (int it = 0; it < nT; it += 2) {
            step(it, std::integral_constant<int, 0>(), s_a, s_b, m_a, m_b);
            if (it + 1 >= nT) break;
            step(it + 1, std::integral_constant<int, 1>(), s_b, s_a, m_b, m_a);
        }

    }

    if (hyb && nD < ri.nP) {
        // every wave is done with the tile buffers; each takes one as its
        // slice for the gather path, over its group's row-wise entries
        if (nT > 0) __syncthreads();
        // V slot 0 of waves 0-3 in the K buffers, slot 1 in the V buffers
        constexpr int VSL = 32 * D * 2;
        char *vs0 = (w < 2 ? bufs.k[0] : bufs.k[1]) + VSL * (w & 1);
        char *vs1 = (w < 2 ? bufs.v[0] : bufs.v[1]) + VSL * (w & 1);
        const uint32_t *ents = a.rent + 256 * (size_t)ri.p0 + 64 * (size_t)w * ri.nP;
        const int ne = a.rcnt[4 * (size_t)row + w];
        gather_stream<D, TIn>(rs, vs0, vs1, ents, ne, qf, Kh, Vh, a.c, a.S, vo);
    }

    // epilogue: total l over the 4 lanes of this query
    const float lt = sum_xor32(sum_xor16(rs.l));
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    if (qi < a.S) {
        TOut *orow = a.O + head + (size_t)qi * D;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt)
            store4<TOut>(orow + 16 * dt + 4 * g, rs.acc[dt] * inv);
    }
}

}  // namespace smh
