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
//     them (one 16-byte read per sub-tile from a table in LDS), so masked
//     scores leave the matrix cores as -inf;
//   * online softmax in base 2 (running max and sum per query) with lazy
//     rescaling (the reference max moves only when passed by more than 8
//     in exponent units); only the 4 lanes sharing a query exchange values
//     (two gfx950 row swaps);
//   * O^T += V^T P^T with the same MFMA: P^T is the B operand straight from
//     the score registers rounded to the input type, V^T the A operand from
//     LDS; the O rows a lane holds belong to the query whose softmax state
//     it holds, so rescaling is lane-local.
// Per-tile dispatch: with sparse partial tiles in the encoding (at most
// SMH_SPARSE_TILE_MAX valid elements), the row's partial tiles are split;
// the tile loop above runs the full and dense partial ones, then each
// wavefront runs the row's sparse ones on the gather path (gather_stream)
// into the same softmax state.
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
// The same as an assembly instruction, which the compiler keeps whatever
// it sees depend on the loads (it may drop the builtin where it sees no
// use of their results, e.g. before reads in assembly).
template <int N> __device__ __attribute__((always_inline)) inline void wait_loads_but_asm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"i"(N) : "memory");
}
// Wait for this wave's outstanding LDS operations (global loads are not
// waited for): vmcnt and expcnt at their maxima, lgkmcnt 0.
__device__ __attribute__((always_inline)) inline void wait_lds() {
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
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

// The starting accumulators of a partial tile come from a 16-entry table in
// LDS (entry n: element i is 0 if bit i of n is set, else -inf), one
// 16-byte read per sub-tile indexed by the lane's four mask bits, instead
// of two vector operations per score.
__device__ __attribute__((always_inline)) inline void fill_mask_lut(f4_t *lut) {
    const int t = threadIdx.x;
    if (t < 64)
        reinterpret_cast<float *>(lut)[t] = (t >> 2 >> (t & 3)) & 1 ? 0.f : -INFINITY;
}

template <int D, typename TIn, bool kPartial>
__device__ __attribute__((always_inline)) inline void qk_tile_k(
    f4_t (&sc)[4], const typename Frag<TIn>::type (&qf)[D / 32],
    const char *kb, const KOff<D> &ko, uint32_t mbits, const f4_t *lut) {
    using F = Frag<TIn>;
    using frag = typename F::type;
    const char *ks = kb + ko.base;
    // the four sub-tiles' products alternate (slice s of d outer), so that
    // consecutive MFMAs never wait for each other's results
#pragma unroll
    for (int s = 0; s < D / 32; ++s)
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const frag a = *reinterpret_cast<const frag *>(
                ks + 16 * st * Lds<D>::CPR * 16 + ko.x[s]);
            f4_t c = sc[st];
            if (s == 0) {
                c = f4_t{0.f, 0.f, 0.f, 0.f};
                if (kPartial) c = lut[(mbits >> (8 * st)) & 0xFu];
            }
            sc[st] = F::mfma(a, qf[s], c);
        }
}

template <int D, typename TIn>
__device__ __attribute__((always_inline)) inline void qk_tile(
    f4_t (&sc)[4], const typename Frag<TIn>::type (&qf)[D / 32],
    const char *kb, const KOff<D> &ko, bool partial, uint32_t mbits, const f4_t *lut) {
    if (partial)
        qk_tile_k<D, TIn, true>(sc, qf, kb, ko, mbits, lut);
    else
        qk_tile_k<D, TIn, false>(sc, qf, kb, ko, mbits, lut);
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
// NST = 4 for an outer tile) and O^T += V^T P^T with V's rows in a
// tile-buffer layout, in three parts: sm_max (row max, lazy rescale; the
// gather path uses it on one sub-tile), sm_exp (probabilities and row sum,
// vector work only) and pv (the matrix-core product).  c = scale * log2(e)
// > 0.
template <int D, int NST>
__device__ __attribute__((always_inline)) inline void sm_max(RowState<D> &rs,
                                                             const f4_t (&sc)[NST], float c) {
    float mx = -INFINITY;
#pragma unroll
    for (int st = 0; st < NST; ++st) {
        mx = fmaxf(fmaxf(mx, sc[st][0]), sc[st][1]);
        mx = fmaxf(fmaxf(mx, sc[st][2]), sc[st][3]);
    }
    // Lazy rescaling: the reference max rs.m moves only when a score passes
    // it by more than 8 in base-2 exponent units, so most tiles skip the
    // rescale; the probabilities then stay below 2^8 (well inside the input
    // type's range) and the final division by l cancels the reference.
    // (mx - m) * c is NaN (no move) when both are -inf, +inf when only m is.
    // A row's max passes that bound only if one of its lanes' maxima does:
    // when no lane's does, the cross-lane max is skipped (same result).
    if (!__builtin_amdgcn_ballot_w64((mx - rs.m) * c > 8.f)) return;
    mx = max_xor32(max_xor16(mx));
    const bool grow = (mx - rs.m) * c > 8.f;
    {
        const float m_new = grow ? mx : rs.m;
        const float alpha = grow ? __builtin_amdgcn_exp2f((rs.m - m_new) * c) : 1.f;
        rs.m = m_new;
        rs.mc = grow ? mx * c : rs.mc;  // a growing max is finite
        rs.l *= alpha;
#pragma unroll
        for (int i = 0; i < D / 16; ++i) rs.acc[i] *= alpha;
    }
}

// P^T as B operand: keys 32u + 4g + j (j < 4), 32u + 16 + 4g + j - 4.
template <int D, typename TIn, int NST>
__device__ __attribute__((always_inline)) inline void sm_exp(
    RowState<D> &rs, const f4_t (&sc)[NST], float c,
    typename Frag<TIn>::type (&pf)[NST / 2]) {
    constexpr int NU = NST / 2;
    const float mc = rs.mc;
    float lsum = rs.l;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        // sub-tiles 2u, 2u + 1 -> elements 0..3, 4..7 of pf[u], packed in
        // pairs as they are made (8 values live at a time)
        float e[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            e[i] = __builtin_amdgcn_exp2f(fmaf(sc[2 * u + (i >> 2)][i & 3], c, -mc));
        const uint32_t pw[4] = {pack2<TIn>(e[0], e[1]), pack2<TIn>(e[2], e[3]),
                                pack2<TIn>(e[4], e[5]), pack2<TIn>(e[6], e[7])};
        __builtin_memcpy(&pf[u], pw, 16);
#pragma unroll
        for (int j = 0; j < 4; ++j) lsum = sum2<TIn>(pw[j], lsum);
    }
    rs.l = lsum;
}

// A operand V^T (rows = output columns 16dt + l%16, slots = keys of the P^T
// slots) read with ds_read_b64_tr_b16 from row-major V: within each 16-lane
// group, lane j = a + 4q points at V[key0 + q][d0 + 4a] and lane i receives
// V[key0 .. key0+3][d0 + i]; key0 = 32u + 4g for slots 0..3 and 32u + 16 +
// 4g for slots 4..7.  vo holds the lane's (q, a) offsets in the swizzled
// buffer.
template <int D, typename TIn, int NU>
__device__ __attribute__((always_inline)) inline void pv(
    RowState<D> &rs, const typename Frag<TIn>::type (&pf)[NU], const char *vb,
    const VOff<D> &vo) {
    using F = Frag<TIn>;
    using frag = typename F::type;
    using L = Lds<D>;
    // key half u outer, so that consecutive MFMAs write different
    // accumulators
#pragma unroll
    for (int u = 0; u < NU; ++u) {
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
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

// The three parts in sequence.
template <int D, typename TIn, int NST = 4>
__device__ __attribute__((always_inline)) inline void softmax_pv(
    RowState<D> &rs, f4_t (&sc)[NST], const char *vb, float c, const VOff<D> &vo) {
    typename Frag<TIn>::type pf[NST / 2];
    sm_max<D, NST>(rs, sc, c);
    sm_exp<D, TIn, NST>(rs, sc, c, pf);
    pv<D, TIn, NST / 2>(rs, pf, vb, vo);
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

// LDS of the row beside the tile buffers: the split's partial tiles, dense
// ones first, each column << 16 | index in the row's partial list, its
// per-wavefront counts, and the table of partial-tile accumulators.
struct HybLds {
    uint32_t list[kHybMaxN];
    int wcnt[16];
    f4_t lut[16];  // starting accumulators of partial tiles (fill_mask_lut)
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
    uint32_t *e[2];  // gather path: entry rings of block parity 0, 1 (64 per wavefront)
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
// built once per mask by the encoder) and computes them in chunks of 16
// keys with the same online-softmax state as the tile path: S^T = K Q^T
// with v_mfma_f32_16x16x32 (one 16-key sub-tile), O^T += V^T P^T with
// v_mfma_f32_16x16x16 (16 keys deep), whose B operand is exactly the four
// scores a lane holds.
// The K and V rows of a chunk come into per-wavefront LDS slots by
// global_load_lds (each instruction whole 256- or 128-byte rows, as the tile
// loads), laid out like a tile buffer's first 16 rows, so that the tile
// path's operand offsets (KOff, VOff) serve.  Slots of chunk parity p lie
// in the tile buffers K_p and V_p, wavefront w's at 16 rows * w, so that
// the slots being read and the slots being filled are different LDS
// objects and the compiler does not make the reads wait for the loads.
// The entries come into per-wavefront LDS rings by global_load_lds as
// well, 64 at a time (an entry block: four chunks), blocks of parity p in
// the separate LDS array E_p, and the keys and row sets are read from
// there: with every load of the loop an LDS DMA, the compiler counts their
// completion exactly (an entry load into registers among the DMAs made it
// wait for all of them before each chunk's first use of its entries, so
// that only one chunk's rows were in flight at a time).
// Pipeline, at chunk c: read the keys of chunk c + 1, request its K and V
// rows, wait for chunk c's rows and compute chunk c; an entry block is
// requested four chunks before its first chunk's keys are read, so that
// only the rows' round trips are waited for.  Loads past the list re-read
// its last entry (or key 0), so every wait counts the same loads.

template <typename TIn> struct Frag4;
template <> struct Frag4<_Float16> {
    typedef _Float16 type __attribute__((ext_vector_type(4)));
    static __device__ inline f4_t mfma(type a, type b, f4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
    }
};
template <> struct Frag4<__bf16> {
    typedef short type __attribute__((ext_vector_type(4)));
    static __device__ inline f4_t mfma(type a, type b, f4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
    }
};

template <int D, typename TIn>
__device__ __attribute__((always_inline)) inline void gather_stream(
    RowState<D> &rs, char *kslot0, char *kslot1, char *vslot0, char *vslot1,
    uint32_t *ering0, uint32_t *ering1,
    const char *ents, int ne, const typename Frag<TIn>::type (&qf)[D / 32],
    const char *Kb, const char *Vb, float c, int S, const KOff<D> &ko, const VOff<D> &vo) {
    using F = Frag<TIn>;
    using F4 = Frag4<TIn>;
    using frag = typename F::type;
    using L = Lds<D>;
    const int lane = threadIdx.x & 63, lq = lane & 15, g = lane >> 4;
    constexpr int RPI = 1024 / (2 * D);  // rows per 1 KB load instruction
    constexpr int NI = 16 / RPI;         // load instructions per chunk, K and V each
    const int nch = (ne + 15) >> 4;
    // Addresses: the bases (entry list, K, V, slots, rings) are wave-uniform
    // (scalar registers, the loads in the scalar-base form), each lane adds
    // a 32-bit byte offset.
    // entry block b (entries 64 b .. 64 b + 63, the entries of chunks
    // 4 b .. 4 b + 3) into ring er (lane l's to er[l]); past the list: its
    // last entry
    auto load_eb = [&](int b, uint32_t *er) __attribute__((always_inline)) {
        __builtin_amdgcn_global_load_lds(
            (gbl_void_t *)(ents + 4u * (uint32_t)min(64 * b + lane, ne - 1)),
            (lds_void_t *)er, 4, 0, 0);
    };
    // chunk ci's keys from its ring: the lane's key for each row load, and
    // its valid score slots (bit i: entry 4g + i is in the chunk and its row
    // set holds the lane's query row)
    struct Keys {
        uint32_t key[NI];
        uint32_t ok;
    };
    // The ring reads are one assembly block that waits for them (and for
    // nothing else) at its end: as plain reads, the compiler made them wait
    // for every LDS load in flight (it does not tell the ring from the
    // slots those fill), and, read only where the lane's row is in the
    // chunk, each became a branch with a wait of its own.  The caller has
    // waited for the ring's own load.  Every lane reads: entry rr of the
    // lane's row load i (RPI rows apart) and entries 4g .. 4g + 3.
    auto read_keys = [&](int ci, const uint32_t *er) __attribute__((always_inline)) {
        Keys k;
        const int n = min(16, ne - 16 * ci);
        const uint32_t *ec = er + 16 * (ci & 3);  // the chunk's 16 entries of its block
        const uint32_t rb = (uint32_t)(uintptr_t)(lds_void_t *)(ec + lane / L::CPR);
        const uint32_t ob = (uint32_t)(uintptr_t)(lds_void_t *)(ec + 4 * g);
        uint32_t e[NI];
        u4_t e4;
        static_assert(NI == 4 || NI == 2, "row loads per chunk");
        if constexpr (NI == 4) {
            asm volatile(
                "ds_read_b32 %0, %5\n\t"
                "ds_read_b32 %1, %5 offset:%c7\n\t"
                "ds_read_b32 %2, %5 offset:%c8\n\t"
                "ds_read_b32 %3, %5 offset:%c9\n\t"
                "ds_read_b128 %4, %6\n\t"
                "s_waitcnt lgkmcnt(0)"
                : "=&v"(e[0]), "=&v"(e[1]), "=&v"(e[2]), "=&v"(e[3]), "=&v"(e4)
                : "v"(rb), "v"(ob), "i"(4 * RPI), "i"(8 * RPI), "i"(12 * RPI));
        } else {
            asm volatile(
                "ds_read_b32 %0, %3\n\t"
                "ds_read_b32 %1, %3 offset:%c5\n\t"
                "ds_read_b128 %2, %4\n\t"
                "s_waitcnt lgkmcnt(0)"
                : "=&v"(e[0]), "=&v"(e[1]), "=&v"(e4)
                : "v"(rb), "v"(ob), "i"(4 * RPI));
        }
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int rr = RPI * i + lane / L::CPR;
            // clamped into the head's rows; past the chunk: key 0
            k.key[i] = rr < n ? (uint32_t)min((int)(e[i] & 0xFFFFu), S - 1) : 0u;
        }
        const uint32_t ev[4] = {e4[0], e4[1], e4[2], e4[3]};
        k.ok = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            k.ok |= (uint32_t)(4 * g + i < n && ((ev[i] >> (16 + lq)) & 1u)) << i;
        return k;
    };
    // chunk rows into slots ks, vs (whole rows per load instruction)
    auto issue = [&](const Keys &k, char *ks, char *vs) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int rr = RPI * i + lane / L::CPR, cp = lane % L::CPR;
            // key < 65536, so key * D * 2 < 2^24
            const uint32_t off = 2u * (k.key[i] * (uint32_t)D + 8u * (uint32_t)(cp ^ L::sw(rr)));
            __builtin_amdgcn_global_load_lds((gbl_void_t *)(Kb + off),
                                             (lds_void_t *)(ks + 1024 * i), 16, 0, 0);
            __builtin_amdgcn_global_load_lds((gbl_void_t *)(Vb + off),
                                             (lds_void_t *)(vs + 1024 * i), 16, 0, 0);
        }
    };
    auto compute = [&](const char *ks, const char *vs, uint32_t ok) __attribute__((always_inline)) {
        // 0 / -inf per valid bit (selects: a read of the tile path's LDS
        // table here measured 7% slower)
        f4_t sc[1];
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[0][i] = (ok >> i) & 1u ? 0.f : -INFINITY;
#pragma unroll
        for (int s2 = 0; s2 < D / 32; ++s2)
            sc[0] = F::mfma(*reinterpret_cast<const frag *>(ks + ko.base + ko.x[s2]), qf[s2], sc[0]);
        sm_max<D, 1>(rs, sc, c);
        typename F4::type p4;
        {
            float e[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) e[i] = __builtin_amdgcn_exp2f(fmaf(sc[0][i], c, -rs.mc));
            const uint32_t pw[2] = {pack2<TIn>(e[0], e[1]), pack2<TIn>(e[2], e[3])};
            __builtin_memcpy(&p4, pw, 8);
            rs.l = sum2<TIn>(pw[1], sum2<TIn>(pw[0], rs.l));
        }
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
            const s4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4_t *)(vs + vo.x[dt]));
            typename F4::type a;
            __builtin_memcpy(&a, &v, 8);
            rs.acc[dt] = F4::mfma(a, p4, rs.acc[dt]);
        }
    };
    if (nch == 0) return;
    load_eb(0, ering0);
    load_eb(1, ering1);
    wait_loads_but_asm<1>();  // entry block 0 is in
    uint32_t oka, okb = 0;
    {
        const Keys k0 = read_keys(0, ering0);
        oka = k0.ok;
        issue(k0, kslot0, vslot0);
    }
    // Step ci (P = ci % 4, a compile-time constant): read the keys of chunk
    // j = ci + 1 from its block's ring and request its rows (slots of parity
    // j & 1: kn, vn; valid bits to okn), wait for chunk ci's rows and compute
    // chunk ci (slots kc, vc, valid bits okc).  When j starts entry block
    // b = j / 4 (P == 3), wait for that block, requested four chunks
    // earlier (after it: the 2NI row loads of chunks j - 4 .. j - 1), and
    // request block b + 1 into the other ring, whose block b - 1 had its
    // last keys read in the previous step.  So an entry block is in flight
    // for four steps and a step waits for memory only for its own rows.
    auto iter = [&](int ci, auto pc, const char *kc, const char *vc, char *kn, char *vn,
                    const uint32_t okc, uint32_t &okn) __attribute__((always_inline)) {
        constexpr int P = decltype(pc)::value;
        const int j = ci + 1, b = j >> 2;
        if constexpr (P == 3) wait_loads_but_asm<8 * NI>();  // entry block b is in
        const Keys k = read_keys(j, (b & 1) ? ering1 : ering0);
        okn = k.ok;
        if constexpr (P == 3) load_eb(b + 1, (b & 1) ? ering0 : ering1);
        issue(k, kn, vn);
        wait_loads_but<2 * NI + (P == 3 ? 1 : 0)>();  // chunk ci's rows are in
        asm volatile("" ::: "memory");
        compute(kc, vc, okc);
    };
    using std::integral_constant;
    for (int ci = 0; ci < nch; ci += 4) {
        iter(ci, integral_constant<int, 0>(), kslot0, vslot0, kslot1, vslot1, oka, okb);
        if (ci + 1 >= nch) break;
        iter(ci + 1, integral_constant<int, 1>(), kslot1, vslot1, kslot0, vslot0, okb, oka);
        if (ci + 2 >= nch) break;
        iter(ci + 2, integral_constant<int, 2>(), kslot0, vslot0, kslot1, vslot1, oka, okb);
        if (ci + 3 >= nch) break;
        iter(ci + 3, integral_constant<int, 3>(), kslot1, vslot1, kslot0, vslot0, okb, oka);
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
    fill_mask_lut(hl.lut);  // read after the barriers that precede any tile
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
    const f4_t *lut = hl.lut;

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
        wait_lds();  // the accumulator table is written before the barrier
        bare_barrier();
        qk_tile<D, TIn>(s_a, qf, bufs.k[0], ko, nF == 0, m_a, lut);
        if (nT > 1) qk_tile<D, TIn>(s_b, qf, bufs.k[1], ko, nF <= 1, m_b, lut);
        softmax_pv<D, TIn>(rs, s_a, bufs.v[0], a.c, vo);
        if (nT > 2) {
            const uint32_t m_c = nF <= 2 ? mask_bits(mk2, nib) : 0u;
            bare_barrier();  // every wave is done with K(0) and V(0)
            store_tile_regs<D>(bufs.k[0], k2, wu, l);
            store_tile_regs<D>(bufs.v[0], v2, wu, l);
            __syncthreads();
            qk_tile<D, TIn>(s_a, qf, bufs.k[0], ko, nF <= 2, m_c, lut);
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
        if (nT > 0) qk_tile<D, TIn>(s_a, qf, bufs.k[0], ko, nF == 0, m_a, lut);
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
                qk_tile<D, TIn>(nxt, qf, bufs.k[nb], ko, it + 1 >= nF, mn, lut);
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
        // every wave is done with the tile buffers; each takes 16 rows of
        // each as its slots for the gather path, over its group's row-wise
        // entries
        if (nT > 0) __syncthreads();
        constexpr int SLOT = 16 * D * 2;
        const char *ents = reinterpret_cast<const char *>(
            uniform_ptr(a.rent + 256 * (size_t)ri.p0 + 64 * (size_t)wu * ri.nP));
        const int ne = __builtin_amdgcn_readfirstlane(a.rcnt[4 * (size_t)row + wu]);
        gather_stream<D, TIn>(rs, bufs.k[0] + SLOT * wu, bufs.k[1] + SLOT * wu,
                              bufs.v[0] + SLOT * wu, bufs.v[1] + SLOT * wu, bufs.e[0] + 64 * wu,
                              bufs.e[1] + 64 * wu, ents, ne, qf, Kb, Vb, a.c, a.S, ko, vo);
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
