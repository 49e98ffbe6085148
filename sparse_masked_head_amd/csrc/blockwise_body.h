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
//   * K and V sit row-major in separate LDS double buffers (plain 16-byte
//     writes; the transpose that V^T needs is done by ds_read_b64_tr_b16
//     when the P V operand is read);
//     K is staged two tiles ahead of its use and V one, so iteration t
//     issues the QK^T MFMAs of tile t+1 before the softmax of tile t and
//     the matrix cores work while the VALU does the softmax; one barrier
//     per tile, global loads one tile ahead of staging;
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

#include "fwd_common.h"

namespace smh {

template <int D> struct Lds {
    // Row stride (elements) of the K and V tiles, chosen on gfx950 so that
    // the operand reads are conflict-free: rows shifted by 32 bytes (a probe
    // of the access patterns: 16-byte shifts conflict, 32-byte do not).
    static constexpr int KLD = D + 16;
    static constexpr int KBUF = 64 * KLD * 2;  // K tile, row-major
    static constexpr int VBUF = 64 * KLD * 2;  // V tile, row-major
    static constexpr int BYTES = 2 * KBUF + 2 * VBUF;
    static __device__ char *kbuf(char *smem, int i) { return smem + i * KBUF; }
    static __device__ char *vbuf(char *smem, int i) {
        return smem + 2 * KBUF + i * VBUF;
    }
};

// Registers carrying one K tile (and, for a partial tile, the four mask
// bytes this lane needs) or one V tile from global memory to LDS.
template <int D> struct KRegs {
    static constexpr int N = 64 * D / 8 / 256;  // 16-byte chunks per thread
    u4_t kr[N];
    uint32_t mb[4];
};
template <int D> struct VRegs {
    static constexpr int N = 64 * D / 8 / 256;  // 16-byte chunks per thread
    u4_t vr[N];
};

// Global loads of K tile J (one contiguous block: thread t takes 16-byte
// chunks t, t+256, ...; a chunk at element offset above `lim` is read from
// `lim` instead, so that the rows of a tile cut by S come from inside K:
// they are masked, and any finite value serves) and, for a partial tile,
// this lane's mask bytes:
// keys 16st + 4g + i of query row r are bits 4(g&1)+i of byte r&7 of inner
// tile (r>>3, 2st + (g>>1)); b_off is that byte's offset for st = 0, each
// further st is two words (16 bytes) on.
template <int D, typename TIn>
__device__ __attribute__((always_inline)) inline void fetch_k(
    KRegs<D> &r, const TIn *__restrict__ Kh, int J, int lim,
    const uint64_t *__restrict__ words, int b_off, int t) {
    const TIn *kt = Kh + (size_t)J * 64 * D;
#pragma unroll
    for (int i = 0; i < KRegs<D>::N; ++i)
        r.kr[i] = *reinterpret_cast<const u4_t *>(kt + min((t + 256 * i) * 8, lim));
    if (words) {
        const uint8_t *wb = reinterpret_cast<const uint8_t *>(words) + b_off;
#pragma unroll
        for (int st = 0; st < 4; ++st) r.mb[st] = wb[16 * st];
    }
}

// The lane's mask bits of a fetched partial tile: bit 8st + i (i < 4) =
// key 16st + 4g + i of its query row (nib = 4(g&1)); the other bits are
// not used.
template <int D>
__device__ __attribute__((always_inline)) inline uint32_t mask_bits(
    const KRegs<D> &r, int nib) {
    return (r.mb[0] | (r.mb[1] << 8) | (r.mb[2] << 16) | (r.mb[3] << 24)) >> nib;
}

// Bit `off` of x as 0 or -1 (v_bfe_i32; written out so that the compiler
// keeps this one-instruction form instead of a compare and a select).
template <int off> __device__ __attribute__((always_inline)) inline int bit_mask(int x) {
    int r;
    asm("v_bfe_i32 %0, %1, %2, 1" : "=v"(r) : "v"(x), "i"(off));
    return r;
}

// Global loads of V tile J, the same contiguous chunks and limit as K (a
// masked key's V row is multiplied by a zero probability).
template <int D, typename TIn>
__device__ __attribute__((always_inline)) inline void fetch_v(
    VRegs<D> &r, const TIn *__restrict__ Vh, int J, int lim, int t) {
    const TIn *vt = Vh + (size_t)J * 64 * D;
#pragma unroll
    for (int i = 0; i < VRegs<D>::N; ++i)
        r.vr[i] = *reinterpret_cast<const u4_t *>(vt + min((t + 256 * i) * 8, lim));
}

// K tile row-major into a K buffer (padded rows).
template <int D, typename TIn>
__device__ __attribute__((always_inline)) inline void stage_k(
    const KRegs<D> &r, char *kb, int t) {
    using L = Lds<D>;
    TIn *ks = reinterpret_cast<TIn *>(kb);
#pragma unroll
    for (int i = 0; i < KRegs<D>::N; ++i) {
        const int e = t + 256 * i;
        const int row = e / (D / 8), col = (e % (D / 8)) * 8;
        *reinterpret_cast<u4_t *>(ks + row * L::KLD + col) = r.kr[i];
    }
}

// V tile row-major into a V buffer (padded rows, like K); the transpose
// that the P V product needs is done by the transposing LDS reads.
template <int D>
__device__ __attribute__((always_inline)) inline void stage_v(
    const VRegs<D> &r, char *vb, int t) {
    using L = Lds<D>;
    uint16_t *vs = reinterpret_cast<uint16_t *>(vb);
#pragma unroll
    for (int i = 0; i < VRegs<D>::N; ++i) {
        const int e = t + 256 * i;
        const int row = e / (D / 8), col = (e % (D / 8)) * 8;
        *reinterpret_cast<u4_t *>(vs + row * L::KLD + col) = r.vr[i];
    }
}

// Running state of one lane: O^T accumulators of its query (d = 16dt +
// 4(l/16) + i), running max (raw score units) and its part of the sum.
template <int D> struct RowState {
    f4_t acc[D / 16];
    float m, l;
};

// S^T = K Q^T for one tile (four 16-key sub-tiles), raw scores.  For a
// partial tile the accumulators start at 0 for a valid key and -inf for a
// masked one (mbits: bit 8st + i = key 16st + 4g + i is valid), so masked
// scores leave the matrix cores as -inf and the softmax needs no masking.
// The two cases are separate code so that a full tile's first products
// take the constant zero accumulator.
template <int D, typename TIn, bool kPartial>
__device__ __attribute__((always_inline)) inline void qk_tile_k(
    f4_t (&sc)[4], const typename Frag<TIn>::type (&qf)[D / 32],
    const char *kb, int k_off, uint32_t mbits) {
    using F = Frag<TIn>;
    using frag = typename F::type;
    const TIn *ks = reinterpret_cast<const TIn *>(kb) + k_off;
    const int inv = (int)~mbits;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
        f4_t c0 = f4_t{0.f, 0.f, 0.f, 0.f};
        if (kPartial)  // all ones where masked -> the bits of -inf
            c0 = f4_t{__int_as_float(bit_mask<0>(inv >> (8 * st)) & (int)0xFF800000u),
                      __int_as_float(bit_mask<1>(inv >> (8 * st)) & (int)0xFF800000u),
                      __int_as_float(bit_mask<2>(inv >> (8 * st)) & (int)0xFF800000u),
                      __int_as_float(bit_mask<3>(inv >> (8 * st)) & (int)0xFF800000u)};
        const frag a0 = *reinterpret_cast<const frag *>(ks + 16 * st * Lds<D>::KLD);
        sc[st] = F::mfma(a0, qf[0], c0);
#pragma unroll
        for (int s = 1; s < D / 32; ++s) {
            const frag a = *reinterpret_cast<const frag *>(
                ks + 16 * st * Lds<D>::KLD + 32 * s);
            sc[st] = F::mfma(a, qf[s], sc[st]);
        }
    }
}

template <int D, typename TIn>
__device__ __attribute__((always_inline)) inline void qk_tile(
    f4_t (&sc)[4], const typename Frag<TIn>::type (&qf)[D / 32],
    const char *kb, int k_off, bool partial, uint32_t mbits) {
    if (partial)
        qk_tile_k<D, TIn, true>(sc, qf, kb, k_off, mbits);
    else
        qk_tile_k<D, TIn, false>(sc, qf, kb, k_off, mbits);
}

// Softmax of one tile's scores (masked ones already -inf) and
// O^T += V^T P^T.  c = scale * log2(e) > 0.
template <int D, typename TIn>
__device__ __attribute__((always_inline)) inline void softmax_pv(
    RowState<D> &rs, f4_t (&sc)[4], const char *vb, float c, int v_off) {
    using F = Frag<TIn>;
    using frag = typename F::type;
    using L = Lds<D>;
    float mx = -INFINITY;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
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
        rs.l *= alpha;
#pragma unroll
        for (int i = 0; i < D / 16; ++i) rs.acc[i] *= alpha;
    }
    const float mc = (rs.m == -INFINITY ? 0.f : rs.m) * c;

    // P^T as B operand: keys 32u + 4g + j (j < 4), 32u + 16 + 4g + j - 4
    frag pf[2];
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            pf[st >> 1][(st & 1) * 4 + i] =
                (TIn)__builtin_amdgcn_exp2f(fmaf(sc[st][i], c, -mc));
    float lsum = rs.l;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
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
    // slots 0..3 and 32u + 16 + 4g for slots 4..7.  v_off is the lane's
    // (q, a) offset in elements.
    const char *vs = vb + 2 * v_off;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const char *p0 = vs + 2 * (32 * u * L::KLD + 16 * dt);
            const char *p1 = p0 + 2 * 16 * L::KLD;
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
// then gives wrong numbers, never an access outside K and V.  lim(J) is the
// last in-bounds 8-element chunk offset of tile J (S cuts the last tile).
struct TileList {
    const int32_t *fci, *pci;
    const uint64_t *bm;
    int f0, nF, p0, nT, nmax, S;
    int c4[4];  // columns of the first four tiles (row_info)
    __device__ int col(int idx) const {
        const int J = idx < 4 ? c4[idx] : idx < nF ? fci[f0 + idx] : pci[p0 + idx - nF];
        return (int)min((unsigned)J, (unsigned)nmax);
    }
    template <int D> __device__ int lim(int J) const {
        return min(64, S - 64 * J) * D - 8;
    }
    __device__ const uint64_t *words(int idx) const {
        return idx < nF ? nullptr : bm + (size_t)(p0 + idx - nF) * 64;
    }
};

// Workgroup work: encoding row `row` (outer-tile row I of its mask, summary
// ri) of head bh.
template <int D, typename TIn, typename TOut>
__device__ __attribute__((always_inline)) inline void blockwise_row(
    const FwdArgs<TIn, TOut> &a, char *smem, int I, int bh, const RowInfo &ri) {
    using frag = typename Frag<TIn>::type;
    using L = Lds<D>;
    const size_t head = (size_t)bh * a.S * D;
    const TIn *Qh = a.Q + head, *Kh = a.K + head, *Vh = a.V + head;

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
    tl.nT = ri.nF + ri.nP;
#pragma unroll
    for (int k = 0; k < 4; ++k) tl.c4[k] = ri.c[k];
    const int nT = tl.nT, nF = tl.nF;

    // this lane's Q rows as the B operand: query r, d = 32s + 8g + 0..7
    // (a query past S, in a tile cut by S, reads query S-1 and is not stored)
    const int qi = 64 * I + r;
    frag qf[D / 32];
    {
        const TIn *qrow = Qh + (size_t)min(qi, a.S - 1) * D;
#pragma unroll
        for (int s = 0; s < D / 32; ++s)
            qf[s] = *reinterpret_cast<const frag *>(qrow + 32 * s + 8 * g);
    }

    RowState<D> rs;
#pragma unroll
    for (int i = 0; i < D / 16; ++i) rs.acc[i] = f4_t{0.f, 0.f, 0.f, 0.f};
    rs.m = -INFINITY;
    rs.l = 0.f;

    // per-lane LDS offsets (elements / bytes), the same in every buffer
    const int k_off = lq * L::KLD + 8 * g;
    const int v_off = (4 * g + (lq >> 2)) * L::KLD + 4 * (lq & 3);
    const int b_off = ((r >> 3) * 8 + (g >> 1)) * 8 + (r & 7);
    const int nib = 4 * (g & 1);

    // Pipeline: K (with its words) is staged two tiles ahead of its use and
    // V one tile ahead, so that tile step `it` can issue QK^T of tile it+1
    // before the softmax of tile it (matrix cores busy during the VALU
    // work).  Buffers: K(it) in kbuf(it&1), V(it) in vbuf(it&1).  The mask
    // bits ride along in registers, taken from the K registers when they
    // are staged.  At d = 64 the loop is unrolled by two so that the two
    // score buffers and mask slots swap roles instead of being copied.
    KRegs<D> kr, kr1;
    VRegs<D> vr;
    f4_t s_a[4], s_b[4];
    uint32_t m_a = 0, m_b = 0;
    // loads of stored tile idx: K (with its mask bytes) or V
    auto load_k = [&](KRegs<D> &dst, int idx) __attribute__((always_inline)) {
        const int J = tl.col(idx);
        fetch_k<D, TIn>(dst, Kh, J, tl.lim<D>(J), tl.words(idx), b_off, t);
    };
    auto load_v = [&](int idx) __attribute__((always_inline)) {
        const int J = tl.col(idx);
        fetch_v<D, TIn>(vr, Vh, J, tl.lim<D>(J), t);
    };
    if (nT > 0) {
        load_k(kr, 0);
        load_v(0);
        if (nT > 1) load_k(kr1, 1);
        stage_k<D, TIn>(kr, L::kbuf(smem, 0), t);
        if (nF == 0) m_a = mask_bits<D>(kr, nib);
        stage_v<D>(vr, L::vbuf(smem, 0), t);
        if (nT > 1) {
            stage_k<D, TIn>(kr1, L::kbuf(smem, 1), t);
            if (1 >= nF) m_b = mask_bits<D>(kr1, nib);
        }
        if (nT > 2) load_k(kr, 2);
        if (nT > 1) load_v(1);
    }
    __syncthreads();
    if (nT > 0) qk_tile<D, TIn>(s_a, qf, L::kbuf(smem, 0), k_off, nF == 0, m_a);
    // every wave has read K(0) before tile step 0 overwrites its buffer
    __syncthreads();

    // One tile step: scores of tile it in `cur` (mask mc), of tile it+1 go
    // to `nxt` (mask mn); mc is then reused for tile it+2's mask.
    auto step = [&](int it, f4_t(&cur)[4], f4_t(&nxt)[4], uint32_t &mc,
                    const uint32_t mn) __attribute__((always_inline)) {
        const int cb = it & 1, nb = cb ^ 1;
        if (it + 1 < nT)
            qk_tile<D, TIn>(nxt, qf, L::kbuf(smem, nb), k_off, it + 1 >= nF, mn);
        softmax_pv<D, TIn>(rs, cur, L::vbuf(smem, cb), a.c, v_off);
        // K(it+2) replaces K(it) (read in the previous step); V(it+1)
        // replaces V(it-1)
        uint32_t m2 = 0;
        if (it + 2 < nT) {
            stage_k<D, TIn>(kr, L::kbuf(smem, cb), t);
            if (it + 2 >= nF) m2 = mask_bits<D>(kr, nib);
        }
        if (it + 1 < nT) stage_v<D>(vr, L::vbuf(smem, nb), t);
        if (it + 3 < nT) load_k(kr, it + 3);
        if (it + 2 < nT) load_v(it + 2);
        __syncthreads();
        mc = m2;
    };
    if constexpr (D == 64) {
        for (int it = 0; it < nT; it += 2) {
            step(it, s_a, s_b, m_a, m_b);
            if (it + 1 >= nT) break;
            step(it + 1, s_b, s_a, m_b, m_a);
        }
    } else {  // measured: the unrolled body is slower at d = 128
        for (int it = 0; it < nT; ++it) {
            step(it, s_a, s_b, m_a, m_b);
#pragma unroll
            for (int st = 0; st < 4; ++st) s_a[st] = s_b[st];
            const uint32_t m2 = m_a;
            m_a = m_b;
            m_b = m2;
        }
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
