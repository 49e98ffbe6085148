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
//   * K (row-major) and V (transposed: row = output column, keys
//     contiguous) sit in LDS, double-buffered.  Global loads run two tiles
//     ahead in registers: while tile t is computed, tile t+1 waits in
//     registers and tile t+2 is in flight; tile t+1 goes to the other LDS
//     buffer after the compute, one barrier per tile;
//   * wavefront w owns queries 16w..16w+15 and computes S^T = K Q^T with
//     v_mfma_f32_16x16x32 (A = K rows from LDS, B = its Q rows held in
//     registers for the whole row).  In this accumulator layout lane l holds
//     query l%16's scores against keys 16st + 4(l/16) + i;
//   * partial tiles reset masked scores to -inf: the tile's 64 words are
//     staged with it and each lane reads the four bytes (one per 16-key
//     sub-tile) that hold its query row's bits;
//   * online softmax in base 2 (running max and sum per query); only the
//     4 lanes sharing a query exchange values (two gfx950 row swaps);
//   * O^T += V^T P^T with the same MFMA: P^T is the B operand straight from
//     the score registers rounded to the input type, V^T the A operand from
//     LDS; the O rows a lane holds belong to the query whose softmax state
//     it holds, so rescaling is lane-local.
// Epilogue: O / l (0 for a row with no valid key), stored in the output type.
#pragma once

#include "fwd_common.h"

namespace smh {

template <int D> struct Lds {
    // Row strides (elements), chosen on gfx950 so that the MFMA operand
    // reads are conflict-free: K rows shifted by 32 bytes per row for the
    // 16-byte reads, V^T rows by 8 bytes for the paired 8-byte reads.
    static constexpr int KLD = D + 16;
    static constexpr int VLD = 64 + 4;
    static constexpr int K_ELEMS = 64 * KLD;
    static constexpr int V_ELEMS = D * VLD;
    static constexpr int WORDS_OFF = 2 * (K_ELEMS + V_ELEMS);  // bytes
    static constexpr int STAGE_BYTES = WORDS_OFF + 64 * 8;
    static constexpr int BYTES = 2 * STAGE_BYTES;
};

// Registers that carry one K/V tile (and a partial tile's 64 words) from
// global memory to LDS.
template <int D> struct Staging {
    static constexpr int KCH = 64 * D / 8 / 256;   // 16-byte K chunks/thread
    static constexpr int VT = 32 * (D / 8) / 256;  // V transpose tasks/thread
    u4_t kr[KCH], va[VT], vb[VT];
    uint64_t bw;
};

// Issue the global loads of tile J: K rows are one contiguous block (thread
// t takes 16-byte chunks t, t+256, ...); for V thread t takes keys 2kp and
// 2kp+1 of 8-column chunk dc, ready for the transpose.
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
// transposed (pairs of keys packed per 32-bit write), the 64 words raw.
template <int D, typename TIn>
__device__ __attribute__((always_inline)) inline void stage_tile(
    const Staging<D> &st, char *base, bool partial, int t) {
    using L = Lds<D>;
    TIn *ks = reinterpret_cast<TIn *>(base);
    uint32_t *vs = reinterpret_cast<uint32_t *>(ks + L::K_ELEMS);
    uint64_t *wd = reinterpret_cast<uint64_t *>(base + L::WORDS_OFF);
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

// Running state of one lane: O^T accumulators of its query (d = 16dt +
// 4(l/16) + i), running max (raw score units) and its part of the sum.
template <int D> struct RowState {
    f4_t acc[D / 16];
    float m, l;
};

// One tile from LDS stage `base`: scores, mask, online softmax, P V.
template <int D, typename TIn>
__device__ __attribute__((always_inline)) inline void compute_tile(
    RowState<D> &rs, const typename Frag<TIn>::type (&qf)[D / 32],
    const char *base, bool partial, float c, int k_off, int v_off, int b_off,
    int nib) {
    using F = Frag<TIn>;
    using frag = typename F::type;
    using L = Lds<D>;
    const TIn *ks = reinterpret_cast<const TIn *>(base) + k_off;
    const TIn *vs = reinterpret_cast<const TIn *>(base) + L::K_ELEMS + v_off;
    const uint8_t *wbytes =
        reinterpret_cast<const uint8_t *>(base + L::WORDS_OFF) + b_off;

    // S^T = K Q^T: four 16-key sub-tiles
    f4_t sc[4];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
        sc[st] = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < D / 32; ++s) {
            const frag a =
                *reinterpret_cast<const frag *>(ks + 16 * st * L::KLD + 32 * s);
            sc[st] = F::mfma(a, qf[s], sc[st]);
        }
    }
    if (partial) {
        // keys 16st + 4g + i of row r: bits 4(g&1)+i of byte r&7 of inner
        // tile (r>>3, 2st + (g>>1))
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const uint32_t bits = (uint32_t)wbytes[16 * st] >> nib;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (!((bits >> i) & 1u)) sc[st][i] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
        mx = fmaxf(fmaxf(mx, sc[st][0]), sc[st][1]);
        mx = fmaxf(fmaxf(mx, sc[st][2]), sc[st][3]);
    }
    mx = max_xor32(max_xor16(mx));
    const float m_new = fmaxf(rs.m, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f((rs.m - m_use) * c);
    const float mc = m_use * c;
    rs.m = m_new;

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
    rs.l = rs.l * alpha + lsum;
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
        for (int i = 0; i < D / 16; ++i) rs.acc[i] *= alpha;
    }

    // O^T += V^T P^T
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const TIn *vp = vs + 16 * dt * L::VLD + 32 * u;
            const u2_t lo = *reinterpret_cast<const u2_t *>(vp);
            const u2_t hi = *reinterpret_cast<const u2_t *>(vp + 16);
            const u4_t packed = {lo[0], lo[1], hi[0], hi[1]};
            frag a;
            __builtin_memcpy(&a, &packed, sizeof(a));
            rs.acc[dt] = F::mfma(a, pf[u], rs.acc[dt]);
        }
    }
}

// The stored tiles of one outer-tile row: full tiles first, then partial.
struct TileList {
    const int32_t *fci, *pci;
    const uint64_t *bm;
    int f0, nF, p0, nT;
    __device__ int col(int idx) const {
        return idx < nF ? fci[f0 + idx] : pci[p0 + idx - nF];
    }
    __device__ const uint64_t *words(int idx) const {
        return idx < nF ? nullptr : bm + (size_t)(p0 + idx - nF) * 64;
    }
};

// Tile `it`: refill `fr` (free) with tile it+2, compute LDS stage `cur`,
// move tile it+1 (waiting in `nx`) into the other stage `other`.
template <int D, typename TIn>
__device__ __attribute__((always_inline)) inline void block_step(
    int it, const TileList &tl, Staging<D> &fr, const Staging<D> &nx,
    const char *cur, char *other, RowState<D> &rs,
    const typename Frag<TIn>::type (&qf)[D / 32], const TIn *Kh,
    const TIn *Vh, float c, int k_off, int v_off, int b_off, int nib, int t) {
    if (it + 2 < tl.nT)
        fetch_tile<D, TIn>(fr, Kh, Vh, tl.col(it + 2), tl.words(it + 2), t);
    compute_tile<D, TIn>(rs, qf, cur, it >= tl.nF, c, k_off, v_off, b_off, nib);
    if (it + 1 < tl.nT) stage_tile<D, TIn>(nx, other, it + 1 >= tl.nF, t);
    __syncthreads();
}

template <int D, typename TIn, typename TOut>
__device__ __attribute__((always_inline)) inline void blockwise_row(
    const FwdArgs<TIn, TOut> &a, char *smem, int I, int bh) {
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
    tl.f0 = a.frp[I];
    tl.nF = a.frp[I + 1] - tl.f0;
    tl.p0 = a.prp[I];
    tl.nT = tl.nF + a.prp[I + 1] - tl.p0;
    const int nT = tl.nT, nF = tl.nF;

    // this lane's Q rows as the B operand: query r, d = 32s + 8g + 0..7
    frag qf[D / 32];
    {
        const TIn *qrow = Qh + (size_t)(64 * I + r) * D;
#pragma unroll
        for (int s = 0; s < D / 32; ++s)
            qf[s] = *reinterpret_cast<const frag *>(qrow + 32 * s + 8 * g);
    }

    RowState<D> rs;
#pragma unroll
    for (int i = 0; i < D / 16; ++i) rs.acc[i] = f4_t{0.f, 0.f, 0.f, 0.f};
    rs.m = -INFINITY;
    rs.l = 0.f;

    // per-lane LDS offsets (elements / bytes), the same in both stages
    const int k_off = lq * L::KLD + 8 * g;
    const int v_off = lq * L::VLD + 4 * g;
    const int b_off = ((r >> 3) * 8 + (g >> 1)) * 8 + (r & 7);
    const int nib = 4 * (g & 1);

    Staging<D> s0, s1;
    s0.bw = 0;
    s1.bw = 0;
    if (nT > 0) fetch_tile<D, TIn>(s0, Kh, Vh, tl.col(0), tl.words(0), t);
    if (nT > 1) fetch_tile<D, TIn>(s1, Kh, Vh, tl.col(1), tl.words(1), t);
    if (nT > 0) stage_tile<D, TIn>(s0, smem, nF == 0, t);
    __syncthreads();

    char *st0 = smem, *st1 = smem + L::STAGE_BYTES;
    for (int it = 0; it < nT; it += 2) {
        block_step<D, TIn>(it, tl, s0, s1, st0, st1, rs, qf, Kh, Vh, a.c,
                           k_off, v_off, b_off, nib, t);
        if (it + 1 < nT)
            block_step<D, TIn>(it + 1, tl, s1, s0, st1, st0, rs, qf, Kh, Vh,
                               a.c, k_off, v_off, b_off, nib, t);
    }

    // epilogue: total l over the 4 lanes of this query
    const float lt = sum_xor32(sum_xor16(rs.l));
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    TOut *orow = a.O + head + (size_t)(64 * I + r) * D;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
        store4<TOut>(orow + 16 * dt + 4 * g, rs.acc[dt] * inv);
}

}  // namespace smh
