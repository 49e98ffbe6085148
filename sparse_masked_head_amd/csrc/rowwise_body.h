// Row-wise sparse attention: the work of one wavefront on 8 query rows,
// used by the row-wise kernel and by the fused kernel that decides on the
// device.
//
// STOF's kernel for highly sparse, short sequences ("Accelerating Sparse
// Transformer Inference on GPU", gist.science explainer, Technical summary >
// Methodology > 1. Unified MHA module, row-wise kernel item: Q is cut into
// rows, each row is handled with intra-warp exchanges only, and there is no
// synchronisation between warps).
//
// The 8 rows are one inner-tile row of an outer-tile row, so for a partial
// outer tile the 8 inner-tile words (ir, 0..7) hold exactly their mask.  The
// wavefront never executes s_barrier; it uses its own slice of LDS.  Its
// work follows the live keys, not the stored tiles:
//   * gather: 8 stored tiles per step, lane = (tile, inner-tile column ic);
//     the OR of the bytes of the lane's 64-bit word gives the keys 8ic + c
//     that some row sees (all of them for a full tile), and for each such
//     key the set of rows seeing it is appended to a ring of pending
//     entries (rows << 24 | key) in LDS (a wave prefix sum places them);
//   * chunks of 64 entries on the matrix cores (rw_chunk): the K rows and
//     V columns of the chunk's keys are gathered straight into MFMA
//     operands, S^T = K Q^T and O^T += V^T P^T with the 8 query rows as 8
//     of the 16 MFMA columns, online softmax per row across the 4 lanes
//     that share it, P rounded to the input type as in the block-wise
//     kernel.
// A wavefront thus touches K and V only for keys some of its rows see, in
// full 64-key chunks, however the keys are spread over the tiles.
#pragma once

#include <type_traits>

#include "fwd_common.h"

namespace smh {

constexpr int kRowsPerWave = 8;

// LDS of one wavefront: the 8 query rows and the ring of pending entries.
template <int D> struct RowLds {
    static constexpr int CAP = 1024;  // > 63 pending + 8 full tiles (512)
    static constexpr int Q_BYTES = kRowsPerWave * D * 2;
    static constexpr int RING_BYTES = CAP * 4;
    static constexpr int BYTES = Q_BYTES + RING_BYTES;
};

// Softmax state of the wavefront's rows on the matrix cores: lane l holds
// row l % 16 (rows 8..15 are padding) and of its O^T the outputs d = 16dt
// + 4(l/16) + i; the running max, its exponent offset (m * c, or 0 while
// m is -inf) and the lane's part of the row sum.
template <int D> struct RwState {
    f4_t acc[D / 16];
    float m, mc, l;
};

// One chunk: entries ring[head .. head+n) (n <= 64; head is a multiple of
// 64, so the ring reads below are aligned and never wrap).  With lane l =
// (row lq = l % 16, group g = l / 16) and the 64 entries as four 16-key
// blocks st:
//   S^T = K Q^T with v_mfma_f32_16x16x32: A = the K rows of block st's
//     entries (lane: entry 16st + lq, d = 32s + 8g .. +7, straight from
//     global memory), B = the 8 query rows (zero rows 8..15) in registers;
//     lane l gets row lq's scores against entries 16st + 4g + i, which
//     start at -inf where the entry is past the chunk or its row set lacks
//     row lq;
//   online softmax per row across the 4 lanes sharing it (lazy rescale as
//     in the block-wise kernel), P rounded to the input type;
//   O^T += V^T P^T: B = P^T straight from the score registers (k-slot
//     order: entries 32u + 4g + j, then 32u + 16 + 4g + j), A = V^T with
//     the same slot order, each lane gathering its column 16dt + lq of
//     those 8 entries' V rows.
template <int D, typename TIn>
__device__ __attribute__((always_inline)) inline void rw_chunk(
    RwState<D> &st, const uint32_t *ring, uint32_t head, int n,
    const typename Frag<TIn>::type (&qf)[D / 32], const TIn *__restrict__ Kh,
    const TIn *__restrict__ Vh, float c, int S) {
    using F = Frag<TIn>;
    using frag = typename F::type;
    constexpr int CAP = RowLds<D>::CAP;
    const int lane = threadIdx.x & 63, lq = lane & 15, g = lane >> 4;
    u4_t ent[4];      // entries 16st + 4g + i
    uint32_t ka[4];   // entry 16st + lq (the K row this lane supplies)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        ent[b] = *reinterpret_cast<const u4_t *>(ring + ((head + 16 * b + 4 * g) & (CAP - 1)));
        ka[b] = ring[(head + 16 * b + lq) & (CAP - 1)];
    }
    // The key of entry ei, clamped into the head's S rows: an encoding that
    // is not this library's (bits set past S in a tile cut by S) then gives
    // wrong numbers, never a read outside K and V.  Past the chunk: any row.
    auto key_of = [&](int ei, uint32_t e) __attribute__((always_inline)) {
        return ei < n ? min((int)(e & 0xFFFFFFu), S - 1) : 0;
    };

    f4_t sc[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        f4_t c0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // rows lq >= 8 are padding: no entry's row set holds them (and
            // the shift below stays under 32)
            const bool ok = 16 * b + 4 * g + i < n && lq < 8 &&
                            ((ent[b][i] >> (24 + (lq & 7))) & 1u);
            c0[i] = ok ? 0.f : -INFINITY;
        }
        const frag *krow = reinterpret_cast<const frag *>(
            Kh + (size_t)key_of(16 * b + lq, ka[b]) * D);
        sc[b] = F::mfma(krow[g], qf[0], c0);
#pragma unroll
        for (int s2 = 1; s2 < D / 32; ++s2) sc[b] = F::mfma(krow[4 * s2 + g], qf[s2], sc[b]);
    }

    float mx = -INFINITY;
#pragma unroll
    for (int b = 0; b < 4; ++b)
        mx = fmaxf(fmaxf(mx, fmaxf(sc[b][0], sc[b][1])), fmaxf(sc[b][2], sc[b][3]));
    mx = max_xor32(max_xor16(mx));
    // (mx - m) * c is NaN (no move) when both are -inf, +inf when only m is
    const bool grow = (mx - st.m) * c > 8.f;
    if (__builtin_amdgcn_ballot_w64(grow)) {
        const float alpha = grow ? __builtin_amdgcn_exp2f((st.m - mx) * c) : 1.f;
        st.m = grow ? mx : st.m;
        st.mc = grow ? mx * c : st.mc;
        st.l *= alpha;
#pragma unroll
        for (int i = 0; i < D / 16; ++i) st.acc[i] *= alpha;
    }
    frag pf[2];
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            pf[b >> 1][(b & 1) * 4 + i] =
                (TIn)__builtin_amdgcn_exp2f(fmaf(sc[b][i], c, -st.mc));
    float lsum = st.l;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        uint32_t pw[4];
        __builtin_memcpy(pw, &pf[u], 16);
#pragma unroll
        for (int j = 0; j < 4; ++j) lsum = sum2<TIn>(pw[j], lsum);
    }
    st.l = lsum;

#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            frag va;
#pragma unroll
            for (int sl = 0; sl < 8; ++sl) {
                const int b = 2 * u + (sl >> 2), i = sl & 3;
                va[sl] = Vh[(size_t)key_of(16 * b + 4 * g + i, ent[b][i]) * D + 16 * dt + lq];
            }
            st.acc[dt] = F::mfma(va, pf[u], st.acc[dt]);
        }
    }
}

// Wavefront work: inner-tile row ir of an encoding row (outer-tile row I
// of its mask, summary ri) of head bh.  Query rows past S (S cuts the last
// outer tile) see no key, read zeros for Q and are not stored.
template <int D, typename TIn, typename TOut>
__device__ __attribute__((always_inline)) inline void rowwise_group(
    const FwdArgs<TIn, TOut> &a, char *slice, int I, int ir, int bh,
    const RowInfo &ri) {
    constexpr int R = kRowsPerWave;
    constexpr int CAP = RowLds<D>::CAP;
    uint32_t *qbuf = reinterpret_cast<uint32_t *>(slice);  // [R][D/2]
    uint32_t *ring = reinterpret_cast<uint32_t *>(slice + RowLds<D>::Q_BYTES);
    const int lane = threadIdx.x & 63;
    const int row0 = 64 * I + 8 * ir;
    const size_t head_off = (size_t)bh * a.S * D;
    const TIn *Kh = a.K + head_off, *Vh = a.V + head_off;
    const int nmax = a.n - 1;

    {  // stage the 8 query rows (contiguous) into the slice
        const u4_t *src = reinterpret_cast<const u4_t *>(a.Q + head_off + (size_t)row0 * D);
        u4_t *dst = reinterpret_cast<u4_t *>(qbuf);
        for (int e = lane; e < R * D / 8; e += 64)
            dst[e] = row0 + e / (D / 8) < a.S ? src[e] : u4_t{0, 0, 0, 0};
    }

    const int f0 = ri.f0, nF = ri.nF, p0 = ri.p0, nP = ri.nP;
    const int nT = nF + nP;

    RwState<D> st;
#pragma unroll
    for (int i = 0; i < D / 16; ++i) st.acc[i] = f4_t{0.f, 0.f, 0.f, 0.f};
    st.m = -INFINITY;
    st.mc = 0.f;
    st.l = 0.f;
    wave_lds_sync();
    // the query rows as the B operand of S^T = K Q^T: lane l holds row l % 16
    // (zero for rows 8..15), d = 32s + 8(l/16) .. +7
    using frag = typename Frag<TIn>::type;
    const int lq = lane & 15, g = lane >> 4;
    frag qf[D / 32];
#pragma unroll
    for (int s2 = 0; s2 < D / 32; ++s2) {
        const frag *qrow = reinterpret_cast<const frag *>(
            reinterpret_cast<const TIn *>(qbuf) + (lq & (R - 1)) * D);
        const frag q = qrow[4 * s2 + g];
        qf[s2] = lq < R ? q : frag{};
    }

    // gather step: tile t0 + lane/8, inner-tile column lane%8; the loads of
    // the next step are issued before this step's work.  They are
    // unconditional (a lane past the row, or a full tile's word, reads the
    // row summary instead) and their values are replaced and clamped where
    // they are used, and the loop is unrolled by two so that the next
    // step's registers are never copied: a load made conditional, a value
    // changed where it is loaded, or a copy of the register makes the
    // compiler wait for the load right there (a full round trip per step).
    const int ic = lane & 7;
    const int32_t *any32 = a.info;
    const uint64_t *any64 = reinterpret_cast<const uint64_t *>(a.info);
    auto fetch = [&](int t0, int32_t &jr, uint64_t &wr) __attribute__((always_inline)) {
        const int tile = t0 + (lane >> 3);
        const bool full = tile < nF, part = tile >= nF && tile < nT;
        const int32_t *jp = full ? a.fci + f0 + tile
                                 : part ? a.pci + p0 + (tile - nF) : any32;
        const uint64_t *wp =
            part ? a.bm + (size_t)(p0 + tile - nF) * 64 + ir * 8 + ic : any64;
        jr = *jp;
        wr = *wp;
    };
    uint32_t head = 0, tail = 0;  // ring positions (uniform)
    auto step = [&](int t0, const int32_t jr, const uint64_t wr, int32_t &jn,
                    uint64_t &wn) __attribute__((always_inline)) {
        fetch(t0 + 8, jn, wn);  // past the row: the row summary, unused
        const int tile = t0 + (lane >> 3);
        const int J = (int)min((unsigned)jr, (unsigned)nmax);  // never outside K, V
        const uint64_t w = tile >= nT ? 0ull : tile < nF ? ~0ull : wr;
        const uint32_t nzb = live_columns(w);
        int total;
        uint32_t pos = tail + (uint32_t)wave_prefix16(__popc(nzb), total);
        uint32_t m = nzb;
        while (m) {
            const int cb = __builtin_ctz(m);
            m &= m - 1;
            const uint32_t rbits = column_rows(w, cb);
            ring[pos & (CAP - 1)] = (rbits << 24) | (uint32_t)(64 * J + 8 * ic + cb);
            ++pos;
        }
        tail += (uint32_t)total;
        wave_lds_sync();
        while (tail - head >= 64) {
            rw_chunk<D, TIn>(st, ring, head, 64, qf, Kh, Vh, a.c, a.S);
            head += 64;
        }
    };
    int32_t ja = 0, jb = 0;
    uint64_t wa = 0, wb = 0;
    fetch(0, ja, wa);
    for (int t0 = 0; t0 < nT; t0 += 16) {
        step(t0, ja, wa, jb, wb);
        if (t0 + 8 >= nT) break;
        step(t0 + 8, jb, wb, ja, wa);
    }
    if (tail != head)
        rw_chunk<D, TIn>(st, ring, head, (int)(tail - head), qf, Kh, Vh, a.c, a.S);

    // total l of each row over its 4 lanes; rows 8..15 are not stored
    const float lt = sum_xor32(sum_xor16(st.l));
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    if (lq < R && row0 + lq < a.S) {
        TOut *orow = a.O + head_off + (size_t)(row0 + lq) * D + 4 * g;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) store4<TOut>(orow + 16 * dt, st.acc[dt] * inv);
    }
    wave_lds_sync();  // the slice may be reused by the next group
}

}  // namespace smh
