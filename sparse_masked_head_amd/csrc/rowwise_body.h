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
//   * chunks of 64 entries, lane = entry: the lane's K row against the 8
//     query rows (v_dot2, fp32 accumulation; pairs outside the mask -inf),
//     online softmax per row with 64-lane DPP max reductions (a row with no
//     key in the chunk is skipped), probabilities through LDS, then P V with
//     lane = output column over the chunk's keys, 8 keys per batch with
//     the next batch's V loads in flight.
// A wavefront thus touches K and V only for keys some of its rows see, in
// full 64-key chunks, however the keys are spread over the tiles.
// Probabilities stay in fp32 here.
#pragma once

#include <type_traits>

#include "fwd_common.h"

namespace smh {

constexpr int kRowsPerWave = 8;

// LDS of one wavefront: the 8 query rows, the ring of pending entries and
// the probabilities of one chunk [64 entries][8 rows].
template <int D> struct RowLds {
    static constexpr int CAP = 1024;  // > 63 pending + 8 full tiles (512)
    static constexpr int Q_BYTES = kRowsPerWave * D * 2;
    static constexpr int RING_BYTES = CAP * 4;
    static constexpr int P_BYTES = 64 * kRowsPerWave * 4;
    static constexpr int BYTES = Q_BYTES + RING_BYTES + P_BYTES;
};

// The columns of an inner tile that some of its rows see: bit c set iff
// bit c of any byte of w is (byte r of w is row r).
__device__ inline uint32_t live_columns(uint64_t w) {
    uint32_t t = (uint32_t)w | (uint32_t)(w >> 32);
    t |= t >> 16;
    t |= t >> 8;
    return t & 0xFFu;
}

// Exclusive prefix sum over the wavefront of a per-lane count below 16,
// and the wavefront's total: the count's four bits as ballots, v_mbcnt
// counting the lanes below this one in each (no cross-lane data moves).
__device__ inline int wave_prefix16(int cnt, int &total) {
    int excl = 0, tot = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const uint64_t m = __builtin_amdgcn_ballot_w64((cnt >> b) & 1);
        excl += (int)__builtin_amdgcn_mbcnt_hi(
                    (uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u))
                << b;
        tot += __popcll(m) << b;
    }
    total = tot;
    return excl;
}

// The rows of an inner tile that see its column c: bit r = bit 8r + c of
// w.  Each 32-bit half holds four rows; after the shift and mask their bits
// sit at 0, 8, 16, 24, and the multiply by 2^24 + 2^17 + 2^10 + 2^3 moves
// them to bits 24..27 (the other partial products land below bit 24 at
// distinct places, so nothing carries into those bits).
__device__ inline uint32_t column_rows(uint64_t w, int c) {
    const uint32_t lo = ((uint32_t)w >> c) & 0x01010101u;
    const uint32_t hi = ((uint32_t)(w >> 32) >> c) & 0x01010101u;
    return ((lo * 0x01020408u) >> 24) | (((hi * 0x01020408u) >> 24) << 4);
}

// Softmax state of the wavefront's 8 rows (lane-local partial sums; the
// output columns of this lane).
template <int D> struct RwState {
    static constexpr int E = D / 64;  // output columns per lane
    float m[kRowsPerWave], lp[kRowsPerWave], o[kRowsPerWave][E];
};

// One chunk: entries ring[head .. head+n) (n <= 64), lane = entry.
template <int D, typename TIn>
__device__ __attribute__((always_inline)) inline void rw_chunk(
    RwState<D> &st, const uint32_t *ring, uint32_t head, int n,
    const uint32_t *qbuf, float *pbuf, const TIn *__restrict__ Kh,
    const TIn *__restrict__ Vh, float c) {
    constexpr int R = kRowsPerWave;
    constexpr int E = RwState<D>::E;
    constexpr int CAP = RowLds<D>::CAP;
    const int lane = threadIdx.x & 63;
    const uint32_t ent = lane < n ? ring[(head + lane) & (CAP - 1)] : 0u;
    const uint32_t rb = ent >> 24;
    const int key = (int)(ent & 0xFFFFFFu);

    float s[R];
#pragma unroll
    for (int r = 0; r < R; ++r) s[r] = 0.f;
    if (rb) {
        const u4_t *krow = reinterpret_cast<const u4_t *>(Kh + (size_t)key * D);
        constexpr int H = D / 8 > 8 ? 8 : D / 8;  // 16-byte pieces per half row
#pragma unroll
        for (int h0 = 0; h0 < D / 8; h0 += H) {
            u4_t kc[H];
#pragma unroll
            for (int cc = 0; cc < H; ++cc) kc[cc] = krow[h0 + cc];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                // one query row at a time: keeps its LDS reads from all
                // being scheduled (and held in registers) at once
                __builtin_amdgcn_sched_barrier(0);
                float acc = s[r];
#pragma unroll
                for (int cc = 0; cc < H; ++cc) {
                    const u4_t qc = *reinterpret_cast<const u4_t *>(
                        qbuf + r * (D / 2) + 4 * (h0 + cc));
                    acc = dot2<TIn>(qc[0], kc[cc][0], acc);
                    acc = dot2<TIn>(qc[1], kc[cc][1], acc);
                    acc = dot2<TIn>(qc[2], kc[cc][2], acc);
                    acc = dot2<TIn>(qc[3], kc[cc][3], acc);
                }
                s[r] = acc;
            }
        }
    }
    float p[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        p[r] = 0.f;
        // a row with no key in this chunk keeps its state unchanged
        if (!__builtin_amdgcn_ballot_w64((rb >> r) & 1)) continue;
        const float sr = (rb >> r) & 1 ? s[r] : -INFINITY;
        const float mx = wave_max(sr);
        const float m_new = fmaxf(st.m[r], mx);
        const float alpha = __builtin_amdgcn_exp2f((st.m[r] - m_new) * c);
        st.m[r] = m_new;
        p[r] = __builtin_amdgcn_exp2f(fmaf(sr, c, -m_new * c));
        st.lp[r] = st.lp[r] * alpha + p[r];
#pragma unroll
        for (int e = 0; e < E; ++e) st.o[r][e] *= alpha;
    }
    wave_lds_sync();  // the previous chunk's readers of pbuf are done
    {
        f4_t *dst = reinterpret_cast<f4_t *>(pbuf + lane * R);
        dst[0] = f4_t{p[0], p[1], p[2], p[3]};
        dst[1] = f4_t{p[4], p[5], p[6], p[7]};
    }
    wave_lds_sync();

    // P V: lane = output columns lane*E .. +E-1, 4 entries per batch, the
    // next batch's V loads issued before this batch's products (batches of 8
    // hold more registers and measured slower: fewer wavefronts per SIMD)
    constexpr int BATCH = 4;
    const TIn *vcol = Vh + lane * E;
    TIn vv[3][BATCH][E];
    // The loads are unconditional (an entry past the chunk reads key 0) and
    // keep the raw values; the products convert them and use 0 for entries
    // past the chunk.  A load under a condition, converted in place, ends up
    // in a branch of its own with a wait for it, and the batch's loads
    // would run one after another.
    auto load = [&](int slot, int b0) __attribute__((always_inline)) {
        // a batch's loads stay where they are issued (hoisted together with
        // later batches' they would hold too many registers)
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            const int ei = b0 + u;
            // the same entry in every lane: a scalar, so the load's address
            // is a scalar base plus the lane's column offset
            const uint32_t ent = __builtin_amdgcn_readfirstlane(ring[(head + ei) & (CAP - 1)]);
            const int k = ei < n ? (int)(ent & 0xFFFFFFu) : 0;
            typedef __attribute__((address_space(1))) const TIn gbl_t;
            gbl_t *vk = (gbl_t *)uniform_ptr(Vh + (size_t)k * D);
#pragma unroll
            for (int e = 0; e < E; ++e) vv[slot][u][e] = vk[lane * E + e];
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    auto val = [&](int ei, TIn x) __attribute__((always_inline)) {
        return ei < n ? (float)x : 0.f;
    };
    // products of batch b0 (its values in slot sl, a compile-time constant)
    auto products = [&](auto slc, int b0) __attribute__((always_inline)) {
        constexpr int sl = decltype(slc)::value;
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            const int ei = b0 + u;
            const f4_t pa = *reinterpret_cast<const f4_t *>(pbuf + ei * R);
            const f4_t pb = *reinterpret_cast<const f4_t *>(pbuf + ei * R + 4);
            const float pr[R] = {pa[0], pa[1], pa[2], pa[3], pb[0], pb[1], pb[2], pb[3]};
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int e = 0; e < E; ++e)
                    st.o[r][e] = fmaf(pr[r], val(ei, vv[sl][u][e]), st.o[r][e]);
        }
    };
    // three slots: the loads of batch b + 2 are issued before the products
    // of batch b, so two batches' loads are in flight behind the one in use
    // (with one, every batch waited for most of a memory round trip)
    using C0 = std::integral_constant<int, 0>;
    using C1 = std::integral_constant<int, 1>;
    using C2 = std::integral_constant<int, 2>;
    // (the loads are unconditional, past the chunk too, where they read key
    // 0: a load under a condition makes the compiler wait for every load
    // in flight where the paths join)
    load(0, 0);
    load(1, BATCH);
    for (int b0 = 0; b0 < n; b0 += 3 * BATCH) {
        load(2, b0 + 2 * BATCH);
        products(C0(), b0);
        if (b0 + BATCH >= n) break;
        load(0, b0 + 3 * BATCH);
        products(C1(), b0 + BATCH);
        if (b0 + 2 * BATCH >= n) break;
        load(1, b0 + 4 * BATCH);
        products(C2(), b0 + 2 * BATCH);
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
    constexpr int E = RwState<D>::E;
    constexpr int CAP = RowLds<D>::CAP;
    uint32_t *qbuf = reinterpret_cast<uint32_t *>(slice);  // [R][D/2]
    uint32_t *ring = reinterpret_cast<uint32_t *>(slice + RowLds<D>::Q_BYTES);
    float *pbuf = reinterpret_cast<float *>(slice + RowLds<D>::Q_BYTES + RowLds<D>::RING_BYTES);
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
    for (int r = 0; r < R; ++r) {
        st.m[r] = -INFINITY;
        st.lp[r] = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) st.o[r][e] = 0.f;
    }
    wave_lds_sync();

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
            rw_chunk<D, TIn>(st, ring, head, 64, qbuf, pbuf, Kh, Vh, a.c);
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
        rw_chunk<D, TIn>(st, ring, head, (int)(tail - head), qbuf, pbuf, Kh, Vh, a.c);

#pragma unroll
    for (int r = 0; r < R; ++r) {
        const float lt = wave_sum(st.lp[r]);
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
        TOut *orow = a.O + head_off + (size_t)(row0 + r) * D + lane * E;
        if (row0 + r < a.S) {
#pragma unroll
            for (int e = 0; e < E; ++e) store1<TOut>(orow + e, st.o[r][e] * inv);
        }
    }
    wave_lds_sync();  // the slice may be reused by the next group
}

}  // namespace smh
