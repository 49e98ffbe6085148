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
// wavefront never executes s_barrier; it uses its own slice of LDS (query
// rows and probabilities).  Per outer tile J (full tiles, then partial):
//   * lane j owns key 64J + j and builds the 8-bit set of rows that see it
//     (all rows for a full tile; a byte gather from the words otherwise); a
//     lane whose set is empty loads nothing;
//   * scores: lane j dots its K row with the 8 query rows (v_dot2, fp32
//     accumulation); pairs outside the mask get -inf;
//   * online softmax per row with 64-lane DPP max reductions; a row with
//     no key in the tile is skipped;
//   * P V with lane = output column: the probabilities pass through the LDS
//     slice and the wavefront walks only the keys some row sees (the ballot
//     of non-empty lanes), four keys per step so their V loads overlap.
// Probabilities stay in fp32 here.
#pragma once

#include "fwd_common.h"

namespace smh {

constexpr int kRowsPerWave = 8;

// LDS of one wavefront: probabilities [64 keys][8 rows] and 8 query rows.
template <int D> struct RowLds {
    static constexpr int P_BYTES = 64 * kRowsPerWave * 4;
    static constexpr int Q_BYTES = kRowsPerWave * D * 2;
    static constexpr int BYTES = P_BYTES + Q_BYTES;
};

template <int D, typename TIn, typename TOut>
__device__ __attribute__((always_inline)) inline void rowwise_group(
    const FwdArgs<TIn, TOut> &a, char *slice, int I, int ir, int bh) {
    constexpr int R = kRowsPerWave;
    constexpr int E = D / 64;  // output columns per lane
    float *pbuf = reinterpret_cast<float *>(slice);              // [64][R]
    uint32_t *qbuf = reinterpret_cast<uint32_t *>(slice + RowLds<D>::P_BYTES);  // [R][D/2]
    const int lane = threadIdx.x & 63;
    const int row0 = 64 * I + 8 * ir;
    const size_t head = (size_t)bh * a.S * D;
    const TIn *Kh = a.K + head, *Vh = a.V + head;

    {  // stage the 8 query rows (contiguous) into the slice
        const u4_t *src = reinterpret_cast<const u4_t *>(a.Q + head + (size_t)row0 * D);
        u4_t *dst = reinterpret_cast<u4_t *>(qbuf);
        for (int e = lane; e < R * D / 8; e += 64) dst[e] = src[e];
    }
    wave_lds_sync();

    const int f0 = a.frp[I], nF = a.frp[I + 1] - f0;
    const int p0 = a.prp[I], nP = a.prp[I + 1] - p0;
    const int nT = nF + nP;

    float m[R], lp[R], o[R][E];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        m[r] = -INFINITY;
        lp[r] = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) o[r][e] = 0.f;
    }

    for (int it = 0; it < nT; ++it) {
        const bool partial = it >= nF;
        const int J = partial ? a.pci[p0 + it - nF] : a.fci[f0 + it];
        uint32_t rb = 0xFFu;  // rows that see key 64J + lane
        if (partial) {
            const uint64_t wd = a.bm[(size_t)(p0 + it - nF) * 64 + ir * 8 + (lane >> 3)];
            // bit 8r + (lane&7) of the word -> bit r: keep the chosen bit of
            // each byte, then one multiply gathers the 8 byte-LSBs into the
            // top byte (no two partial products meet in bits 56..63)
            const uint64_t x = (wd >> (lane & 7)) & 0x0101010101010101ull;
            rb = (uint32_t)((x * 0x0102040810204080ull) >> 56);
        }

        float s[R];
#pragma unroll
        for (int r = 0; r < R; ++r) s[r] = 0.f;
        if (rb) {
            const u4_t *krow = reinterpret_cast<const u4_t *>(Kh + (size_t)(64 * J + lane) * D);
#pragma unroll 4
            for (int cc = 0; cc < D / 8; ++cc) {
                const u4_t kc = krow[cc];
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const u4_t qc = *reinterpret_cast<const u4_t *>(qbuf + r * (D / 2) + 4 * cc);
                    float acc = s[r];
                    acc = dot2<TIn>(qc[0], kc[0], acc);
                    acc = dot2<TIn>(qc[1], kc[1], acc);
                    acc = dot2<TIn>(qc[2], kc[2], acc);
                    acc = dot2<TIn>(qc[3], kc[3], acc);
                    s[r] = acc;
                }
            }
        }
        float p[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            p[r] = 0.f;
            // a row with no key in this tile keeps its state unchanged
            if (!__builtin_amdgcn_ballot_w64((rb >> r) & 1)) continue;
            const float sr = (rb >> r) & 1 ? s[r] : -INFINITY;
            const float mx = wave_max(sr);
            const float m_new = fmaxf(m[r], mx);
            const float m_use = m_new == -INFINITY ? 0.f : m_new;
            const float alpha = __builtin_amdgcn_exp2f((m[r] - m_use) * a.c);
            m[r] = m_new;
            p[r] = __builtin_amdgcn_exp2f(fmaf(sr, a.c, -m_use * a.c));
            lp[r] = lp[r] * alpha + p[r];
#pragma unroll
            for (int e = 0; e < E; ++e) o[r][e] *= alpha;
        }
        wave_lds_sync();  // the previous tile's readers of pbuf are done
        {
            f4_t *dst = reinterpret_cast<f4_t *>(pbuf + lane * R);
            dst[0] = f4_t{p[0], p[1], p[2], p[3]};
            dst[1] = f4_t{p[4], p[5], p[6], p[7]};
        }
        wave_lds_sync();

        uint64_t live = __ballot(rb != 0);
        const TIn *vt = Vh + (size_t)64 * J * D + lane * E;
        while (live) {
            int js[4];
            float vv[4][E];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                js[u] = live ? __builtin_ctzll(live) : -1;
                if (live) live &= live - 1;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int e = 0; e < E; ++e)
                    vv[u][e] = js[u] >= 0 ? (float)vt[(size_t)js[u] * D + e] : 0.f;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (js[u] < 0) break;
                const f4_t pa = *reinterpret_cast<const f4_t *>(pbuf + js[u] * R);
                const f4_t pb = *reinterpret_cast<const f4_t *>(pbuf + js[u] * R + 4);
                const float pr[R] = {pa[0], pa[1], pa[2], pa[3], pb[0], pb[1], pb[2], pb[3]};
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int e = 0; e < E; ++e) o[r][e] = fmaf(pr[r], vv[u][e], o[r][e]);
            }
        }
    }

#pragma unroll
    for (int r = 0; r < R; ++r) {
        const float lt = wave_sum(lp[r]);
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
        TOut *orow = a.O + head + (size_t)(row0 + r) * D + lane * E;
#pragma unroll
        for (int e = 0; e < E; ++e) store1<TOut>(orow + e, o[r][e] * inv);
    }
    wave_lds_sync();  // the slice may be reused by the next group
}

}  // namespace smh
