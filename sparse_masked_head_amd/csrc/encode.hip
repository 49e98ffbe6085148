// Two-level mask encoder on the GPU.
//
// Format ("Accelerating Sparse Transformer Inference on GPU", gist.science
// explainer, Technical summary > Methodology > 1. Unified MHA module,
// storage-format items): 64x64 outer tiles; empty tiles are left out; full
// tiles are listed by column only; partial tiles are listed and carry one
// uint64 bitmap per 8x8 inner tile.  Exact layout: include/smh.h.
//
// Three launches:
//   1. enc_tiles   one workgroup per outer tile: reads the 4 KiB of mask,
//                  builds the 64 inner-tile words in LDS, counts the valid
//                  elements, records which of the 64 tile rows have any
//                  valid element, and parks the words of a partial tile in
//                  scratch.
//   2. enc_scan    one workgroup: exclusive scans of the full / partial
//                  flags in row-major tile order give every stored tile its
//                  list position and the CSR row pointers; also the
//                  statistics and the heavy-first row order.
//   3. enc_compact one wavefront per tile: writes column indices and moves
//                  the partial tiles' words to their final place.
// The positions come from a scan in fixed tile order, so the result is
// deterministic and identical to appending tiles row by row, column by
// column.
#include "smh_internal.h"

namespace smh {
namespace {

constexpr int kScanThreads = 1024;

// High bit of each byte of w set iff that byte is nonzero.
__device__ inline uint32_t nonzero_bytes(uint32_t w) {
    return (((w & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | w) & 0x80808080u;
}

// Collapse the four byte flags of nonzero_bytes() into bits 0..3.
// After the shift the flags sit at bits 0, 8, 16, 24; multiplying by
// 1 + 2^7 + 2^14 + 2^21 moves flag k to bit 21 + k with no carries.
__device__ inline uint32_t gather4(uint32_t hb) {
    return ((hb >> 7) * 0x00204081u >> 21) & 0xFu;
}

// 8 mask bytes (two dwords, byte c = column c) -> 8-bit row of an inner tile.
__device__ inline uint32_t row_bits8(uint32_t lo, uint32_t hi) {
    return gather4(nonzero_bytes(lo)) | (gather4(nonzero_bytes(hi)) << 4);
}

__global__ __launch_bounds__(256) void enc_tiles(
    const uint8_t *__restrict__ mask, int S, int n, int32_t *__restrict__ cnt,
    uint64_t *__restrict__ rowany, uint64_t *__restrict__ tile_words) {
    __shared__ uint64_t words[64];  // inner tile ir*8+ic, byte r = its row r
    __shared__ int wsum[4];
    const int tile = blockIdx.x;
    const int I = tile / n, J = tile - I * n;
    const int t = threadIdx.x;
    const int row = t >> 2, quarter = t & 3;  // 4 threads per tile row

    const uint4 v = *reinterpret_cast<const uint4 *>(
        mask + (size_t)(64 * I + row) * S + 64 * J + 16 * quarter);
    const uint32_t b0 = row_bits8(v.x, v.y);  // inner-tile column 2*quarter
    const uint32_t b1 = row_bits8(v.z, v.w);  // inner-tile column 2*quarter+1
    uint8_t *wb = reinterpret_cast<uint8_t *>(words);
    const int ir = row >> 3, r = row & 7;
    wb[(ir * 8 + 2 * quarter) * 8 + r] = (uint8_t)b0;
    wb[(ir * 8 + 2 * quarter + 1) * 8 + r] = (uint8_t)b1;

    int c = __popc(b0) + __popc(b1);
    for (int off = 32; off > 0; off >>= 1) c += __shfl_xor(c, off);
    if ((t & 63) == 0) wsum[t >> 6] = c;
    __syncthreads();
    const int total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
    if (t < 64) {
        // rows: thread t checks tile row t across the 8 inner-tile columns
        uint32_t any = 0;
        for (int ic = 0; ic < 8; ++ic)
            any |= wb[((t >> 3) * 8 + ic) * 8 + (t & 7)];
        const uint64_t ball = __ballot(any != 0);
        if (t == 0) {
            cnt[tile] = total;
            rowany[tile] = ball;
        }
        if (total > 0 && total < 64 * 64)
            tile_words[(size_t)tile * 64 + t] = words[t];
    }
}

// Exclusive scan of one int per thread across the workgroup (1024 threads).
__device__ inline int block_exclusive_scan(int x, int *sh, int *total) {
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    int incl = x;
    for (int off = 1; off < 64; off <<= 1) {
        int y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
    }
    if (lane == 63) sh[wv] = incl;
    __syncthreads();
    if (t < 64) {
        int w = t < kScanThreads / 64 ? sh[t] : 0;
        int wi = w;
        for (int off = 1; off < 64; off <<= 1) {
            int y = __shfl_up(wi, off);
            if (lane >= off) wi += y;
        }
        sh[64 + t] = wi - w;  // exclusive prefix of wave totals
        if (t == kScanThreads / 64 - 1) sh[128] = wi;
    }
    __syncthreads();
    const int res = sh[64 + wv] + incl - x;
    *total = sh[128];
    __syncthreads();
    return res;
}

__device__ inline long long block_sum64(long long x, long long *sh) {
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = x;
    __syncthreads();
    long long s = 0;
    for (int i = 0; i < kScanThreads / 64; ++i) s += sh[i];
    __syncthreads();
    return s;
}

__global__ __launch_bounds__(kScanThreads) void enc_scan(
    int n, const int32_t *__restrict__ cnt, const uint64_t *__restrict__ rowany,
    int32_t *__restrict__ pos, int32_t *__restrict__ full_row_ptr,
    int32_t *__restrict__ part_row_ptr, int64_t *__restrict__ stats,
    int32_t *__restrict__ row_order) {
    extern __shared__ int rowcnt[];  // [n]
    __shared__ int shf[160], shp[160];
    __shared__ long long sh64[kScanThreads / 64];
    const int t = threadIdx.x;
    const long long n2 = (long long)n * n;
    const long long chunk = (n2 + kScanThreads - 1) / kScanThreads;
    const long long lo = min(n2, chunk * t), hi = min(n2, lo + chunk);

    int nf = 0, np = 0;
    long long nnz = 0;
    for (long long e = lo; e < hi; ++e) {
        const int c = cnt[e];
        nnz += c;
        nf += c == 64 * 64;
        np += c > 0 && c < 64 * 64;
    }
    int tot_f, tot_p;
    int bf = block_exclusive_scan(nf, shf, &tot_f);
    int bp = block_exclusive_scan(np, shp, &tot_p);
    for (long long e = lo; e < hi; ++e) {
        const int c = cnt[e];
        if (e % n == 0) {
            full_row_ptr[e / n] = bf;
            part_row_ptr[e / n] = bp;
        }
        if (c == 64 * 64)
            pos[e] = bf++;
        else if (c > 0)
            pos[e] = bp++;
    }
    if (t == 0) {
        full_row_ptr[n] = tot_f;
        part_row_ptr[n] = tot_p;
    }

    // rows with no valid key: per outer-tile row, OR the row masks
    long long empty = 0;
    for (int I = t; I < n; I += kScanThreads) {
        uint64_t any = 0;
        int stored = 0;
        for (int J = 0; J < n; ++J) {
            any |= rowany[(size_t)I * n + J];
            stored += cnt[(size_t)I * n + J] > 0;
        }
        empty += __popcll(~any);
        rowcnt[I] = stored;
    }
    const long long nnz_all = block_sum64(nnz, sh64);
    const long long empty_all = block_sum64(empty, sh64);
    __syncthreads();
    long long mrt = 0;
    for (int I = t; I < n; I += kScanThreads) mrt = max(mrt, (long long)rowcnt[I]);
    for (int off = 32; off > 0; off >>= 1) mrt = max(mrt, __shfl_xor(mrt, off));
    if ((t & 63) == 0) sh64[t >> 6] = mrt;
    __syncthreads();
    if (t == 0) {
        long long mx = 0;
        for (int i = 0; i < kScanThreads / 64; ++i) mx = max(mx, sh64[i]);
        stats[0] = nnz_all;
        stats[1] = tot_f;
        stats[2] = tot_p;
        stats[3] = empty_all;
        stats[4] = mx;
    }
    __syncthreads();
    // heavy-first schedule: rank = number of rows that sort before row I
    for (int I = t; I < n; I += kScanThreads) {
        const int ci = rowcnt[I];
        int rank = 0;
        for (int I2 = 0; I2 < n; ++I2) {
            const int c2 = rowcnt[I2];
            rank += (c2 > ci) || (c2 == ci && I2 < I);
        }
        row_order[rank] = I;
    }
}

__global__ __launch_bounds__(256) void enc_compact(
    int n, const int32_t *__restrict__ cnt, const int32_t *__restrict__ pos,
    const uint64_t *__restrict__ tile_words, int32_t *__restrict__ full_col_idx,
    int32_t *__restrict__ part_col_idx, uint64_t *__restrict__ part_bitmaps) {
    const long long n2 = (long long)n * n;
    const long long tile = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (tile >= n2) return;
    const int c = cnt[tile];
    if (c == 0) return;
    const int p = pos[tile];
    const int J = (int)(tile % n);
    if (c == 64 * 64) {
        if (lane == 0) full_col_idx[p] = J;
        return;
    }
    if (lane == 0) part_col_idx[p] = J;
    part_bitmaps[(size_t)p * 64 + lane] = tile_words[tile * 64 + lane];
}

// S == 0: an empty encoding.  Row pointers {0}, all statistics zero.
__global__ void enc_empty(int32_t *full_row_ptr, int32_t *part_row_ptr,
                          int64_t *stats) {
    if (threadIdx.x == 0) {
        full_row_ptr[0] = 0;
        part_row_ptr[0] = 0;
    }
    if (threadIdx.x < 5) stats[threadIdx.x] = 0;
}

}  // namespace

hipError_t launch_encode(const uint8_t *mask, int32_t S, char *ws,
                         const EncLayout &L, hipStream_t stream) {
    auto at = [&](size_t off) { return ws + off; };
    int32_t *frp = (int32_t *)at(L.full_row_ptr);
    int32_t *prp = (int32_t *)at(L.part_row_ptr);
    int64_t *stats = (int64_t *)at(L.stats);
    if (S == 0) {
        hipLaunchKernelGGL(enc_empty, dim3(1), dim3(64), 0, stream, frp, prp,
                           stats);
        return hipGetLastError();
    }
    const int n = (int)L.n;
    const long long n2 = (long long)n * n;
    int32_t *cnt = (int32_t *)at(L.tile_cnt);
    uint64_t *rowany = (uint64_t *)at(L.tile_rowany);
    int32_t *pos = (int32_t *)at(L.tile_pos);
    uint64_t *tw = (uint64_t *)at(L.tile_bitmaps);
    hipLaunchKernelGGL(enc_tiles, dim3((unsigned)n2), dim3(256), 0, stream,
                       mask, S, n, cnt, rowany, tw);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(enc_scan, dim3(1), dim3(kScanThreads),
                       sizeof(int) * n, stream, n, cnt, rowany, pos, frp, prp,
                       stats, (int32_t *)at(L.row_order));
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(enc_compact, dim3((unsigned)((n2 + 3) / 4)), dim3(256),
                       0, stream, n, cnt, pos, tw, (int32_t *)at(L.full_col_idx),
                       (int32_t *)at(L.part_col_idx),
                       (uint64_t *)at(L.part_bitmaps));
    return hipGetLastError();
}

}  // namespace smh
