// Two-level mask encoder on the GPU.
//
// Format ("Accelerating Sparse Transformer Inference on GPU", gist.science
// explainer, Technical summary > Methodology > 1. Unified MHA module,
// storage-format items): 64x64 outer tiles; empty tiles are left out; full
// tiles are listed by column only; partial tiles are listed and carry one
// uint64 bitmap per 8x8 inner tile.  Exact layout: include/smh.h.
//
// Two launches, one workgroup per outer-tile row I in both:
//   1. enc_rows    streams the 64 x S strip of mask rows of I, eight outer
//                  tiles (512 contiguous bytes per mask row) per step with
//                  the next step's loads in flight.  Builds the 64 inner-tile
//                  words of each tile in LDS, counts its valid elements, and
//                  appends the tile to the row's own full or partial list
//                  (row-local positions, ascending J) in scratch, partial
//                  tiles with their 64 words.  Also counts the row's valid
//                  pairs and its query rows without a valid key.
//   2. enc_finish  turns the per-row counts into the row's offsets in the
//                  global lists (a sum over the rows before it), copies the
//                  row's lists and words into place, writes the row
//                  pointers, the row's rank in the heavy-first schedule and,
//                  in the last row's workgroup, the statistics.
// Every value is a pure function of the mask (no atomics, no order
// dependence), so the result is deterministic and equals appending tiles
// row by row, column by column.
#include "smh_internal.h"

namespace smh {
namespace {

constexpr int kT = 8;  // outer tiles per step of enc_rows

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

// 8 mask bytes (two dwords, byte c = column c) -> one 8-bit inner-tile row.
__device__ inline uint32_t row_bits8(uint32_t lo, uint32_t hi) {
    return gather4(nonzero_bytes(lo)) | (gather4(nonzero_bytes(hi)) << 4);
}

struct Scratch {
    int32_t *row_nf, *row_np, *row_empty;
    int64_t *row_nnz;
    int32_t *full_local, *part_local;  // [n][n], row-local lists of J
    uint64_t *words;                   // [n][n][64], row-local order
};

// 256 threads.  Thread t reads, for k = 0..7, mask row 8k + (t >> 5) of the
// strip, bytes 16*(t & 31) .. +15 of the current 8-tile window: tile
// jj = (t & 31) >> 2, columns 16*((t & 31) & 3) .. +15 of that tile.  Each
// wavefront instruction thus reads two contiguous 512-byte row pieces.
__global__ __launch_bounds__(256) void enc_rows(const uint8_t *__restrict__ mask,
                                                int S, int n, Scratch sc) {
    __shared__ uint64_t words[kT][64];
    __shared__ int wsum[kT][4];
    __shared__ uint32_t rows_any[8];
    const int I = blockIdx.x;
    const int t = threadIdx.x, w = t >> 6, lane = t & 63;
    const int r0 = t >> 5, c = t & 31, jj = c >> 2, quarter = c & 3;
    const uint8_t *strip = mask + (size_t)64 * I * S;
    uint8_t *wb = reinterpret_cast<uint8_t *>(&words[0][0]);

    uint4 cur[8], nxt[8];
    auto load = [&](uint4 (&v)[8], int J0) {
        const bool ok = J0 + jj < n;
#pragma unroll
        for (int k = 0; k < 8; ++k)
            v[k] = ok ? *reinterpret_cast<const uint4 *>(
                            strip + (size_t)(8 * k + r0) * S + 64 * J0 + 16 * c)
                      : make_uint4(0, 0, 0, 0);
    };

    uint32_t any_rows = 0;  // bit k: row 8k + r0 has a valid element so far
    int run_f = 0, run_p = 0;
    long long nnz = 0;
    load(cur, 0);
    for (int J0 = 0; J0 < n; J0 += kT) {
        if (J0 + kT < n) load(nxt, J0 + kT);
        int cnt = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            // inner tile (k, 2*quarter) and (k, 2*quarter+1), its row r0
            const uint32_t b0 = row_bits8(cur[k].x, cur[k].y);
            const uint32_t b1 = row_bits8(cur[k].z, cur[k].w);
            wb[jj * 512 + (k * 8 + 2 * quarter) * 8 + r0] = (uint8_t)b0;
            wb[jj * 512 + (k * 8 + 2 * quarter + 1) * 8 + r0] = (uint8_t)b1;
            cnt += __popc(b0) + __popc(b1);
            any_rows |= (uint32_t)((b0 | b1) != 0) << k;
        }
        // lanes of one tile within this wavefront: quarters (xor 1, 2) and
        // the two row offsets (xor 32)
        cnt += __shfl_xor(cnt, 1);
        cnt += __shfl_xor(cnt, 2);
        cnt += __shfl_xor(cnt, 32);
        if (lane < 32 && quarter == 0) wsum[jj][w] = cnt;
        __syncthreads();

        // walk the window's tiles in column order (uniform in every thread)
#pragma unroll
        for (int j = 0; j < kT; ++j) {
            const int J = J0 + j;
            if (J >= n) break;
            const int cj = wsum[j][0] + wsum[j][1] + wsum[j][2] + wsum[j][3];
            if (cj == 0) continue;
            nnz += cj;
            if (cj == 64 * 64) {
                if (t == 0) sc.full_local[(size_t)I * n + run_f] = J;
                ++run_f;
            } else {
                if (t == 0) sc.part_local[(size_t)I * n + run_p] = J;
                if (w == (j & 3))
                    sc.words[((size_t)I * n + run_p) * 64 + lane] = words[j][lane];
                ++run_p;
            }
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < 8; ++k) cur[k] = nxt[k];
    }

    // rows without a valid key: OR the masks of the 32 lanes that share r0
    uint32_t a = any_rows;
#pragma unroll
    for (int off = 1; off < 32; off <<= 1) a |= __shfl_xor(a, off);
    if (c == 0) rows_any[r0] = a;
    __syncthreads();
    if (t == 0) {
        int empty = 0;
        for (int r = 0; r < 8; ++r) empty += 8 - __popc(rows_any[r] & 0xFFu);
        sc.row_nf[I] = run_f;
        sc.row_np[I] = run_p;
        sc.row_nnz[I] = nnz;
        sc.row_empty[I] = empty;
    }
}

template <typename T> __device__ inline T block_sum(T x, T *sh) {
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = x;
    __syncthreads();
    return sh[0] + sh[1] + sh[2] + sh[3];
}

__device__ inline int block_max(int x, int *sh) {
    for (int off = 32; off > 0; off >>= 1) x = max(x, __shfl_xor(x, off));
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = x;
    __syncthreads();
    return max(max(sh[0], sh[1]), max(sh[2], sh[3]));
}

__global__ __launch_bounds__(256) void enc_finish(int n, Scratch sc,
                                                  smh_mask_enc enc) {
    __shared__ int shi[4];
    __shared__ long long shl[4];
    const int I = blockIdx.x, t = threadIdx.x;
    const int nf = sc.row_nf[I], np = sc.row_np[I], ci = nf + np;
    int pf = 0, pp = 0, rank = 0;
    for (int J = t; J < n; J += 256) {
        const int f = sc.row_nf[J], p = sc.row_np[J];
        if (J < I) {
            pf += f;
            pp += p;
        }
        rank += (f + p > ci) || (f + p == ci && J < I);
    }
    pf = block_sum(pf, shi);
    pp = block_sum(pp, shi);
    rank = block_sum(rank, shi);
    if (t == 0) {
        enc.full_row_ptr[I] = pf;
        enc.part_row_ptr[I] = pp;
        enc.row_order[rank] = I;
    }
    if (I == n - 1) {
        long long nnz = 0;
        int empty = 0, mx = 0;
        for (int J = t; J < n; J += 256) {
            nnz += sc.row_nnz[J];
            empty += sc.row_empty[J];
            mx = max(mx, sc.row_nf[J] + sc.row_np[J]);
        }
        nnz = block_sum(nnz, shl);
        empty = block_sum(empty, shi);
        mx = block_max(mx, shi);
        if (t == 0) {
            enc.full_row_ptr[n] = pf + nf;
            enc.part_row_ptr[n] = pp + np;
            enc.stats[0] = nnz;
            enc.stats[1] = pf + nf;
            enc.stats[2] = pp + np;
            enc.stats[3] = empty;
            enc.stats[4] = mx;
        }
    }
    for (int i = t; i < nf; i += 256)
        enc.full_col_idx[pf + i] = sc.full_local[(size_t)I * n + i];
    for (int i = t; i < np; i += 256)
        enc.part_col_idx[pp + i] = sc.part_local[(size_t)I * n + i];
    // the row's partial-tile words are one contiguous block in both places
    const uint4 *src = reinterpret_cast<const uint4 *>(sc.words + (size_t)I * n * 64);
    uint4 *dst = reinterpret_cast<uint4 *>(enc.part_bitmaps + (size_t)pp * 64);
    const int chunks = np * 32;
    for (int e = t; e < chunks; e += 256) dst[e] = src[e];
}

// S == 0: an empty encoding.  Row pointers {0}, all statistics zero.
__global__ void enc_empty(smh_mask_enc enc) {
    if (threadIdx.x == 0) {
        enc.full_row_ptr[0] = 0;
        enc.part_row_ptr[0] = 0;
    }
    if (threadIdx.x < 5) enc.stats[threadIdx.x] = 0;
}

}  // namespace

hipError_t launch_encode(const uint8_t *mask, int32_t S, char *ws,
                         const EncLayout &L, const smh_mask_enc &enc,
                         hipStream_t stream) {
    if (S == 0) {
        hipLaunchKernelGGL(enc_empty, dim3(1), dim3(64), 0, stream, enc);
        return hipGetLastError();
    }
    const int n = (int)L.n;
    Scratch sc;
    sc.row_nf = (int32_t *)(ws + L.row_nf);
    sc.row_np = (int32_t *)(ws + L.row_np);
    sc.row_empty = (int32_t *)(ws + L.row_empty);
    sc.row_nnz = (int64_t *)(ws + L.row_nnz);
    sc.full_local = (int32_t *)(ws + L.full_local);
    sc.part_local = (int32_t *)(ws + L.part_local);
    sc.words = (uint64_t *)(ws + L.tile_words);
    hipLaunchKernelGGL(enc_rows, dim3(n), dim3(256), 0, stream, mask, S, n, sc);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(enc_finish, dim3(n), dim3(256), 0, stream, n, sc, enc);
    return hipGetLastError();
}

}  // namespace smh
