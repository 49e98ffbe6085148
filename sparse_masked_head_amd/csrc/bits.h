// Bit manipulation of inner-tile words (bit 8r + c = row r, column c of
// an 8 x 8 inner tile) and a wavefront prefix sum, shared by the encoder
// (row-wise entries) and the attention kernels (gather steps).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace smh {

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
    // counts of 0 or 1 only (the common case for a sparse mask): one ballot
    const uint64_t any = __builtin_amdgcn_ballot_w64(cnt != 0);
    if (__builtin_amdgcn_ballot_w64(cnt > 1) == 0) {
        total = __popcll(any);
        return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(any >> 32),
                                              __builtin_amdgcn_mbcnt_lo((uint32_t)any, 0u));
    }
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

}  // namespace smh
