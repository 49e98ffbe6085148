"""Masks given by a pattern, reference side: the dense mask a pattern
describes, written out element by element (vectorised over rows).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The pattern ("Accelerating Sparse Transformer Inference on GPU", gist.science
explainer, Technical summary > Methodology > 1. Unified MHA module: the
format is built from the mask's structure without materialising the whole
sparse matrix; Experimental results: the causal, sliding-window,
Longformer, BigBird and random masks it is measured on) is a union of
parts, limited to the causal triangle when asked.  Element (i, j), i, j < S,
is valid iff

    (not causal or j <= i) and (
        (window >= 0 and |i - j| <= window)
     or i < global_rows or j < global_cols
     or blocks[i // 64, j // 64] == 1
     or (blocks[i // 64, j // 64] not in (0, 1) and u(i, j) < keep16)
     or (blocks[i // 64, j // 64] == 0 and u(i, j) < rand16))

keep16 = floor(block_keep * 65536), rand16 = floor(random_p * 65536), both
in float32; u(i, j) = bits 16 (e % 4) .. +15 of output number e // 4 of
SplitMix64 seeded with `seed`, e = i * S + j.

SplitMix64 (G. L. Steele, D. Lea, C. H. Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014): output k of the stream seeded with s is
mix(s + (k + 1) * 0x9E3779B97F4A7C15), mix(z) = z3 ^ (z3 >> 31) with
z2 = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9, z3 = (z2 ^ (z2 >> 27)) *
0x94D049BB133111EB, all modulo 2^64.
"""
import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
MUL1 = np.uint64(0xBF58476D1CE4E5B9)
MUL2 = np.uint64(0x94D049BB133111EB)


def splitmix64(seed, k):
    """Output number k (array, from 0) of SplitMix64 seeded with `seed`."""
    k = np.asarray(k, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(seed) + (k + np.uint64(1)) * GAMMA
        z = (z ^ (z >> np.uint64(30))) * MUL1
        z = (z ^ (z >> np.uint64(27))) * MUL2
    return z ^ (z >> np.uint64(31))


def threshold16(p):
    """floor(p * 65536) in float32."""
    return int(np.floor(np.float32(p) * np.float32(65536.0)))


def draws16(S, rows, seed):
    """u(i, j) for the given rows (array) and every j < S: [len(rows), S]."""
    i = np.asarray(rows, dtype=np.uint64)[:, None]
    j = np.arange(S, dtype=np.uint64)[None, :]
    e = i * np.uint64(S) + j
    x = splitmix64(seed, e >> np.uint64(2))
    return ((x >> (np.uint64(16) * (e & np.uint64(3)))) &
            np.uint64(0xFFFF)).astype(np.int64)


def pattern_rows(S, rows, causal=False, window=-1, global_rows=0,
                 global_cols=0, blocks=None, block_keep=1.0, random_p=0.0,
                 seed=0):
    """Rows `rows` (array of query indices) of the [S, S] bool mask the
    pattern describes: [len(rows), S].  Element (i, j) is valid iff it is
    in a global row or column, in the band |i - j| <= window, in a block
    of map value 1, or drawn: u(i, j) < floor(block_keep * 65536) in a
    block of another nonzero value, u(i, j) < floor(random_p * 65536)
    elsewhere; then, when causal, only j <= i."""
    S = int(S)
    keep16, rand16 = threshold16(block_keep), threshold16(random_p)
    rows = np.asarray(rows, dtype=np.int64)
    i = rows[:, None]
    j = np.arange(S, dtype=np.int64)[None, :]
    v = (i < global_rows) | (j < global_cols)
    if window >= 0:
        v |= np.abs(i - j) <= window
    blk = (np.asarray(blocks, dtype=np.uint8)[i // 64, j // 64]
           if blocks is not None else np.zeros((len(rows), S), np.uint8))
    v |= blk == 1
    if keep16 > 0 or rand16 > 0:
        u = draws16(S, rows, seed)
        v |= (blk != 0) & (blk != 1) & (u < keep16)
        v |= (blk == 0) & (u < rand16)
    if causal:
        v &= j <= i
    return v


def pattern_mask(S, causal=False, window=-1, global_rows=0, global_cols=0,
                 blocks=None, block_keep=1.0, random_p=0.0, seed=0,
                 row_block=512):
    """The dense [S, S] bool mask the pattern describes (pattern_rows, a
    block of rows at a time)."""
    S = int(S)
    m = np.zeros((S, S), dtype=bool)
    for r0 in range(0, S, row_block):
        rows = np.arange(r0, min(S, r0 + row_block), dtype=np.int64)
        m[r0:r0 + len(rows)] = pattern_rows(S, rows, causal, window,
                                            global_rows, global_cols, blocks,
                                            block_keep, random_p, seed)
    return m
