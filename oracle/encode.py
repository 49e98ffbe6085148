"""Two-level mask encoding, reference side.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

``encode_c`` runs the scalar C loop in ``encode_ref.c`` (built by
``oracle.build``); ``encode_py`` is a pure-Python twin of the same
definition for small masks, written independently of the C loop;
``encode_stack`` encodes a stack of masks [Bm, Hm, S, S] (one per sequence
and/or head) as the masks' encodings one after another.  All return a
dict:

    full_row_ptr  int32 [n_ot+1]     full_col_idx  int32 [n_full]
    part_row_ptr  int32 [n_ot+1]     part_col_idx  int32 [n_partial]
    part_bitmaps  uint64 [n_partial, 64]
    nnz, n_full, n_partial, n_empty_rows   (Python ints)

Definition ("Accelerating Sparse Transformer Inference on GPU", gist.science
explainer, Technical summary > Methodology > 1. Unified MHA module,
storage-format items): 64x64 outer tiles; empty ones skipped; all-valid ones
listed as full; the rest listed as partial with one uint64 per 8x8 inner
tile, inner tile (ir, ic) stored at position 8*ir+ic, element (r, c) of an
inner tile at bit 8*r+c.  For S not a multiple of 64 the tiles cover
ceil(S/64)*64 rows and columns and elements outside the S x S mask are not
valid.
"""
import ctypes
import os

import numpy as np

OT = 64
IT = 8

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libencref.so")
_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build
            build.build()
        lib = ctypes.CDLL(LIB_PATH)
        p = ctypes.c_void_p
        lib.ref_encode.argtypes = [p, ctypes.c_int64, p, p, p, p, p, p]
        lib.ref_encode.restype = ctypes.c_int
        _lib = lib
    return _lib


def encode_c(mask):
    """Scalar C encoder.  mask: [S, S] bool/uint8 numpy array."""
    m = np.ascontiguousarray(np.asarray(mask).astype(np.uint8, copy=False))
    S = m.shape[0]
    assert m.shape == (S, S)
    if S <= 0:
        raise ValueError("S must be positive")
    n = (S + OT - 1) // OT
    frp = np.zeros(n + 1, np.int32)
    prp = np.zeros(n + 1, np.int32)
    fci = np.zeros(n * n, np.int32)
    pci = np.zeros(n * n, np.int32)
    bm = np.zeros((n * n, 64), np.uint64)
    st = np.zeros(4, np.int64)
    rc = _load().ref_encode(m.ctypes.data, S, frp.ctypes.data, fci.ctypes.data,
                            prp.ctypes.data, pci.ctypes.data, bm.ctypes.data,
                            st.ctypes.data)
    if rc != 0:
        raise ValueError("ref_encode rejected the mask")
    nf, npart = int(st[1]), int(st[2])
    return dict(full_row_ptr=frp, full_col_idx=fci[:nf].copy(),
                part_row_ptr=prp, part_col_idx=pci[:npart].copy(),
                part_bitmaps=bm[:npart].copy(), nnz=int(st[0]), n_full=nf,
                n_partial=npart, n_empty_rows=int(st[3]))


def encode_py(mask):
    """Pure-Python twin, element by element (small masks only)."""
    m = np.asarray(mask).astype(bool)
    S = m.shape[0]
    if S <= 0:
        raise ValueError("S must be positive")
    n = -(-S // OT)

    def at(i, j):  # elements outside the S x S mask are not valid
        return i < S and j < S and bool(m[i, j])
    frp, fci, prp, pci, bms = [0], [], [0], [], []
    nnz = 0
    for I in range(n):
        for J in range(n):
            tile = [[at(OT * I + r, OT * J + c) for c in range(OT)]
                    for r in range(OT)]
            cnt = sum(sum(row) for row in tile)
            nnz += cnt
            if cnt == 0:
                continue
            if cnt == OT * OT:
                fci.append(J)
                continue
            words = []
            for ir in range(IT):
                for ic in range(IT):
                    w = 0
                    for r in range(IT):
                        for c in range(IT):
                            if tile[IT * ir + r][IT * ic + c]:
                                w |= 1 << (IT * r + c)
                    words.append(w)
            pci.append(J)
            bms.append(words)
        frp.append(len(fci))
        prp.append(len(pci))
    empty = sum(1 for i in range(S) if not any(bool(x) for x in m[i]))
    return dict(full_row_ptr=np.array(frp, np.int32),
                full_col_idx=np.array(fci, np.int32),
                part_row_ptr=np.array(prp, np.int32),
                part_col_idx=np.array(pci, np.int32),
                part_bitmaps=np.array(bms, np.uint64).reshape(-1, 64),
                nnz=nnz, n_full=len(fci), n_partial=len(pci),
                n_empty_rows=empty)


def encode_stack(masks, encode=None):
    """Encoding of a stack of masks [Bm, Hm, S, S]: the rows of mask
    g = gb * Hm + gh follow those of mask g - 1, so the row pointers of
    mask g are its own offset by the tiles of the masks before it, and the
    lists and bitmaps are concatenated in that order.  Counts are totals.
    Row g * n_ot + I of the result is outer-tile row I of mask g."""
    encode = encode_c if encode is None else encode
    m = np.asarray(masks)
    assert m.ndim == 4 and m.shape[2] == m.shape[3]
    parts = [encode(m[gb, gh]) for gb in range(m.shape[0])
             for gh in range(m.shape[1])]
    out = {}
    for key in ("full", "part"):
        ptrs, cols, base = [np.zeros(1, np.int32)], [], 0
        for e in parts:
            ptrs.append(e[key + "_row_ptr"][1:] + base)
            cols.append(e[key + "_col_idx"])
            base += int(e[key + "_row_ptr"][-1])
        out[key + "_row_ptr"] = np.concatenate(ptrs).astype(np.int32)
        out[key + "_col_idx"] = np.concatenate(cols).astype(np.int32)
    out["part_bitmaps"] = np.concatenate(
        [e["part_bitmaps"].reshape(-1, 64) for e in parts]).astype(np.uint64)
    for key in ("nnz", "n_full", "n_partial", "n_empty_rows"):
        out[key] = sum(int(e[key]) for e in parts)
    return out


def row_entries(mask, theta):
    """Row-wise entries of the sparse outer tiles of one [S, S] mask.

    The abstract's row-wise kernel reads a storage format of its own ("row-
    wise or block-wise kernels with unique storage formats", arXiv record
    of "Accelerating Sparse Transformer Inference on GPU", abstract); the
    pages do not print it.  Reading taken here: for outer-tile row I and
    group q of 16 query rows (rows 64I + 16q .. 64I + 16q + 15), every key
    j of a *sparse* tile of row I (a tile with some but at most ``theta``
    valid elements) that some row of the group attends to, in ascending j,
    as the pair (j, rows) with bit k of rows set iff row 64I + 16q + k
    attends to j.  Written from the dense mask (numpy over the tiles of a
    row); rows and columns past S are not valid.

    Returns {(I, q): [(j, rows), ...]} for every I < ceil(S/64), q < 4
    (empty lists included)."""
    m = np.asarray(mask, dtype=bool)
    S = m.shape[0]
    n = (S + OT - 1) // OT
    pad = np.zeros((n * OT, n * OT), dtype=bool)
    pad[:S, :S] = m
    weight = (1 << np.arange(16, dtype=np.int64))        # bit k = row k
    out = {}
    for I in range(n):
        strip = pad[OT * I:OT * I + OT].reshape(OT, n, OT)  # [row, J, col]
        cnt = strip.sum(axis=(0, 2))
        sparse = np.nonzero((cnt > 0) & (cnt < OT * OT) & (cnt <= theta))[0]
        for q in range(4):
            rows = np.einsum("kjc,k->jc", strip[16 * q:16 * q + 16, sparse]
                             .astype(np.int64), weight)     # [tile, col]
            keys = (OT * sparse[:, None] + np.arange(OT)[None, :])
            live = rows != 0
            out[(I, q)] = list(zip(keys[live].tolist(), rows[live].tolist()))
    return out
