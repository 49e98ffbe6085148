"""Pins of the reference encoder (scalar C loop and pure-Python twin).

* hand-derived closed forms (tests/golden/encoding_closed_forms.json): tile
  counts, nnz and inner-tile bitmap words of the causal, window, Longformer,
  BigBird and long-sequence masks;
* hand-built single-element, full and empty masks;
* round trip: decoding the encoding (decoder written here, independently)
  gives the mask back;
* counting identity nnz = 4096 * n_full + popcount of all partial bitmaps;
* structure: row pointers monotone, column indices strictly ascending and
  disjoint between the lists, partial tiles neither empty nor full;
* the C loop and the Python twin agree on small masks;
* ragged S (not a multiple of 64): closed forms of the full and causal
  masks, and the padding identity (a ragged mask encodes like the same mask
  padded with invalid elements to 64 * ceil(S/64)).
"""
import json
import os

import numpy as np
import pytest

from oracle.encode import encode_c, encode_py

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                   "encoding_closed_forms.json")))
LOWER = int(GOLD["it_lower_incl_diag"]["value"], 16)
UPPER = int(GOLD["it_upper_incl_diag"]["value"], 16)
ONES = (1 << 64) - 1


def decode(enc, S):
    """Independent inverse of the format: rebuild the dense mask (the
    padding beyond S of a ragged mask must decode as invalid)."""
    n = -(-S // 64)
    m = np.zeros((64 * n, 64 * n), bool)
    for I in range(n):
        for t in range(enc["full_row_ptr"][I], enc["full_row_ptr"][I + 1]):
            J = int(enc["full_col_idx"][t])
            m[64 * I:64 * I + 64, 64 * J:64 * J + 64] = True
        for t in range(enc["part_row_ptr"][I], enc["part_row_ptr"][I + 1]):
            J = int(enc["part_col_idx"][t])
            words = enc["part_bitmaps"][t]
            for it in range(64):
                w = int(words[it])
                ir, ic = divmod(it, 8)
                for bit in range(64):
                    if (w >> bit) & 1:
                        r, c = divmod(bit, 8)
                        m[64 * I + 8 * ir + r, 64 * J + 8 * ic + c] = True
    assert not m[S:].any() and not m[:, S:].any()
    return m[:S, :S]


def check_structure(enc, S):
    n = -(-S // 64)
    frp, prp = enc["full_row_ptr"], enc["part_row_ptr"]
    assert frp[0] == 0 and prp[0] == 0
    assert (np.diff(frp) >= 0).all() and (np.diff(prp) >= 0).all()
    assert frp[-1] == enc["n_full"] and prp[-1] == enc["n_partial"]
    for I in range(n):
        f = enc["full_col_idx"][frp[I]:frp[I + 1]]
        p = enc["part_col_idx"][prp[I]:prp[I + 1]]
        assert (np.diff(f) > 0).all() and (np.diff(p) > 0).all()
        assert not set(f.tolist()) & set(p.tolist())
        assert ((f >= 0) & (f < n)).all() and ((p >= 0) & (p < n)).all()
    pc = popcounts(enc["part_bitmaps"])
    assert ((pc > 0) & (pc < 4096)).all()
    assert enc["nnz"] == 4096 * enc["n_full"] + int(pc.sum())


def popcounts(bm):
    b = np.ascontiguousarray(bm).view(np.uint8).reshape(len(bm), -1)
    return np.unpackbits(b, axis=1).sum(axis=1).astype(np.int64)


def same(a, b):
    for key in ("full_row_ptr", "full_col_idx", "part_row_ptr",
                "part_col_idx", "part_bitmaps"):
        assert np.array_equal(np.asarray(a[key]), np.asarray(b[key])), key
    for key in ("nnz", "n_full", "n_partial", "n_empty_rows"):
        assert a[key] == b[key], key


def test_single_element():
    for (r, c) in [(0, 0), (5, 62), (63, 63), (17, 9)]:
        m = np.zeros((64, 64), bool)
        m[r, c] = True
        for enc in (encode_c(m), encode_py(m)):
            assert enc["n_full"] == 0 and enc["n_partial"] == 1
            assert enc["nnz"] == 1 and enc["n_empty_rows"] == 63
            words = [0] * 64
            words[(r // 8) * 8 + c // 8] = 1 << (8 * (r % 8) + (c % 8))
            assert enc["part_bitmaps"][0].tolist() == words
            assert enc["part_col_idx"].tolist() == [0]
            assert enc["part_row_ptr"].tolist() == [0, 1]


def test_full_and_empty():
    enc = encode_c(np.ones((128, 128), bool))
    assert enc["n_full"] == 4 and enc["n_partial"] == 0
    assert enc["full_row_ptr"].tolist() == [0, 2, 4]
    assert enc["full_col_idx"].tolist() == [0, 1, 0, 1]
    assert enc["nnz"] == 128 * 128 and enc["n_empty_rows"] == 0
    enc = encode_c(np.zeros((192, 192), bool))
    assert enc["n_full"] == 0 and enc["n_partial"] == 0 and enc["nnz"] == 0
    assert enc["full_row_ptr"].tolist() == [0] * 4
    assert enc["n_empty_rows"] == 192


def test_ragged_full_closed_form():
    """All-valid mask of S = 100: tiles (0,0) full; (0,1), (1,0), (1,1)
    partial with 64x36, 36x64 and 36x36 valid elements.  Inner-tile column
    4 of a tile holds mask columns 96..103, of which 96..99 exist: byte
    0x0F in every row; inner-tile row 4 holds mask rows 96..103: bytes 0..3
    all ones."""
    S = 100
    for enc in (encode_c(np.ones((S, S), bool)), encode_py(np.ones((S, S), bool))):
        assert enc["full_row_ptr"].tolist() == [0, 1, 1]
        assert enc["full_col_idx"].tolist() == [0]
        assert enc["part_row_ptr"].tolist() == [0, 1, 3]
        assert enc["part_col_idx"].tolist() == [1, 0, 1]
        assert enc["nnz"] == S * S and enc["n_empty_rows"] == 0
        col4 = 0x0F0F0F0F0F0F0F0F        # columns c < 4 in all 8 rows
        row4 = 0x00000000FFFFFFFF        # rows r < 4, all 8 columns
        t01 = [ONES if ic < 4 else (col4 if ic == 4 else 0)
               for ir in range(8) for ic in range(8)]
        t10 = [ONES if ir < 4 else (row4 if ir == 4 else 0)
               for ir in range(8) for ic in range(8)]
        t11 = [(ONES if ir < 4 else row4 if ir == 4 else 0) &
               (ONES if ic < 4 else col4 if ic == 4 else 0)
               for ir in range(8) for ic in range(8)]
        assert enc["part_bitmaps"].tolist() == [t01, t10, t11]


@pytest.mark.parametrize("S", [1, 65, 100, 191])
def test_ragged_causal_closed_form(S):
    """Causal mask of ragged S: nnz = S(S+1)/2; row I of n = ceil(S/64)
    tiles stores tiles 0..I, tiles J < I full unless cut by S."""
    m = np.tril(np.ones((S, S), bool))
    n = -(-S // 64)
    for enc in (encode_c(m), encode_py(m)):
        assert enc["nnz"] == S * (S + 1) // 2 and enc["n_empty_rows"] == 0
        full = [(I, J) for I in range(n) for J in range(I)
                if 64 * (I + 1) <= S]       # below the diagonal, row not cut
        assert enc["n_full"] == len(full)
        assert enc["n_full"] + enc["n_partial"] == n * (n + 1) // 2
        check_structure(enc, S)
        assert np.array_equal(decode(enc, S), m)


@pytest.mark.parametrize("S,p,seed", [(70, 0.3, 1), (130, 0.05, 2),
                                      (200, 0.9, 3), (257, 0.5, 4)])
def test_ragged_equals_padded(S, p, seed):
    """A ragged mask encodes exactly like the same mask padded with invalid
    elements to 64 * ceil(S/64), except that the padding's rows are not
    counted as empty rows; the C loop and the Python twin agree."""
    rng = np.random.default_rng(seed)
    m = rng.random((S, S)) < p
    Sp = 64 * -(-S // 64)
    mp = np.zeros((Sp, Sp), bool)
    mp[:S, :S] = m
    a, b = encode_c(m), encode_c(mp)
    for key in ("full_row_ptr", "full_col_idx", "part_row_ptr",
                "part_col_idx", "part_bitmaps"):
        assert np.array_equal(a[key], b[key]), key
    assert a["nnz"] == b["nnz"] == int(m.sum())
    assert a["n_empty_rows"] == b["n_empty_rows"] - (Sp - S)
    assert a["n_empty_rows"] == int((~m.any(axis=1)).sum())
    same(a, encode_py(m))
    assert np.array_equal(decode(a, S), m)


def test_rejects_nonpositive():
    with pytest.raises(ValueError):
        encode_c(np.ones((0, 0), bool))
    with pytest.raises(ValueError):
        encode_py(np.ones((0, 0), bool))


@pytest.mark.parametrize("S", [64, 256, 1024])
def test_causal_closed_form(S):
    m = np.tril(np.ones((S, S), bool))
    enc = encode_c(m)
    n = S // 64
    assert enc["n_full"] == n * (n - 1) // 2 and enc["n_partial"] == n
    assert enc["nnz"] == S * (S + 1) // 2
    assert enc["part_col_idx"].tolist() == list(range(n))
    for I in range(n):
        assert enc["full_col_idx"][enc["full_row_ptr"][I]:
                                   enc["full_row_ptr"][I + 1]].tolist() \
            == list(range(I))
    for p in range(n):
        for it in range(64):
            ir, ic = divmod(it, 8)
            want = ONES if ic < ir else (0 if ic > ir else LOWER)
            assert int(enc["part_bitmaps"][p, it]) == want
    if S == 256:
        g = GOLD["causal"]["S256"]
        for key in g:
            assert enc[key] == g[key]


def test_window_closed_form(config_mask):
    m = config_mask(2)
    enc = encode_c(m)
    g = GOLD["window64_S512"]
    for key in ("nnz", "n_full", "n_partial", "n_empty_rows"):
        assert enc[key] == g[key]
    n = 8
    p = 0
    for I in range(n):
        cols = enc["part_col_idx"][enc["part_row_ptr"][I]:
                                   enc["part_row_ptr"][I + 1]].tolist()
        assert cols == [J for J in (I - 1, I + 1) if 0 <= J < n]
        assert enc["full_col_idx"][enc["full_row_ptr"][I]:
                                   enc["full_row_ptr"][I + 1]].tolist() == [I]
        for J in cols:
            w = enc["part_bitmaps"][p]
            for ir in range(8):
                if J == I + 1:
                    assert int(w[ir * 8 + ir]) == LOWER
                else:
                    assert int(w[ir * 8 + ir]) == UPPER
            if J == I + 1:
                assert int(w[1]) == 0 and int(w[8]) == ONES
            p += 1


@pytest.mark.parametrize("cid,key", [(3, "longformer_S2048"),
                                     (4, "bigbird_S4096"),
                                     (5, "long_random_S16384")])
def test_workload_closed_forms(cid, key, config_encoding):
    enc = config_encoding(cid)
    for k, v in GOLD[key].items():
        if k != "derivation":
            assert enc[k] == v, k


@pytest.mark.parametrize("cid", [1, 2, 3, 4])
def test_workload_structure_and_roundtrip(cid, config_mask, config_encoding):
    m, enc = config_mask(cid), config_encoding(cid)
    check_structure(enc, m.shape[0])
    assert enc["nnz"] == int(m.sum())
    if m.shape[0] <= 2048:
        assert np.array_equal(decode(enc, m.shape[0]), m)


def test_long_sequence_structure(config_mask, config_encoding):
    m, enc = config_mask(5), config_encoding(5)
    check_structure(enc, m.shape[0])
    assert enc["nnz"] == int(np.count_nonzero(m))


@pytest.mark.parametrize("seed,p", [(1, 0.01), (2, 0.3), (3, 0.97),
                                    (4, 0.5)])
def test_random_roundtrip_and_twin(seed, p):
    rng = np.random.default_rng(seed)
    S = 192
    m = rng.random((S, S)) < p
    m[:, 64:128] = False                        # an empty OT column
    m[0:64, 128:192] = True                     # a full OT
    m[130] = False                              # an empty row
    enc = encode_c(m)
    check_structure(enc, S)
    assert np.array_equal(decode(enc, S), m)
    same(enc, encode_py(m))
    assert enc["n_empty_rows"] == int((~m.any(axis=1)).sum())


def test_structured_twin(config_mask):
    same(encode_c(config_mask(1)), encode_py(config_mask(1)))
    from workloads import mask_family
    for fam, kw in [("window", {"w": 3}), ("random", {"p": 0.02}),
                    ("bigbird", {})]:
        m = mask_family(fam, 256, seed=9, **kw) if fam != "bigbird" else \
            mask_family("bigbird", 512, seed=9)[:256, :256]
        enc = encode_c(m)
        check_structure(enc, 256)
        same(enc, encode_py(m))


def section(enc, g, n):
    """Mask g's part of a stacked encoding, as a one-mask encoding."""
    out = {}
    for key in ("full", "part"):
        ptr = np.asarray(enc[key + "_row_ptr"][g * n:g * n + n + 1])
        out[key + "_row_ptr"] = ptr - ptr[0]
        out[key + "_col_idx"] = enc[key + "_col_idx"][ptr[0]:ptr[-1]]
        if key == "part":
            out["part_bitmaps"] = enc["part_bitmaps"][ptr[0]:ptr[-1]]
    out["n_full"] = int(out["full_row_ptr"][-1])
    out["n_partial"] = int(out["part_row_ptr"][-1])
    return out


@pytest.mark.parametrize("mb,mh,S", [(2, 3, 130), (1, 4, 64), (3, 1, 100),
                                     (1, 1, 256)])
def test_stack_sections_decode(mb, mh, S):
    """Each mask of a stack decodes back from its rows of the stacked
    encoding (mask g = gb * Hm + gh owns rows g * n_ot .. g * n_ot + n_ot-1),
    counts are totals, and the Python twin builds the same stack."""
    from oracle.encode import encode_stack
    rng = np.random.default_rng(S + mb + mh)
    dens = rng.uniform(0.001, 0.6, (mb, mh, 1, 1))
    masks = rng.random((mb, mh, S, S)) < dens
    masks[0, 0, :S // 3] = True          # some full tiles
    enc = encode_stack(masks)
    n = -(-S // 64)
    assert len(enc["full_row_ptr"]) == mb * mh * n + 1
    for gb in range(mb):
        for gh in range(mh):
            sec = section(enc, gb * mh + gh, n)
            assert np.array_equal(decode(sec, S), masks[gb, gh])
    assert enc["nnz"] == int(masks.sum())
    assert enc["n_empty_rows"] == int((~masks.any(axis=3)).sum())
    assert enc["nnz"] == 4096 * enc["n_full"] + int(
        popcounts(enc["part_bitmaps"]).sum())
    if S <= 130:
        same(encode_stack(masks, encode=encode_py), enc)
    if mb * mh == 1:
        same(enc, encode_c(masks[0, 0]))


# ---- row-wise entries of sparse tiles (oracle.encode.row_entries) ----

def test_row_entries_by_hand():
    """Hand-built tiles: one element, a whole column, a whole row, the
    threshold (theta valid elements in, theta + 1 out), full and dense
    tiles (no entries), a ragged S."""
    from oracle.encode import row_entries
    S = 256
    m = np.zeros((S, S), bool)
    m[70, 130] = True                 # tile (1, 2): one element
    m[128:192, 200] = True            # tile (2, 3): a whole column
    m[5, 64:128] = True               # tile (0, 1): a whole row
    m[192:256, 0:64] = True           # tile (3, 0): full, no entries
    m[200, 70] = True                 # tile (3, 1): one element
    e = row_entries(m, theta=64)
    assert e[(1, 0)] == [(130, 1 << 6)]
    assert all(not e[(1, q)] for q in (1, 2, 3))
    for q in range(4):                # the column: one entry per group
        assert e[(2, q)] == [(200, 0xFFFF)]
    assert e[(0, 0)] == [(j, 1 << 5) for j in range(64, 128)]
    assert e[(3, 0)] == [(70, 1 << 8)]
    # the 64-element row and column tiles have 64 <= theta elements; with
    # theta = 63 they are dense and leave no entries
    e2 = row_entries(m, theta=63)
    assert not e2[(0, 0)] and all(not e2[(2, q)] for q in range(4))
    assert e2[(1, 0)] == [(130, 1 << 6)]
    # ragged S: elements past S do not exist, so every tile but (0, 0)
    # (full) is cut, hence partial, hence sparse under theta = 4095
    r = row_entries(np.ones((100, 100), bool), theta=4095)
    for q in range(4):                # row 0: tile (0, 1), keys 64 .. 99
        assert r[(0, q)] == [(j, 0xFFFF) for j in range(64, 100)]
    assert r[(1, 0)] == [(j, 0xFFFF) for j in range(100)]
    assert r[(1, 1)] == [(j, 0xFFFF) for j in range(100)]
    assert r[(1, 2)] == [(j, 0xF) for j in range(100)]   # rows 96 .. 99
    assert not r[(1, 3)]


def test_row_entries_reconstruct_sparse_tiles():
    """Decoding the entries gives back exactly the valid pairs of the
    sparse tiles (and nothing of the other tiles); keys ascend."""
    from oracle.encode import row_entries
    rng = np.random.default_rng(5)
    S, theta = 320, 256
    m = rng.random((S, S)) < 0.03
    m |= np.abs(np.arange(S)[:, None] - np.arange(S)[None, :]) <= 20
    e = row_entries(m, theta)
    back = np.zeros_like(m)
    for (I, q), lst in e.items():
        keys = [j for j, _ in lst]
        assert keys == sorted(set(keys))
        for j, rows in lst:
            assert rows
            for k in range(16):
                if rows >> k & 1:
                    back[64 * I + 16 * q + k, j] = True
    n = S // 64
    sparse = np.zeros_like(m)
    for I in range(n):
        for J in range(n):
            t = m[64 * I:64 * I + 64, 64 * J:64 * J + 64]
            if 0 < t.sum() <= theta:
                sparse[64 * I:64 * I + 64, 64 * J:64 * J + 64] = t
    assert sparse.any() and np.array_equal(back, sparse)


def test_row_entries_brute_force():
    """Against an element-by-element loop over tiles, groups, columns and
    rows, on a small random mask with sparse, dense and full tiles."""
    from oracle.encode import row_entries
    rng = np.random.default_rng(8)
    S, theta = 200, 256
    m = rng.random((S, S)) < rng.choice([0.005, 0.03, 0.5], (S, 1))
    m[0:64, 0:64] = True
    e = row_entries(m, theta)
    n = -(-S // 64)
    for I in range(n):
        for q in range(4):
            want = []
            for J in range(n):
                cnt = sum(1 for r in range(64) for c in range(64)
                          if 64 * I + r < S and 64 * J + c < S and
                          m[64 * I + r, 64 * J + c])
                if cnt == 0 or cnt == 4096 or cnt > theta:
                    continue
                for c in range(64):
                    j = 64 * J + c
                    rows = 0
                    for k in range(16):
                        i = 64 * I + 16 * q + k
                        if i < S and j < S and m[i, j]:
                            rows |= 1 << k
                    if rows:
                        want.append((j, rows))
            assert e[(I, q)] == want, (I, q)
