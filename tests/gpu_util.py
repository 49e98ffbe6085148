"""Helpers for the GPU tests (device checks and oracle comparisons)."""
import numpy as np
import pytest
import torch

TOL = {"f16": 2e-3, "bf16": 1e-2}   # max abs error vs the fp64 oracle
TDT = {"f16": torch.float16, "bf16": torch.bfloat16}


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    name = torch.cuda.get_device_properties(0).gcnArchName
    assert name.startswith("gfx950"), f"built for gfx950, found {name}"
    return torch.device("cuda:0")


def enc_to_host(enc, st):
    a = {k: v.cpu().numpy() for k, v in enc.arrays(st).items()}
    a["part_bitmaps"] = a["part_bitmaps"].view(np.uint64)
    a.update(nnz=st["nnz"], n_full=st["n_full"], n_partial=st["n_partial"],
             n_empty_rows=st["n_empty_rows"], n_sparse=st["n_sparse"],
             sparse_nnz=st["sparse_nnz"], row_entries=st["row_entries"])
    return a


def assert_same_encoding(got, ref):
    for key in ("full_row_ptr", "full_col_idx", "part_row_ptr",
                "part_col_idx"):
        assert np.array_equal(got[key], ref[key]), key
    assert got["part_bitmaps"].shape == ref["part_bitmaps"].shape
    bad = np.nonzero((got["part_bitmaps"] != ref["part_bitmaps"]).any(1))[0]
    assert bad.size == 0, f"bitmaps of partial tiles {bad[:8]} differ"
    for key in ("nnz", "n_full", "n_partial", "n_empty_rows"):
        assert got[key] == ref[key], key
    if "part_pop" in got:
        assert np.array_equal(got["part_pop"], expected_part_pop(ref)), \
            "part_pop"
        pop = expected_part_pop(ref)
        sp = pop <= SPARSE_TILE_MAX
        assert got["n_sparse"] == int(sp.sum()), "n_sparse"
        assert got["sparse_nnz"] == int(pop[sp].sum()), "sparse_nnz"
    if "row_info" in got:
        # the row-entry total in every row summary is the encoding's own
        # statistic; assert_same_row_entries pins it to the oracle
        assert np.array_equal(got["row_info"],
                              expected_row_info(dict(ref, row_entries=got["row_entries"]))), \
            "row_info"


SPARSE_TILE_MAX = 112   # smh.h SMH_SPARSE_TILE_MAX: a partial tile of at
                        # most this many valid elements is sparse


def expected_part_pop(ref):
    """Valid elements of each partial tile: the population count of its 64
    inner-tile words."""
    bm = np.ascontiguousarray(ref["part_bitmaps"]).view(np.uint64).reshape(-1, 64)
    if len(bm) == 0:
        return np.zeros(0, np.int32)
    bits = np.unpackbits(bm.view(np.uint8).reshape(len(bm), 512), axis=1)
    return bits.sum(axis=1).astype(np.int32)


def expected_row_info(ref):
    """Per row: list starts and counts, then its first four stored tiles'
    columns (full tiles, then partial), -1 past the row's last tile, then
    the statistics (nnz low and high words, n_full, n_partial,
    max_row_tiles, n_sparse, row_entries low and high words; the reference
    must carry row_entries, the oracle's count of row-wise entries)."""
    frp, prp = ref["full_row_ptr"], ref["part_row_ptr"]
    R = len(frp) - 1
    out = np.full((R, 16), -1, np.int32)
    cnt = np.diff(frp) + np.diff(prp)
    nnz = int(ref["nnz"])
    pop = expected_part_pop(ref)
    sp = pop <= SPARSE_TILE_MAX
    ents = int(ref["row_entries"])
    stats = [nnz & 0xFFFFFFFF, nnz >> 32, ref["n_full"], ref["n_partial"],
             int(cnt.max()) if R else 0, int(sp.sum()), ents & 0xFFFFFFFF,
             ents >> 32]
    for r in range(R):
        cols = list(ref["full_col_idx"][frp[r]:frp[r + 1]]) + \
            list(ref["part_col_idx"][prp[r]:prp[r + 1]])
        out[r, :4] = [frp[r], frp[r + 1] - frp[r], prp[r], prp[r + 1] - prp[r]]
        out[r, 4:8] = (cols[:4] + [-1] * 4)[:4]
        out[r, 8:16] = np.array(stats, np.int64).astype(np.uint32).view(np.int32)
    return out


def expected_row_order(ref):
    n = len(ref["full_row_ptr"]) - 1
    cnt = np.diff(ref["full_row_ptr"]) + np.diff(ref["part_row_ptr"])
    return sorted(range(n), key=lambda I: (-cnt[I], I)), int(cnt.max()
                                                              if n else 0)


def assert_same_row_entries(got, masks, S):
    """The encoding's row-wise entries (row_ent, row_ent_cnt of enc_to_host)
    against oracle.encode.row_entries of each mask of [S, S] or a stack
    [Bm, Hm, S, S]: bit-exact lists per (encoding row, group); all counts
    0 when S > 65536 (no row-wise format)."""
    from oracle.encode import row_entries
    m = np.asarray(masks)
    mlist = [m] if m.ndim == 2 else [m[a, b] for a in range(m.shape[0])
                                     for b in range(m.shape[1])]
    n = -(-S // 64)
    cnt = got["row_ent_cnt"]
    if S > 65536:
        assert (cnt == 0).all() and got["row_entries"] == 0
        return
    total = 0
    prp = got["part_row_ptr"]
    ent = got["row_ent"].view(np.uint32)
    for g, mg in enumerate(mlist):
        want = row_entries(mg, SPARSE_TILE_MAX)
        for I in range(n):
            r = g * n + I
            np_r = int(prp[r + 1] - prp[r])
            for q in range(4):
                w = want[(I, q)]
                total += len(w)
                assert int(cnt[r, q]) == len(w), (g, I, q)
                if not w:
                    continue
                base = 256 * int(prp[r]) + 64 * q * np_r
                e = ent[base:base + len(w)]
                wk = np.array([j for j, _ in w], np.uint32)
                wr = np.array([x for _, x in w], np.uint32)
                assert np.array_equal(e & 0xFFFF, wk), (g, I, q)
                assert np.array_equal(e >> 16, wr), (g, I, q)
    assert got["row_entries"] == total, "row_entries"


def counted_row_entries(arr):
    """The row-wise entries an encoding holds (arrays() of a MaskEncoding,
    device or host): the counted entries of every (row, group) region,
    concatenated in row and group order (the regions' other slots are
    never written)."""
    prp = np.asarray(arr["part_row_ptr"].cpu() if hasattr(arr["part_row_ptr"], "cpu")
                     else arr["part_row_ptr"])
    cnt = np.asarray(arr["row_ent_cnt"].cpu() if hasattr(arr["row_ent_cnt"], "cpu")
                     else arr["row_ent_cnt"])
    ent = np.asarray(arr["row_ent"].cpu() if hasattr(arr["row_ent"], "cpu")
                     else arr["row_ent"])
    out = []
    for r in range(len(prp) - 1):
        np_r = int(prp[r + 1] - prp[r])
        for q in range(4):
            base = 256 * int(prp[r]) + 64 * q * np_r
            out.append(ent[base:base + int(cnt[r, q])])
    return np.concatenate(out) if out else np.zeros(0, np.int32)
