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
             n_empty_rows=st["n_empty_rows"])
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
    if "row_info" in got:
        assert np.array_equal(got["row_info"], expected_row_info(ref)), \
            "row_info"


def expected_row_info(ref):
    """Per row: list starts and counts, then its first four stored tiles'
    columns (full tiles, then partial), -1 past the row's last tile, then
    the statistics (nnz low and high words, n_full, n_partial,
    max_row_tiles) and three zeros."""
    frp, prp = ref["full_row_ptr"], ref["part_row_ptr"]
    R = len(frp) - 1
    out = np.full((R, 16), -1, np.int32)
    cnt = np.diff(frp) + np.diff(prp)
    nnz = int(ref["nnz"])
    stats = [nnz & 0xFFFFFFFF, nnz >> 32, ref["n_full"], ref["n_partial"],
             int(cnt.max()) if R else 0, 0, 0, 0]
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
