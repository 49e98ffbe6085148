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


def expected_row_order(ref):
    n = len(ref["full_row_ptr"]) - 1
    cnt = np.diff(ref["full_row_ptr"]) + np.diff(ref["part_row_ptr"])
    return sorted(range(n), key=lambda I: (-cnt[I], I)), int(cnt.max()
                                                              if n else 0)
