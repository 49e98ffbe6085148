"""GPU encoder against the scalar C reference encoder: bit-exact equality of
every array and statistic (integer work)."""
import numpy as np
import pytest
import torch

import sparse_masked_head_amd as smh
from oracle.encode import encode_c
from tests.gpu_util import (assert_same_encoding, assert_same_row_entries,
                            enc_to_host, expected_row_order, need_gpu)
from workloads import mask_family

pytestmark = pytest.mark.gpu


def gpu_encode(mask_np, dev):
    m = torch.from_numpy(np.ascontiguousarray(mask_np)).to(dev)
    enc = smh.encode_mask(m)
    st = smh.mask_stats_get(enc)
    return enc, st, enc_to_host(enc, st)


def check(mask_np, dev):
    enc, st, got = gpu_encode(mask_np, dev)
    ref = encode_c(mask_np)
    assert_same_encoding(got, ref)
    assert_same_row_entries(got, mask_np, mask_np.shape[-1])
    order, mrt = expected_row_order(ref)
    assert got["row_order"].tolist() == order
    assert st["max_row_tiles"] == mrt
    return enc, st, got


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_workload_masks_bit_exact(cid, config_mask, config_encoding):
    dev = need_gpu()
    print(f"encoder workload {cid}", flush=True)
    m = config_mask(cid)
    enc, st, got = gpu_encode(m, dev)
    ref = config_encoding(cid)
    assert_same_encoding(got, ref)
    assert_same_row_entries(got, m, m.shape[0])
    order, mrt = expected_row_order(ref)
    assert got["row_order"].tolist() == order and st["max_row_tiles"] == mrt


@pytest.mark.parametrize("fam,S,kw", [
    ("empty", 256, {}), ("full", 256, {}), ("causal", 64, {}),
    ("window", 320, {"w": 5}), ("random", 512, {"p": 0.001}),
    ("random", 512, {"p": 0.5}), ("random", 448, {"p": 0.999}),
    ("bigbird", 1024, {})])
def test_corner_and_random_masks(fam, S, kw):
    dev = need_gpu()
    check(mask_family(fam, S, seed=S, **kw), dev)


def band_and_points(S, w, npts, seed):
    """Band |i - j| <= w, a full block of rows and scattered single points:
    full, partial and empty tiles in every outer-tile row, cheap at any S."""
    m = np.zeros((S, S), bool)
    for d in range(-w, w + 1):
        i = np.arange(max(0, -d), min(S, S - d))
        m[i, i + d] = True
    m[64:192, : S // 2] = True
    rng = np.random.default_rng(seed)
    m[rng.integers(0, S, npts), rng.integers(0, S, npts)] = True
    return m


@pytest.mark.parametrize("S", [576, 6400, 16448, 19200, 25600])
def test_segment_cuts(S):
    """Sizes whose rows are cut into several segments of one or more
    windows, the last segment and its last window ragged (n = 9, 100, 257,
    300, 400 outer tiles per side; n = 400 makes 2800 segments, past the
    fused placement's limit, so the scan runs as a launch of its own)."""
    dev = need_gpu()
    print(f"encoder segment cuts S={S}", flush=True)
    check(band_and_points(S, 70, 4 * S, seed=S), dev)


def test_single_elements_and_diagonal():
    dev = need_gpu()
    S = 192
    m = np.zeros((S, S), bool)
    for (i, j) in [(0, 0), (63, 64), (100, 191), (191, 0), (130, 77)]:
        m[i, j] = True
    check(m, dev)
    check(np.eye(S, dtype=bool), dev)


def test_nonzero_bytes_count_as_valid():
    dev = need_gpu()
    S = 128
    rng = np.random.default_rng(5)
    vals = rng.choice(np.array([0, 1, 2, 127, 128, 255], np.uint8), (S, S))
    enc_u8, _, got = gpu_encode(vals, dev)
    assert_same_encoding(got, encode_c(vals != 0))


def test_empty_sequence():
    dev = need_gpu()
    enc = smh.encode_mask(torch.zeros((0, 0), dtype=torch.bool, device=dev))
    st = smh.mask_stats_get(enc)
    assert st["nnz"] == 0 and st["n_full"] == 0 and st["n_partial"] == 0


@pytest.mark.parametrize("S,p", [(1, 1.0), (8, 0.5), (65, 0.3), (80, 0.9),
                                 (100, 1.0), (130, 0.05), (200, 0.5),
                                 (257, 0.02), (1000, 0.2), (1040, 0.6),
                                 (3001, 0.01)])
def test_ragged_sequence(S, p):
    """S not a multiple of 64: elements past S are not valid, the cut tiles
    are never full, rows past S are not counted.  S % 16 == 0 (80, 1040)
    reads whole 16-byte pieces, other S read bytes."""
    dev = need_gpu()
    print(f"encoder ragged S={S}", flush=True)
    m = mask_family("random", S, seed=S, p=p)
    m[: S // 4, : S // 2] = True
    check(m, dev)
    check(np.tril(np.ones((S, S), bool)), dev)


def stack_check(masks, dev):
    from oracle.encode import encode_stack
    mt = torch.from_numpy(np.ascontiguousarray(masks)).to(dev)
    enc = smh.encode_mask(mt)
    st = smh.mask_stats_get(enc)
    assert (st["mask_b"], st["mask_h"]) == masks.shape[:2]
    got = enc_to_host(enc, st)
    ref = encode_stack(masks)
    assert_same_encoding(got, ref)
    assert_same_row_entries(got, masks, masks.shape[-1])
    order, mrt = expected_row_order(ref)
    assert got["row_order"].tolist() == order
    assert st["max_row_tiles"] == mrt


@pytest.mark.parametrize("mb,mh,S", [(2, 3, 130), (1, 12, 512), (8, 1, 256),
                                     (4, 4, 100), (1, 72, 1024),
                                     (32, 32, 512)])
def test_mask_stack(mb, mh, S):
    """One encoding of a stack of masks, bit-exact with the masks'
    encodings one after another.  72 x 16 rows is past the fused scan's
    1024 rows (the scan runs as a launch of its own); 32 x 32 x 8 rows is
    the largest stack accepted (8192 rows)."""
    dev = need_gpu()
    print(f"encoder stack {mb}x{mh} S={S}", flush=True)
    rng = np.random.default_rng(mb * 1000 + mh * 10 + S)
    dens = rng.uniform(0.0005, 0.7, (mb, mh, 1, 1))
    masks = rng.random((mb, mh, S, S)) < dens
    masks[0, -1] = np.tril(np.ones((S, S), bool))
    stack_check(masks, dev)


def test_stack_limits():
    dev = need_gpu()
    assert smh.encode_workspace_bytes(512, 32, 32) > 0
    assert smh.encode_workspace_bytes(512, 32, 33) == 0     # 8448 rows
    assert smh.encode_workspace_bytes(64, 0, 1) == 0
    with pytest.raises(smh.SmhError) as e:
        smh.encode_mask(torch.ones((1, 8193, 64, 64), dtype=torch.bool,
                                   device=dev))
    assert e.value.status == 1


def test_deterministic_and_reusable_workspace():
    dev = need_gpu()
    m = mask_family("random", 640, seed=3, p=0.2)
    _, _, a = gpu_encode(m, dev)
    # a dirty, reused workspace gives the same result
    ws = torch.full((smh.encode_workspace_bytes(640),), 0xAB,
                    dtype=torch.uint8, device=dev)
    enc = smh.encode_mask(torch.from_numpy(m).to(dev), workspace=ws)
    b = enc_to_host(enc, smh.mask_stats_get(enc))
    assert_same_encoding(b, a)
    enc = smh.encode_mask(torch.from_numpy(~m).to(dev), workspace=ws)
    c = enc_to_host(enc, smh.mask_stats_get(enc))
    assert_same_encoding(c, encode_c(~m))


def test_workspace_reused_across_sizes():
    """One workspace serves encodes of different S in turn."""
    dev = need_gpu()
    ws = torch.full((smh.encode_workspace_bytes(1024),), 0xAB,
                    dtype=torch.uint8, device=dev)
    for S, p in [(1024, 0.2), (256, 0.5), (64, 0.9), (1024, 0.01), (512, 0.3)]:
        m = mask_family("random", S, seed=S, p=p)
        enc = smh.encode_mask(torch.from_numpy(m).to(dev), workspace=ws)
        got = enc_to_host(enc, smh.mask_stats_get(enc))
        assert_same_encoding(got, encode_c(m))
