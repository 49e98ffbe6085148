"""GPU pattern encoder against the scalar C reference encoder run on the
dense mask the oracle builds from the same pattern: bit-exact equality of
every array and statistic; attention through a pattern encoding."""
import numpy as np
import pytest
import torch

import sparse_masked_head_amd as smh
from oracle.attention import attention
from oracle.encode import encode_c
from oracle.pattern import pattern_mask
from tests.gpu_util import (TOL, assert_same_encoding, assert_same_row_entries,
                            enc_to_host, expected_row_order, need_gpu)
from workloads import get_config, make_qkv, pattern_of

pytestmark = pytest.mark.gpu


def gpu_pattern(S, dev, pat):
    kw = dict(pat)
    if kw.get("blocks") is not None:
        kw["blocks"] = torch.from_numpy(np.ascontiguousarray(kw["blocks"])).to(dev)
    enc = smh.encode_pattern(S, device=dev, **kw)
    st = smh.mask_stats_get(enc)
    return enc, st, enc_to_host(enc, st)


def check(S, dev, pat):
    enc, st, got = gpu_pattern(S, dev, pat)
    dense = pattern_mask(S, **pat)
    ref = encode_c(dense)
    assert_same_encoding(got, ref)
    assert_same_row_entries(got, dense, S)
    order, mrt = expected_row_order(ref)
    assert got["row_order"].tolist() == order and st["max_row_tiles"] == mrt
    return enc, st


@pytest.mark.parametrize("cid", [1, 2, 3, 4])
def test_workload_patterns_bit_exact(cid):
    dev = need_gpu()
    cfg = get_config(cid)
    print(f"pattern workload {cid}", flush=True)
    check(cfg.S, dev, pattern_of(cfg))


@pytest.mark.parametrize("S", [4096, 16384])
def test_long_random_pattern_bit_exact(S):
    """The long-sequence family (causal, band 1024, 2% elsewhere) at
    S = 4096 and at the 16k workload's own length (the oracle builds the
    268 MB dense mask in about 15 s)."""
    dev = need_gpu()
    print(f"long_random pattern S={S}", flush=True)
    check(S, dev, dict(causal=True, window=1024, random_p=0.02, seed=5))


@pytest.mark.parametrize("S,pat", [
    (1, dict(window=0)),
    (100, dict(causal=True, window=100)),
    (130, dict(window=7, global_rows=3, global_cols=70)),
    (333, dict(causal=True, random_p=0.05, seed=11)),
    (1000, dict(window=40, random_p=0.003, seed=2)),
    (640, dict(random_p=1.0)),
    (640, dict(random_p=0.5, seed=(1 << 64) - 3)),
    (256, dict(window=-1)),                      # nothing valid
    (2050, dict(causal=True, global_cols=130, random_p=0.001, seed=4)),
])
def test_patterns_bit_exact(S, pat):
    dev = need_gpu()
    print(f"pattern S={S} {pat}", flush=True)
    check(S, dev, pat)


def test_block_maps_bit_exact():
    dev = need_gpu()
    rng = np.random.default_rng(1)
    for S in (512, 777):
        n = -(-S // 64)
        blocks = rng.choice(np.array([0, 0, 0, 1, 2, 7], np.uint8), (n, n))
        check(S, dev, dict(blocks=blocks, block_keep=0.3, random_p=0.01,
                           seed=S))
        check(S, dev, dict(blocks=blocks, causal=True, window=20))


def test_rejects_bad_patterns():
    dev = need_gpu()
    for kw in (dict(window=-2), dict(global_rows=-1), dict(random_p=1.5),
               dict(block_keep=-0.1), dict(random_p=float("nan"))):
        with pytest.raises(smh.SmhError) as e:
            smh.encode_pattern(256, device=dev, **kw)
        assert e.value.status == 1
    with pytest.raises(ValueError):
        smh.encode_pattern(256, device=dev,
                           blocks=torch.zeros((3, 3), dtype=torch.uint8,
                                              device=dev))


@pytest.mark.parametrize("kernel", ["auto", "blockwise", "rowwise"])
def test_attention_through_pattern(kernel):
    """A pattern encoding is an encoding like any other: the forward pass
    gives bitwise what it gives on the dense mask's encoding, and matches
    the oracle."""
    dev = need_gpu()
    S, d = 384, 64
    pat = dict(causal=True, window=60, global_cols=5, random_p=0.02, seed=7)
    mask = pattern_mask(S, **pat)
    q, k, v = make_qkv(2, 2, S, d, "f16", seed=7)
    qd, kd, vd = (x.to(dev) for x in (q, k, v))
    ep = smh.encode_pattern(S, device=dev, **pat)
    em = smh.encode_mask(torch.from_numpy(mask).to(dev))
    st = smh.mask_stats_get(em)
    a = smh.sparse_mha_fwd(qd, kd, vd, ep, kernel=kernel,
                           stats=None if kernel == "auto" else st)
    b = smh.sparse_mha_fwd(qd, kd, vd, em, kernel=kernel,
                           stats=None if kernel == "auto" else st)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    err = float(np.abs(a.double().cpu().numpy() - attention(q, k, v, mask)).max())
    assert err <= TOL["f16"], err


@pytest.mark.parametrize("kernel", ["auto", "blockwise", "blockwise_dense", "rowwise"])
def test_longest_masks_without_row_entries(kernel):
    """S = 66000 (past 65536 keys: no row-wise entries are built, and 1032
    outer tiles per side: the block-wise kernel keeps every partial tile on
    its tile path), encoded from a pattern (its dense mask would take 4.4
    GB): the statistics say so, and sampled output rows, among them rows in
    the last outer tile and the last row, match the oracle computed from
    those rows' mask rows alone."""
    from oracle.attention import attention_rows
    from oracle.pattern import pattern_rows
    dev = need_gpu()
    S, B, H, d = 66000, 1, 2, 64
    pat = dict(causal=True, window=100, random_p=0.001, seed=5)
    print(f"pattern S={S} {pat} kernel {kernel}", flush=True)
    enc = smh.encode_pattern(S, device=dev, **pat)
    st = smh.mask_stats_get(enc)
    assert st["row_entries"] == 0 and st["n_sparse"] > 0
    q, k, v = make_qkv(B, H, S, d, "f16", seed=66)
    o = smh.sparse_mha_fwd(q.to(dev), k.to(dev), v.to(dev), enc, kernel=kernel,
                           stats=None if kernel == "auto" else st)
    torch.cuda.synchronize()
    rng = np.random.default_rng(67)
    rows = np.unique(np.concatenate([[0, 1, 63, 64, 101, 4096, 33000, 65535, 65536,
                                      65599, 65600, 65983, 65984, S - 1],
                                     rng.integers(0, S, 18)]))
    mrows = pattern_rows(S, rows, **pat)
    for h in range(H):
        ref = attention_rows(q, k, v, None, 0, h, rows, mask_rows=mrows)
        got = o[0, h].index_select(0, torch.as_tensor(rows, device=dev)).double().cpu().numpy()
        err = float(np.abs(got - ref).max())
        assert err <= TOL["f16"], (h, err)
