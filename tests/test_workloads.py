"""The seeded generators produce the workloads' stated shapes and patterns."""
import numpy as np
import pytest
import torch

from workloads import CONFIGS, make_qkv, mask_family


def test_config_shapes():
    assert [(c.B, c.H, c.S, c.d, c.dtype) for c in CONFIGS.values()] == [
        (1, 2, 256, 64, "f16"), (8, 12, 512, 64, "f16"),
        (4, 32, 2048, 128, "bf16"), (2, 16, 4096, 64, "f16"),
        (1, 32, 16384, 128, "bf16"), (1, 64, 4096, 64, "f16"),
        (1, 32, 16384, 128, "bf16")]


def test_qkv_seeded_and_rounded():
    q, k, v = make_qkv(1, 2, 64, 16, "bf16", seed=3)
    q2, _, _ = make_qkv(1, 2, 64, 16, "bf16", seed=3)
    assert q.dtype == torch.bfloat16 and torch.equal(q, q2)
    g = torch.Generator().manual_seed(3)
    ref = torch.randn(1, 2, 64, 16, generator=g).to(torch.bfloat16)
    assert torch.equal(q, ref) and not torch.equal(q, k)
    assert abs(float(v.float().std()) - 1.0) < 0.1


def test_mask_patterns(config_mask):
    S = 256
    c = config_mask(1)
    assert np.array_equal(c, np.tril(np.ones((S, S), bool)))
    w = config_mask(2)
    i, j = np.nonzero(w)
    assert (np.abs(i - j) <= 64).all() and w.sum() == 61888
    lf = config_mask(3)
    assert not np.triu(lf, 1).any()
    assert lf[2047, :16].all() and not lf[2047, 16:1790].any()
    bb = config_mask(4)
    blocks = bb.reshape(64, 64, 64, 64).any(axis=(1, 3))
    assert (blocks.sum(axis=1) >= 6).all() and (blocks.sum(axis=1) <= 8).all()
    lr = config_mask(5)
    assert not np.triu(lr[:2048, :2048], 1).any()
    assert lr[16383, 16383 - 1024:].all()
    far = lr[8192:9216, 0:1024].mean()
    assert abs(far - 0.02) < 0.002


@pytest.mark.parametrize("fam", ["full", "empty", "random"])
def test_simple_families(fam):
    m = mask_family(fam, 128, seed=1, p=0.25)
    assert m.shape == (128, 128) and m.dtype == bool
    if fam == "random":
        assert abs(m.mean() - 0.25) < 0.03
