"""Pins of the reference output projection (oracle/out_proj.py): an
element-by-element sum with math.fsum on small shapes, the identity weight
(the result is the head-merged attention output), torch's own head merge
and linear layer in fp64, and additivity of bias and residual."""
import math

import numpy as np
import torch

from oracle.out_proj import merge_heads, out_proj


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_elementwise_sum():
    B, H, S, d, D = 2, 3, 5, 4, 6
    o, w, b, r = rand((B, H, S, d), 1), rand((D, H * d), 2), rand(D, 3), \
        rand((B, S, D), 4)
    got = out_proj(o, w, b, r)
    for bb in range(B):
        for s in range(S):
            for n in range(D):
                terms = [o[bb, h, s, k] * w[n, h * d + k]
                         for h in range(H) for k in range(d)]
                want = math.fsum(terms + [b[n], r[bb, s, n]])
                assert abs(got[bb, s, n] - want) < 1e-12


def test_identity_weight_merges_heads():
    B, H, S, d = 2, 4, 7, 8
    o = rand((B, H, S, d), 5)
    got = out_proj(o, np.eye(H * d))
    for h in range(H):
        assert np.array_equal(got[:, :, h * d:(h + 1) * d], o[:, h])
    assert np.array_equal(merge_heads(o), got)


def test_matches_torch_linear():
    B, H, S, d, D = 2, 3, 9, 16, 32
    o, w, b, r = rand((B, H, S, d), 6), rand((D, H * d), 7), rand(D, 8), \
        rand((B, S, D), 9)
    ot = torch.from_numpy(o)
    x = ot.transpose(1, 2).reshape(B, S, H * d)
    want = torch.nn.functional.linear(x, torch.from_numpy(w),
                                      torch.from_numpy(b)) + torch.from_numpy(r)
    np.testing.assert_allclose(out_proj(o, w, b, r), want.numpy(), rtol=0,
                               atol=1e-12)


def test_bias_and_residual_add():
    B, H, S, d, D = 1, 2, 4, 8, 16
    o, w, b, r = rand((B, H, S, d), 10), rand((D, H * d), 11), rand(D, 12), \
        rand((B, S, D), 13)
    base = out_proj(o, w)
    np.testing.assert_allclose(out_proj(o, w, b), base + b, atol=1e-13)
    np.testing.assert_allclose(out_proj(o, w, None, r), base + r, atol=1e-13)


def test_abs_products_elementwise_fsum():
    """abs_products (the scale of the fp32 accumulation error that sets the
    per-element GPU bar) is sum_k |x_k| |w_k| per output element: checked
    against an element-by-element math.fsum on signed data, so a dropped
    absolute value (which lets terms cancel) or a transposed weight fails."""
    from oracle.out_proj import abs_products
    B, H, S, d, D = 2, 3, 4, 5, 7
    o, w = rand((B, H, S, d), 21), rand((D, H * d), 22)
    assert (o < 0).any() and (w < 0).any()
    got = abs_products(o, w)
    assert got.shape == (B, S, D)
    for bb in range(B):
        for s in range(S):
            for n in range(D):
                want = math.fsum(abs(o[bb, h, s, k]) * abs(w[n, h * d + k])
                                 for h in range(H) for k in range(d))
                assert abs(got[bb, s, n] - want) <= 1e-12 * want
    # bounded below by the magnitude of the signed sum
    assert (got >= np.abs(out_proj(o, w)) - 1e-12).all()
