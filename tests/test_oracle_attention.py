"""Pins of the fp64 attention oracle against things other than itself.

* library special cases: torch's scaled_dot_product_attention in fp64 on
  the CPU, with no mask, is_causal, and boolean attn_mask (every row with a
  valid key);
* exhaustive tiny masks: every one of the 2^(S*S) masks at S = 2 and 3;
* closed forms: one valid key returns that V row exactly; Q = 0 returns the
  mean of the valid V rows; a row with no valid key returns 0;
* invariants: key and query permutations, a shared shift of every key,
  affine maps of V;
* in-workload special rows: row 0 of the causal and Longformer masks has
  exactly one key (key 0).
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle.attention import attention, attention_rows


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _sdpa(q, k, v, mask=None, causal=False):
    t = [torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, v)]
    am = None if mask is None else torch.from_numpy(np.asarray(mask, bool))
    return F.scaled_dot_product_attention(*t, attn_mask=am,
                                          is_causal=causal).numpy()


@pytest.mark.parametrize("S,d", [(5, 4), (64, 16), (130, 64), (257, 128)])
def test_full_mask_matches_sdpa(S, d):
    q, k, v = (_rand((2, 3, S, d), s) for s in (1, 2, 3))
    got = attention(q, k, v, np.ones((S, S), bool))
    np.testing.assert_allclose(got, _sdpa(q, k, v), rtol=0, atol=1e-12)


@pytest.mark.parametrize("S,d", [(7, 8), (200, 64), (2100, 32)])
def test_causal_matches_sdpa(S, d):
    q, k, v = (_rand((1, 2, S, d), s) for s in (4, 5, 6))
    mask = np.tril(np.ones((S, S), bool))       # j <= i
    got = attention(q, k, v, mask)
    np.testing.assert_allclose(got, _sdpa(q, k, v, causal=True),
                               rtol=0, atol=1e-12)


@pytest.mark.parametrize("p", [0.05, 0.3, 0.9])
def test_random_mask_matches_sdpa(p):
    S, d = 96, 32
    rng = np.random.default_rng(7)
    mask = rng.random((S, S)) < p
    mask[np.arange(S), rng.integers(0, S, S)] = True   # no empty row
    q, k, v = (_rand((2, 2, S, d), s) for s in (8, 9, 10))
    got = attention(q, k, v, mask)
    np.testing.assert_allclose(got, _sdpa(q, k, v, mask=mask),
                               rtol=0, atol=1e-12)


def test_nonsquare_scale_and_large_scores():
    # large scores must not overflow (subtracting the row max)
    S, d = 40, 16
    q, k, v = (_rand((1, 1, S, d), s, 30.0) for s in (11, 12, 13))
    mask = np.random.default_rng(14).random((S, S)) < 0.5
    mask[:, 0] = True
    got = attention(q, k, v, mask)
    assert np.isfinite(got).all()
    np.testing.assert_allclose(got, _sdpa(q, k, v, mask=mask),
                               rtol=0, atol=1e-10)


@pytest.mark.parametrize("S", [2, 3])
def test_every_tiny_mask(S):
    """All 2^(S*S) masks: rows with a valid key follow sdpa, empty rows
    return exactly 0."""
    d = 3
    q, k, v = (_rand((1, 1, S, d), s) for s in (20, 21, 22))
    for code in range(1 << (S * S)):
        bits = [(code >> t) & 1 for t in range(S * S)]
        mask = np.array(bits, bool).reshape(S, S)
        got = attention(q, k, v, mask)
        for i in range(S):
            if not mask[i].any():
                assert (got[0, 0, i] == 0).all()
            else:
                want = _sdpa(q[:, :, i:i + 1], k[:, :, mask[i]],
                             v[:, :, mask[i]])[0, 0, 0]
                np.testing.assert_allclose(got[0, 0, i], want, rtol=0,
                                           atol=1e-13)


def test_single_valid_key_returns_that_row_exactly():
    S, d = 50, 16
    q, k, v = (_rand((2, 2, S, d), s, 5.0) for s in (30, 31, 32))
    j = np.random.default_rng(33).integers(0, S, S)
    mask = np.zeros((S, S), bool)
    mask[np.arange(S), j] = True
    got = attention(q, k, v, mask)
    assert np.array_equal(got, v[:, :, j, :])


def test_zero_query_returns_mean_of_valid_rows():
    S, d = 33, 8
    k, v = (_rand((1, 2, S, d), s) for s in (34, 35))
    q = np.zeros((1, 2, S, d))
    mask = np.random.default_rng(36).random((S, S)) < 0.4
    mask[:, 3] = True
    got = attention(q, k, v, mask)
    for i in range(S):
        want = v[:, :, mask[i], :].mean(axis=2)
        np.testing.assert_allclose(got[:, :, i], want, rtol=0, atol=1e-14)


def test_empty_rows_return_zero():
    S, d = 20, 8
    q, k, v = (_rand((1, 1, S, d), s) for s in (37, 38, 39))
    mask = np.random.default_rng(40).random((S, S)) < 0.5
    mask[[0, 7, 19]] = False
    got = attention(q, k, v, mask)
    assert (got[0, 0, [0, 7, 19]] == 0).all()
    assert np.isfinite(got).all()
    assert not (got[0, 0, 1] == 0).all()


def test_invariants():
    S, d = 48, 16
    q, k, v = (_rand((1, 1, S, d), s) for s in (41, 42, 43))
    rng = np.random.default_rng(44)
    mask = rng.random((S, S)) < 0.3
    mask[np.arange(S), np.arange(S)] = True
    base = attention(q, k, v, mask)
    # keys permuted together with the mask columns: no change
    pk = rng.permutation(S)
    got = attention(q, k[:, :, pk], v[:, :, pk], mask[:, pk])
    np.testing.assert_allclose(got, base, rtol=0, atol=1e-13)
    # queries permuted together with the mask rows: rows permuted
    pq = rng.permutation(S)
    got = attention(q[:, :, pq], k, v, mask[pq])
    np.testing.assert_allclose(got, base[:, :, pq], rtol=0, atol=1e-13)
    # the same vector added to every key shifts a row's scores uniformly
    u = rng.standard_normal(d)
    got = attention(q, k + u, v, mask)
    np.testing.assert_allclose(got, base, rtol=0, atol=1e-12)
    # O is an affine (weighted-mean) function of V
    w = rng.standard_normal(d)
    got = attention(q, k, 2.5 * v + w, mask)
    np.testing.assert_allclose(got, 2.5 * base + w, rtol=0, atol=1e-12)


def test_scale_argument():
    S, d = 16, 8
    q, k, v = (_rand((1, 1, S, d), s) for s in (45, 46, 47))
    mask = np.ones((S, S), bool)
    got = attention(q, k, v, mask, scale=0.3)
    want = attention(q * (0.3 * math.sqrt(d)), k, v, mask)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-13)


def test_rows_entry_matches_full():
    S, d = 300, 32
    q, k, v = (_rand((2, 2, S, d), s) for s in (48, 49, 50))
    mask = np.random.default_rng(51).random((S, S)) < 0.2
    mask[5] = False
    full = attention(q, k, v, mask, row_block=64)
    rows = np.array([0, 5, 63, 64, 299])
    got = attention_rows(q, k, v, mask, 1, 0, rows)
    np.testing.assert_allclose(got, full[1, 0, rows], rtol=0, atol=1e-13)
    qt, kt, vt = (torch.from_numpy(x).to(torch.float16) for x in (q, k, v))
    full16 = attention(qt, kt, vt, mask)
    got16 = attention_rows(qt, kt, vt, mask, 0, 1, rows)
    np.testing.assert_allclose(got16, full16[0, 1, rows], rtol=0, atol=1e-13)
    # the same rows given by their mask rows alone (no [S, S] mask)
    got_r = attention_rows(q, k, v, None, 1, 0, rows, mask_rows=mask[rows])
    np.testing.assert_allclose(got_r, full[1, 0, rows], rtol=0, atol=1e-13)


@pytest.mark.parametrize("cid", [1, 3])
def test_workload_row0_has_single_key(cid, config_mask):
    from workloads import get_config, make_qkv
    cfg = get_config(cid)
    mask = config_mask(cid)
    assert mask[0].sum() == 1 and mask[0, 0]
    q, k, v = make_qkv(1, 1, cfg.S, cfg.d, cfg.dtype, seed=cid)
    got = attention_rows(q, k, v, mask, 0, 0, [0])
    assert np.array_equal(got[0], v[0, 0, 0].double().numpy())


@pytest.mark.parametrize("mb,mh,S", [(2, 1, 48), (1, 3, 70), (2, 3, 33),
                                     (1, 1, 40)])
def test_mask_stack_matches_sdpa(mb, mh, S):
    """A mask per sequence and/or head: the library's broadcasting of a
    boolean attn_mask [Bm, Hm, S, S] over [B, H] is the same rule."""
    B, H, d = 2, 3, 16
    rng = np.random.default_rng(mb * 10 + mh + S)
    masks = rng.random((mb, mh, S, S)) < 0.3
    masks[..., np.arange(S), np.arange(S)] = True     # no empty row
    q, k, v = (_rand((B, H, S, d), s) for s in (21, 22, 23))
    got = attention(q, k, v, masks)
    np.testing.assert_allclose(got, _sdpa(q, k, v, mask=masks),
                               rtol=0, atol=1e-12)
    # rows of the per-row entry point see the same masks
    rows = [0, S // 2, S - 1]
    for b in range(B):
        for h in range(H):
            np.testing.assert_allclose(
                attention_rows(q, k, v, masks, b, h, rows), got[b, h, rows],
                rtol=0, atol=1e-13)


def test_mask_stack_rejects_wrong_shape():
    q = _rand((2, 3, 8, 4), 1)
    with pytest.raises(AssertionError):
        attention(q, q, q, np.ones((3, 1, 8, 8), bool))
    with pytest.raises(AssertionError):
        attention(q, q, q, np.ones((1, 2, 8, 8), bool))
