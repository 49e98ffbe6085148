"""Pins of the reference pattern masks (oracle/pattern.py).

* the generator: published SplitMix64 outputs (tests/golden/splitmix64.json),
  and the element draws of a row are the 16-bit pieces of those outputs;
* patterns without random parts equal the workload masks built
  independently in workloads/ (causal, sliding window, Longformer) and
  hand-built block maps;
* random parts: the fraction of drawn elements within 5 sigma of the
  probability, probabilities 0 and 1 exact, the causal and S limits.
"""
import json
import os

import numpy as np
import pytest

from oracle.pattern import draws16, pattern_mask, splitmix64, threshold16
from workloads import get_config, make_mask, mask_family, pattern_of

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                   "splitmix64.json")))


def test_splitmix64_published_outputs():
    for st in GOLD["streams"]:
        want = st.get("outputs") or [int(h, 16) for h in st["outputs_hex"]]
        got = splitmix64(st["seed"], np.arange(len(want)))
        assert [int(x) for x in got] == want


def test_draws_are_pieces_of_the_outputs():
    st = GOLD["streams"][1]
    S = 10                                   # e = 0..9 on row 0, 10.. on row 1
    u = draws16(S, [0, 1], st["seed"])
    for e in range(12):
        i, j = divmod(e, S)
        x = st["outputs"][e // 4]
        assert u[i, j] == (x >> (16 * (e % 4))) & 0xFFFF


@pytest.mark.parametrize("cid", [1, 2, 3])
def test_deterministic_workloads_equal_their_masks(cid):
    cfg = get_config(cid)
    assert np.array_equal(pattern_mask(cfg.S, **pattern_of(cfg)),
                          make_mask(cfg))


@pytest.mark.parametrize("S", [64, 100, 333])
def test_band_global_causal_by_hand(S):
    i = np.arange(S)[:, None]
    j = np.arange(S)[None, :]
    assert np.array_equal(pattern_mask(S, window=5), np.abs(i - j) <= 5)
    assert np.array_equal(pattern_mask(S, causal=True, window=S), j <= i)
    want = (i < 3) | (j < 7)
    assert np.array_equal(pattern_mask(S, global_rows=3, global_cols=7), want)
    assert np.array_equal(pattern_mask(S, causal=True, global_rows=3,
                                       global_cols=7), want & (j <= i))
    assert not pattern_mask(S).any()         # no part: nothing valid


def test_block_map_by_hand():
    S = 200                                  # 4 x 4 blocks, the last cut
    blocks = np.zeros((4, 4), np.uint8)
    blocks[0, 3] = 1
    blocks[2, 1] = 1
    blocks[3, 3] = 1
    m = pattern_mask(S, blocks=blocks)
    want = np.zeros((S, S), bool)
    want[0:64, 192:200] = True
    want[128:192, 64:128] = True
    want[192:200, 192:200] = True
    assert np.array_equal(m, want)


def test_threshold16_values_by_definition():
    """floor(p * 65536) with p rounded to float32 first.  Values derived by
    hand from the float32 neighbours of p (a multiplication by 2^16 is
    exact, so only the rounding of p and the floor matter):
      0.02  -> float32 0.0199999995529651641845703125,
               * 65536 = 1310.71997..., floor 1310 (rounding would give 1311)
      0.8   -> float32 0.800000011920928955078125, * 65536 = 52428.80078,
               floor 52428
      0.001 -> float32 0.001000000047497451305389404296875,
               * 65536 = 65.536003..., floor 65
      0.5   -> exact, 32768;  1.0 -> 65536;  0.0 -> 0
      2^-16 -> exact, 1;  just below 2^-16 (float32 0x377FFFFF) -> 0"""
    assert threshold16(0.02) == 1310
    assert threshold16(0.8) == 52428
    assert threshold16(0.001) == 65
    assert threshold16(0.5) == 32768
    assert threshold16(1.0) == 65536
    assert threshold16(0.0) == 0
    assert threshold16(2.0 ** -16) == 1
    below = float(np.frombuffer(np.uint32(0x377FFFFF).tobytes(), np.float32)[0])
    assert below < 2.0 ** -16
    assert threshold16(below) == 0


def test_random_fractions_and_limits():
    S = 1024
    m = pattern_mask(S, random_p=0.02, seed=9)
    p = m.mean()
    sd = np.sqrt(0.02 * 0.98 / S / S)
    assert abs(p - threshold16(0.02) / 65536) < 5 * sd
    assert pattern_mask(S, random_p=1.0).all()
    assert not pattern_mask(S, random_p=0.0, seed=3).any()
    # different seeds, different draws
    assert (pattern_mask(S, random_p=0.3, seed=1) !=
            pattern_mask(S, random_p=0.3, seed=2)).mean() > 0.3
    # sampled blocks keep about block_keep of their elements, other
    # elements follow random_p
    blocks = np.zeros((16, 16), np.uint8)
    blocks[::2, 1::2] = 2
    mb = pattern_mask(S, blocks=blocks, block_keep=0.8, random_p=0.01, seed=4)
    inb = np.kron(blocks == 2, np.ones((64, 64), bool))
    assert abs(mb[inb].mean() - 0.8) < 0.01
    assert abs(mb[~inb].mean() - 0.01) < 0.002
    # causal limit and ragged S
    mc = pattern_mask(333, causal=True, random_p=0.5, seed=1)
    assert not np.triu(mc, 1).any() and mc.shape == (333, 333)


def test_bigbird_pattern_blocks_match_workload_blocks():
    cfg = get_config(4)
    pat = pattern_of(cfg)
    m = pattern_mask(cfg.S, **pat)
    ref = make_mask(cfg)
    # same block structure: the stored blocks of both masks coincide
    nb = cfg.S // 64
    bm = m.reshape(nb, 64, nb, 64).any(axis=(1, 3))
    br = ref.reshape(nb, 64, nb, 64).any(axis=(1, 3))
    assert np.array_equal(bm, br)
    assert np.array_equal(bm, pat["blocks"] != 0)


def test_pattern_rows_are_the_mask_rows():
    """pattern_rows on any set of query rows (unordered, repeated, the last
    one) equals those rows of the whole mask, for each kind of term."""
    from oracle.pattern import pattern_rows
    S = 300
    rng = np.random.default_rng(21)
    blocks = rng.integers(0, 3, size=(5, 5)).astype(np.uint8)
    rows = np.array([299, 0, 64, 63, 150, 150, 7, 298])
    for kw in (dict(causal=True, window=20, random_p=0.05, seed=3),
               dict(global_rows=5, global_cols=9, random_p=0.01, seed=11),
               dict(blocks=blocks, block_keep=0.3, random_p=0.002, seed=8)):
        full = pattern_mask(S, **kw)
        assert np.array_equal(pattern_rows(S, rows, **kw), full[rows]), kw
