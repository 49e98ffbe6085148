"""Per-tile dispatch of the block-wise kernel: partial tiles of at most
SMH_SPARSE_TILE_MAX valid elements are computed on its gather path (each
wavefront gathers the keys its 16 query rows see), the others on the tile
path.  Whole outputs against the fp64 oracle for masks whose rows mix
full, dense partial and sparse partial tiles, rows with only sparse tiles,
tiles at the threshold, ragged S and mask stacks; the same masks on the
tile path alone (blockwise_dense) and through SMH_AUTO."""
import numpy as np
import pytest
import torch

import sparse_masked_head_amd as smh
from oracle.attention import attention
from tests.gpu_util import TOL, need_gpu
from workloads import make_qkv, mask_family

pytestmark = pytest.mark.gpu

THETA = smh._lib.SMH_SPARSE_TILE_MAX


def band_or_random(S, w, p, seed, causal=True):
    rng = np.random.default_rng(seed)
    i = np.arange(S)[:, None]
    j = np.arange(S)[None, :]
    m = (np.abs(i - j) <= w) | (rng.random((S, S)) < p)
    return m & (j <= i) if causal else m


def threshold_mask(S=512, seed=3):
    """Tiles with exactly THETA and THETA + 1 valid elements, a full tile, a
    dense partial tile, one-element tiles, a row whose only key lies in a
    sparse tile and an empty row."""
    rng = np.random.default_rng(seed)
    m = np.zeros((S, S), bool)

    def fill(I, J, k):
        idx = rng.choice(4096, k, replace=False)
        t = np.zeros(4096, bool)
        t[idx] = True
        m[64 * I:64 * I + 64, 64 * J:64 * J + 64] = t.reshape(64, 64)
    fill(1, 0, THETA)          # sparse, at the threshold
    fill(1, 2, THETA + 1)      # dense, just above
    fill(1, 5, 3000)           # dense partial
    m[128:192, 64:128] = True  # full
    fill(2, 7, 1)
    fill(2, 3, 40)
    fill(3, 3, 4095)
    fill(4, 0, THETA)
    fill(4, 6, THETA)
    m[300] = False
    m[300, 500] = True         # one key, in a sparse tile
    m[301] = False             # empty row
    return m


ENTRY_TARGETS = [0, 1, 15, 16, 17, 31, 32, 33, 48, 49, 80, 130,
                 63, 64, 65, 0, 127, 128, 129, 1, 192, 193, 2, 3]


def entry_count_mask(S=1024, seed=21):
    """Outer-tile rows 1-6: a full diagonal tile (the tile path runs first),
    and per 16-row group a set number of row-wise entries (distinct keys
    two of its rows see, overlapping, in sparse tiles 8-15): ENTRY_TARGETS,
    so that a wavefront's entry list is empty, ends inside, at and just
    past the 16-entry chunk boundaries and the 64-entry block boundaries
    (entries are fetched four chunks at a time), and runs for many
    chunks."""
    rng = np.random.default_rng(seed)
    m = np.zeros((S, S), bool)
    targets = ENTRY_TARGETS
    cols = np.arange(8 * 64, 16 * 64)
    for idx, n_ent in enumerate(targets):
        I, q = 1 + idx // 4, idx % 4
        m[64 * I:64 * I + 64, 64 * I:64 * I + 64] = True
        if n_ent == 0:
            continue
        keys = rng.choice(cols, n_ent, replace=False)
        r0 = 64 * I + 16 * q
        a = n_ent // 4
        m[r0, keys[:max(1, n_ent - a)]] = True   # the union is all n_ent keys
        m[r0 + 7, keys[a:]] = True
    return m


CASES = [  # (name, B, H, S, d, dtype, mask builder)
    ("band+2% causal", 1, 3, 1024, 64, "f16",
     lambda: band_or_random(1024, 128, 0.02, 1)),
    ("random 1%, no full tile", 2, 2, 768, 128, "bf16",
     lambda: mask_family("random", 768, seed=2, p=0.01)),
    ("ragged window|2%", 1, 2, 1000, 64, "f16",
     lambda: band_or_random(1000, 50, 0.02, 3, causal=False)),
    ("far random causal 2%", 1, 2, 2048, 128, "bf16",
     lambda: mask_family("far_random", 2048, seed=4)),
    ("threshold tiles", 2, 2, 512, 64, "f16", threshold_mask),
    ("threshold tiles d128", 1, 2, 512, 128, "bf16", threshold_mask),
    ("0.1% random", 1, 4, 4096, 64, "f16",
     lambda: mask_family("sparse_random", 4096, seed=6)),
    ("entry counts at chunk and block boundaries", 1, 2, 1024, 64, "f16", entry_count_mask),
    ("entry counts at chunk and block boundaries d128", 2, 1, 1024, 128, "bf16", entry_count_mask),
    # the other two (d, input type) instances of the gather path
    ("band+2% causal d64 bf16", 1, 2, 768, 64, "bf16",
     lambda: band_or_random(768, 96, 0.02, 41)),
    ("far random causal 2% d128 f16", 1, 2, 1024, 128, "f16",
     lambda: mask_family("far_random", 1024, seed=42)),
]


def run(q, k, v, mask, kernel, dev, out_dtype=None):
    enc = smh.encode_mask(torch.from_numpy(np.ascontiguousarray(mask)).to(dev))
    st = smh.mask_stats_get(enc)
    o = smh.sparse_mha_fwd(q.to(dev), k.to(dev), v.to(dev), enc, kernel=kernel,
                           out_dtype=out_dtype,
                           stats=None if kernel == "auto" else st)
    torch.cuda.synchronize()
    return o, st


@pytest.mark.parametrize("kernel", ["blockwise", "blockwise_dense", "auto"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0].replace(" ", "_"))
def test_mixed_tiles_whole_output(case, kernel):
    dev = need_gpu()
    name, B, H, S, d, dt, build = case
    print(f"hybrid {kernel} {name}", flush=True)
    mask = build()
    q, k, v = make_qkv(B, H, S, d, dt, seed=S + d)
    out_dt = torch.float32 if dt == "bf16" else None
    o, st = run(q, k, v, mask, kernel, dev, out_dt)
    assert st["n_sparse"] > 0
    ref = attention(q, k, v, mask)
    err = float(np.abs(o.double().cpu().numpy() - ref).max())
    print(f"  n_sparse {st['n_sparse']} of {st['n_partial']} partial, "
          f"max abs err {err:.3e}", flush=True)
    assert torch.isfinite(o).all()
    assert err <= TOL[dt], err


def test_entry_count_mask_counts():
    """The chunk- and block-boundary mask has the intended entry counts per
    16-row group (oracle's entry builder; no GPU)."""
    from oracle.encode import row_entries
    ent = row_entries(entry_count_mask(), THETA)
    counts = [len(ent[(I, q)]) for I in range(1, 7) for q in range(4)]
    assert counts == ENTRY_TARGETS, counts


def test_threshold_rows_exact():
    """A row whose only key sits in a sparse tile returns that V row; an
    empty row returns 0."""
    dev = need_gpu()
    mask = threshold_mask()
    q, k, v = make_qkv(1, 2, 512, 64, "f16", seed=9)
    o, st = run(q, k, v, mask, "blockwise", dev, torch.float32)
    o = o.cpu()
    assert torch.allclose(o[:, :, 300], v[:, :, 500].float(), rtol=0, atol=1e-5)
    assert (o[:, :, 301] == 0).all()


def test_mask_stack_sparse_tiles():
    """One mask per head, some of them sparse, through the gather path."""
    dev = need_gpu()
    B, H, S, d = 2, 3, 640, 64
    rng = np.random.default_rng(12)
    masks = np.zeros((1, H, S, S), bool)
    masks[0, 0] = rng.random((S, S)) < 0.005
    masks[0, 1] = band_or_random(S, 100, 0.02, 13)
    masks[0, 2] = np.tril(np.ones((S, S), bool))
    q, k, v = make_qkv(B, H, S, d, "f16", seed=14)
    o, st = run(q, k, v, masks, "blockwise", dev, torch.float32)
    assert st["n_sparse"] > 0
    err = float(np.abs(o.double().cpu().numpy() - attention(q, k, v, masks)).max())
    assert err <= TOL["f16"], err
