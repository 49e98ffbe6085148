"""Seeded generators for masks and Q/K/V.

Recipe (all draws are seeded by the workload id, so every consumer sees the
same bits):

* Q, K, V: ``torch.Generator().manual_seed(seed)``; Q, then K, then V are
  drawn as float32 ``randn(B, H, S, d)`` and rounded to fp16 or bf16
  (round-to-nearest-even).  Nothing else is applied.
* Masks: ``numpy.random.default_rng(seed)`` (PCG64).  True means the
  (query i, key j) pair takes part in attention.  One [S, S] mask serves
  every (batch, head), or ``padding_stack`` gives each sequence of the
  batch its own mask: the pattern cut to that sequence's length (query and
  key positions past it take no part), lengths uniform in [S/2, S] from
  ``default_rng(seed + 1000)``.
"""
import numpy as np
import torch

_TORCH_DT = {"f16": torch.float16, "bf16": torch.bfloat16,
             "f32": torch.float32}


def torch_dtype(name):
    return _TORCH_DT[name]


def make_qkv(B, H, S, d, dtype, seed, device="cpu"):
    """Return (q, k, v) as [B, H, S, d] tensors of ``dtype`` on ``device``."""
    g = torch.Generator().manual_seed(int(seed))
    out = []
    for _ in range(3):
        x = torch.randn(B, H, S, d, generator=g, dtype=torch.float32)
        out.append(x.to(_TORCH_DT[dtype]).to(device))
    return tuple(out)


def _causal(S):
    return np.tril(np.ones((S, S), dtype=bool))


def _band(S, w):
    m = np.zeros((S, S), dtype=bool)
    for r0 in range(0, S, 1024):
        i = np.arange(r0, min(S, r0 + 1024), dtype=np.int32)[:, None]
        j = np.arange(S, dtype=np.int32)[None, :]
        m[r0:r0 + 1024] = np.abs(i - j) <= w
    return m


def _bigbird_blocks(nb, rng, n_random=3):
    """Block rows of BigBird: sliding {I-1, I, I+1} and global {0, nb-1}
    blocks (base), and n_random seeded random blocks among the rest."""
    base = np.zeros((nb, nb), dtype=bool)
    rand = np.zeros((nb, nb), dtype=bool)
    for I in range(nb):
        chosen = {x for x in (I - 1, I, I + 1) if 0 <= x < nb} | {0, nb - 1}
        cand = sorted(set(range(nb)) - chosen)
        picks = rng.choice(cand, n_random, replace=False)
        for J in chosen:
            base[I, J] = True
        for J in picks:
            rand[I, J] = True
    return base, rand


def _bigbird(S, rng, block=64, n_random=3, drop=0.2):
    nb = S // block
    base, rand = _bigbird_blocks(nb, rng, n_random)
    keep = rng.random((S, S), dtype=np.float32) >= drop
    one = np.ones((block, block), dtype=bool)
    return np.kron(base, one) | (np.kron(rand, one) & keep)


def _long_random(S, rng, w=1024, p=0.02):
    u = rng.random((S, S), dtype=np.float32)
    m = u < p
    del u
    for r0 in range(0, S, 1024):
        i = np.arange(r0, min(S, r0 + 1024), dtype=np.int32)[:, None]
        j = np.arange(S, dtype=np.int32)[None, :]
        m[r0:r0 + 1024] |= np.abs(i - j) <= w
        m[r0:r0 + 1024] &= j <= i
    return m


def mask_family(family, S, seed=0, **kw):
    """Build an [S, S] bool mask of one family.

    families: ``causal``; ``window64`` (|i-j| <= 64); ``window`` (|i-j| <=
    kw['w']); ``longformer`` (causal AND (|i-j| <= 256 OR i < 16 OR j < 16));
    ``bigbird``; ``long_random`` (causal AND (|i-j| <= 1024 OR U < 0.02));
    ``random`` (Bernoulli(kw['p']) per element); ``sparse_random``
    (Bernoulli(0.001)); ``far_random`` (causal AND U < 0.02: long_random
    without its band); ``full``; ``empty``.
    """
    rng = np.random.default_rng(int(seed))
    if family == "causal":
        return _causal(S)
    if family == "window64":
        return _band(S, 64)
    if family == "window":
        return _band(S, int(kw["w"]))
    if family == "longformer":
        i = np.arange(S, dtype=np.int32)[:, None]
        j = np.arange(S, dtype=np.int32)[None, :]
        return (j <= i) & ((np.abs(i - j) <= 256) | (i < 16) | (j < 16))
    if family == "bigbird":
        return _bigbird(S, rng)
    if family == "long_random":
        return _long_random(S, rng, w=int(kw.get("w", 1024)),
                            p=float(kw.get("p", 0.02)))
    if family == "far_random":
        return _long_random(S, rng, w=-1, p=float(kw.get("p", 0.02)))
    if family == "random":
        return rng.random((S, S), dtype=np.float32) < float(kw["p"])
    if family == "sparse_random":
        return rng.random((S, S), dtype=np.float32) < float(kw.get("p", 0.001))
    if family == "full":
        return np.ones((S, S), dtype=bool)
    if family == "empty":
        return np.zeros((S, S), dtype=bool)
    raise ValueError(f"unknown mask family {family!r}")


def make_mask(cfg):
    """The [S, S] bool mask of a workload Config (seeded by cfg.cid)."""
    return mask_family(cfg.family, cfg.S, seed=cfg.cid)


def padding_stack(mask, B, seed):
    """[B, 1, S, S] bool: sequence b keeps mask[i, j] for i, j < L_b, with
    L_b drawn uniformly from [S // 2, S] (variable-length batches)."""
    S = mask.shape[0]
    rng = np.random.default_rng(int(seed) + 1000)
    lens = rng.integers(S // 2, S + 1, B)
    out = np.zeros((B, 1, S, S), dtype=bool)
    for b, L in enumerate(lens):
        out[b, 0, :L, :L] = mask[:L, :L]
    return out


def pattern_of(cfg):
    """The workload's mask family as a pattern (keyword arguments of the
    pattern encoder and of oracle.pattern.pattern_mask).  Causal, window and
    Longformer masks are the same masks as make_mask's; BigBird keeps the
    same block choice (rng seeded the same) and long_random the same band,
    with their element draws from the pattern's SplitMix64 stream (seed =
    workload id) instead of PCG64, so those two are the same families with
    other random elements."""
    S, fam = cfg.S, cfg.family
    if fam == "causal":
        return dict(causal=True, window=S)
    if fam == "window64":
        return dict(window=64)
    if fam == "longformer":
        return dict(causal=True, window=256, global_rows=16, global_cols=16)
    if fam == "bigbird":
        base, rand = _bigbird_blocks(S // 64, np.random.default_rng(cfg.cid))
        blocks = base.astype(np.uint8) + 2 * (rand & ~base).astype(np.uint8)
        return dict(blocks=blocks, block_keep=0.8, seed=cfg.cid)
    if fam == "long_random":
        return dict(causal=True, window=1024, random_p=0.02, seed=cfg.cid)
    if fam == "sparse_random":
        return dict(random_p=0.001, seed=cfg.cid)
    if fam == "far_random":
        return dict(causal=True, random_p=0.02, seed=cfg.cid)
    raise ValueError(f"no pattern for family {fam!r}")
