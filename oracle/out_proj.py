"""Output projection with bias and residual, reference side: the
definition written out in fp64.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The fused operator after MHA ("Accelerating Sparse Transformer Inference on
GPU", gist.science explainer, Technical summary > Methodology > 2. operator
fusion): the attention output of every head, concatenated per token
(head-major), times the projection weight, plus bias and the residual:

    out[b, s, n] = sum_h sum_k O[b, h, s, k] W[n, h*d + k] + bias[n]
                   + residual[b, s, n]
"""
import numpy as np


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):
        import torch
        return x.detach().to("cpu").to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def merge_heads(o):
    """[B, H, S, d] -> [B, S, H*d]: token (b, s) lists head 0's d values,
    then head 1's, ..."""
    o = _f64(o)
    B, H, S, d = o.shape
    return o.transpose(0, 2, 1, 3).reshape(B, S, H * d)


def out_proj(o, w, bias=None, residual=None):
    """fp64 [B, S, D]."""
    x = merge_heads(o)
    out = x @ _f64(w).T
    if bias is not None:
        out = out + _f64(bias)
    if residual is not None:
        out = out + _f64(residual)
    return out


def abs_products(o, w):
    """sum_k |x[b, s, k]| |W[n, k]|: scale of the fp32 accumulation error."""
    return np.abs(merge_heads(o)) @ np.abs(_f64(w)).T
