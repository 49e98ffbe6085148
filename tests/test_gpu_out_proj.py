"""GPU output projection (one fused launch: head merge, MFMA product,
bias, residual) against the fp64 oracle, element by element.

Bar, per element: |got - ref| <= 2^-p |ref| + 1e-4 (sum_k |x_k w_k| +
|bias| + |residual|) + 2^-24, p = 10 for fp16 and 7 for bf16 outputs: the
one rounding of the result to the output type (at most half a unit in the
last place, 2^-(p+1) |ref|, here with twice that room) plus fp32
accumulation of K <= 2048 products (K * 2^-24 relative to the sum of
magnitudes, under 1.3e-4 K/2048) and the fp16 subnormal spacing."""
import numpy as np
import pytest
import torch

import sparse_masked_head_amd as smh
from oracle.out_proj import abs_products, out_proj
from tests.gpu_util import TDT, need_gpu

pytestmark = pytest.mark.gpu

P = {"f16": 10, "bf16": 7}


def inputs(B, H, S, d, D, dt, seed):
    g = torch.Generator().manual_seed(seed)
    K = H * d
    o = torch.randn(B, H, S, d, generator=g).to(TDT[dt])
    w = (torch.randn(D, K, generator=g) / K ** 0.5).to(TDT[dt])
    b = (0.1 * torch.randn(D, generator=g)).to(TDT[dt])
    r = torch.randn(B, S, D, generator=g).to(TDT[dt])
    return o, w, b, r


def check(got, o, w, b, r, dt):
    ref = out_proj(o, w, b, r)
    scale = abs_products(o, w)
    if b is not None:
        scale = scale + np.abs(b.double().numpy())
    if r is not None:
        scale = scale + np.abs(r.double().numpy())
    tol = 2.0 ** -P[dt] * np.abs(ref) + 1e-4 * scale + 2.0 ** -24
    err = np.abs(got.double().cpu().numpy() - ref)
    bad = err > tol
    assert not bad.any(), (f"{int(bad.sum())} elements over the bar; worst "
                           f"{float((err - tol).max()):.3e}")


@pytest.mark.parametrize("B,H,S,d,D,dt", [
    (1, 1, 64, 64, 64, "f16"),
    (2, 3, 100, 64, 128, "f16"),        # ragged rows (B*S = 200)
    (2, 12, 512, 64, 768, "f16"),       # BERT-base shaped
    (1, 4, 33, 128, 256, "bf16"),
    (4, 32, 70, 128, 512, "bf16"),      # K = 4096
    # 128 x 128 tiles (>= 256 of them, fewer than 256 of 256 x 256)
    (2, 4, 2048, 64, 1024, "f16"),
    (1, 2, 4000, 128, 1024, "bf16"),    # ragged last row tile
    # 256 x 256 tiles (N % 256 == 0, >= 256 workgroups, K % 128 == 0)
    (2, 4, 2000, 64, 4096, "f16"),      # ragged last row tile (M = 4000)
    (1, 8, 4096, 128, 4096, "bf16"),    # K = 1024: the stage ring wraps
])
def test_out_proj_matches_oracle(B, H, S, d, D, dt):
    dev = need_gpu()
    print(f"out_proj {B} {H} {S} {d} {D} {dt}", flush=True)
    o, w, b, r = inputs(B, H, S, d, D, dt, seed=S + D)
    got = smh.out_proj(o.to(dev), w.to(dev), b.to(dev), r.to(dev))
    torch.cuda.synchronize()
    check(got, o, w, b, r, dt)


def test_optional_terms_and_in_place():
    dev = need_gpu()
    B, H, S, d, D, dt = 2, 2, 96, 64, 192, "f16"
    o, w, b, r = inputs(B, H, S, d, D, dt, seed=3)
    od, wd, bd, rd = (x.to(dev) for x in (o, w, b, r))
    check(smh.out_proj(od, wd), o, w, None, None, dt)
    check(smh.out_proj(od, wd, bias=bd), o, w, b, None, dt)
    check(smh.out_proj(od, wd, residual=rd), o, w, None, r, dt)
    inplace = rd.clone()
    smh.out_proj(od, wd, bd, inplace, out=inplace)     # residual += proj
    torch.cuda.synchronize()
    check(inplace, o, w, b, r, dt)


def test_attention_then_projection():
    """The fused pair as a layer would run it: attention output straight
    into the projection (nothing reshaped in between)."""
    dev = need_gpu()
    from oracle.attention import attention
    from workloads import make_qkv, mask_family
    B, H, S, d, D = 2, 4, 192, 64, 256
    mask = mask_family("window", S, w=40)
    q, k, v = make_qkv(B, H, S, d, "f16", seed=5)
    enc = smh.encode_mask(torch.from_numpy(mask).to(dev))
    att = smh.sparse_mha_fwd(q.to(dev), k.to(dev), v.to(dev), enc)
    _, w, b, r = inputs(B, H, S, d, D, "f16", seed=6)
    got = smh.out_proj(att, w.to(dev), b.to(dev), r.to(dev))
    torch.cuda.synchronize()
    # the projection of the kernel's own attention output, and close to the
    # projection of the exact attention
    check(got, att.cpu(), w, b, r, "f16")
    ref = out_proj(attention(q, k, v, mask), w, b, r)
    assert float(np.abs(got.double().cpu().numpy() - ref).max()) < 1e-2


def test_validation():
    dev = need_gpu()
    o = torch.zeros((1, 2, 64, 64), dtype=torch.float16, device=dev)
    w = torch.zeros((96, 128), dtype=torch.float16, device=dev)
    with pytest.raises(smh.SmhError) as e:            # D % 64 != 0
        smh.out_proj(o, w)
    assert e.value.status == 2
    with pytest.raises(ValueError):
        smh.out_proj(o, torch.zeros((64, 100), dtype=torch.float16,
                                    device=dev))
    out = smh.out_proj(o[:0], torch.zeros((64, 128), dtype=torch.float16,
                                          device=dev))
    assert out.shape == (0, 64, 64)
