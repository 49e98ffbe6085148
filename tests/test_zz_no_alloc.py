"""The allocation-free encoder entry point against the workspace encoder.

smh_encode_masks_noalloc (its scratch: the library's static device array)
must give bit-identical encodings to smh_encode_masks (its scratch: the
caller's workspace).  Called through the C ABI on several calls in a row,
each later one smaller than the one before it (the static scratch keeps
the previous call's contents), including the largest mask the static
scratch admits (the 16k workload)."""
import ctypes

import numpy as np
import pytest
import torch

import sparse_masked_head_amd as smh
from sparse_masked_head_amd import _lib as L
from tests.gpu_util import counted_row_entries, need_gpu
from workloads import get_config, make_mask, make_qkv, mask_family

pytestmark = pytest.mark.gpu


def noalloc_call(mask_d, buf):
    """smh_encode_masks_noalloc through ctypes into the preallocated buf."""
    S = int(mask_d.shape[-1])
    mb, mh = (1, 1) if mask_d.dim() == 2 else tuple(int(x) for x in
                                                    mask_d.shape[:2])
    need = ctypes.c_size_t(0)
    rc = L.lib().smh_encode_masks_noalloc(None, mb, mh, S, None,
                                          ctypes.byref(need), None, None)
    assert rc == L.SMH_OK and 0 < need.value <= buf.numel()
    cap = ctypes.c_size_t(buf.numel())
    e = L.MaskEnc()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = L.lib().smh_encode_masks_noalloc(
        ctypes.c_void_p(mask_d.data_ptr()), mb, mh, S,
        ctypes.c_void_p(buf.data_ptr()), ctypes.byref(cap), ctypes.byref(e),
        stream)
    assert rc == L.SMH_OK, L.status_string(rc)
    return smh.MaskEncoding(buf, e, S, mb, mh)


def assert_same(a, b):
    sa, sb = smh.mask_stats_get(a), smh.mask_stats_get(b)
    assert sa == sb
    xa, xb = a.arrays(sa), b.arrays(sb)
    for k in xa:
        if k != "row_ent":     # only its counted entries are written
            assert torch.equal(xa[k], xb[k]), k
    assert np.array_equal(counted_row_entries(xa), counted_row_entries(xb))


def test_noalloc_matches_workspace_encoder():
    dev = need_gpu()
    # one buffer for every call: the largest encoding below
    buf = torch.empty(smh.encode_noalloc_bytes(16384), dtype=torch.uint8,
                      device=dev)
    rng = np.random.default_rng(5)
    cases = [
        ("16k workload mask", make_mask(get_config(5))),
        ("S=3000 band + 3%", (mask_family("window", 3000, w=200) |
                              (rng.random((3000, 3000)) < 0.03))),
        ("stack 2x3 S=300", rng.random((2, 3, 300, 300)) < 0.2),
        ("S=100 causal", mask_family("causal", 100)),
    ]
    for name, mask in cases:
        print(f"noalloc {name}", flush=True)
        md = torch.from_numpy(np.ascontiguousarray(mask)).to(dev)
        buf.fill_(0xAB)                       # stale bytes in the output
        got = noalloc_call(md, buf)
        want = smh.encode_mask(md)
        torch.cuda.synchronize()
        assert_same(got, want)
        if mask.ndim == 2 and mask.shape[0] <= 3000:   # the encoding works
            S = mask.shape[0]
            q, k, v = (x.to(dev) for x in make_qkv(1, 2, S, 64, "f16", 3))
            a = smh.sparse_mha_fwd(q, k, v, got, kernel="auto")
            b = smh.sparse_mha_fwd(q, k, v, want, kernel="auto")
            torch.cuda.synchronize()
            assert torch.equal(a, b)


def test_noalloc_rejects_without_touching_the_device():
    """Scratch beyond the static array and a short buffer are refused
    before anything is enqueued."""
    need = ctypes.c_size_t(0)
    f = L.lib().smh_encode_masks_noalloc
    assert f(None, 2, 1, 16384, None, ctypes.byref(need), None, None) == 0
    cap = ctypes.c_size_t(need.value)
    e = L.MaskEnc()
    fake = ctypes.c_void_p(1 << 20)
    assert f(fake, 2, 1, 16384, fake, ctypes.byref(cap), ctypes.byref(e),
             None) == L.SMH_EUNSUPPORTED
    assert f(None, 1, 1, 4096, None, ctypes.byref(need), None, None) == 0
    small = ctypes.c_size_t(need.value - 256)
    assert f(fake, 1, 1, 4096, fake, ctypes.byref(small), ctypes.byref(e),
             None) == L.SMH_ENOSPACE
