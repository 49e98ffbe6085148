"""smh: sparse masked multi-head attention forward for AMD MI355X (gfx950).

Python binding of libsmh.so (include/smh.h), argument marshalling only:
every step runs in the library's HIP kernels.  torch provides device memory
and the current stream.  Function names are the C names without the
``smh_`` prefix.

    enc = encode_mask(mask)                 # mask: cuda bool/uint8 [S, S]
                                            # or [Bm, Hm, S, S], Bm in {1, B},
                                            # Hm in {1, H}: one mask per
                                            # batch and/or head
    st = mask_stats_get(enc)                # host statistics (syncs)
    which = select_kernel(st, B, H, d, torch.float16)
    o = sparse_mha_fwd(q, k, v, enc, kernel="auto", stats=st)
"""
import ctypes

import torch

from ._lib import (SMH_AUTO, SMH_BF16, SMH_BLOCKWISE, SMH_BLOCKWISE_DENSE,
                   SMH_F16, SMH_F32,
                   SMH_MAX_S, SMH_OK, SMH_ROWWISE, MaskEnc, MaskStats,
                   Pattern, SmhError, check, lib, status_string)

__all__ = ["encode_mask", "encode_masks_noalloc", "encode_pattern",
           "encode_workspace_bytes",
           "mask_stats_get",
           "select_kernel", "select_costs", "sparse_mha_fwd", "out_proj",
           "version",
           "MaskEncoding", "SmhError", "KERNELS"]

KERNELS = {"auto": SMH_AUTO, "rowwise": SMH_ROWWISE,
           "blockwise": SMH_BLOCKWISE, "blockwise_dense": SMH_BLOCKWISE_DENSE}
_KNAME = {v: k for k, v in KERNELS.items()}
_DT = {torch.float16: SMH_F16, torch.bfloat16: SMH_BF16,
       torch.float32: SMH_F32}


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dt(x):
    if x not in _DT:
        raise TypeError(f"unsupported dtype {x}")
    return _DT[x]


def version():
    return lib().smh_version().decode()


def encode_workspace_bytes(S, mask_b=1, mask_h=1):
    return int(lib().smh_encode_masks_workspace_bytes(int(mask_b),
                                                      int(mask_h), int(S)))


class MaskEncoding:
    """The encoding of a stack of masks [mask_b, mask_h, S, S]: the device
    workspace that holds it and the C struct of pointers into that
    workspace."""

    def __init__(self, workspace, enc, S, mask_b=1, mask_h=1):
        self.workspace = workspace
        self.enc = enc
        self.S = S
        self.mask_b = mask_b
        self.mask_h = mask_h
        self.device = workspace.device

    @property
    def rows(self):
        """Outer-tile rows of the encoding (masks * ceil(S / 64))."""
        return self.mask_b * self.mask_h * (-(-self.S // 64))

    def arrays(self, stats=None):
        """Views of the encoding arrays (device tensors), trimmed to their
        used length (needs the host statistics)."""
        st = stats if stats is not None else mask_stats_get(self)
        n = self.rows
        base = self.workspace.data_ptr()

        def view(ptr, count, dtype, width):
            off = ptr - base
            return self.workspace[off:off + count * width].view(dtype)
        e = self.enc
        return dict(
            full_row_ptr=view(e.full_row_ptr, n + 1, torch.int32, 4),
            full_col_idx=view(e.full_col_idx, st["n_full"], torch.int32, 4),
            part_row_ptr=view(e.part_row_ptr, n + 1, torch.int32, 4),
            part_col_idx=view(e.part_col_idx, st["n_partial"], torch.int32, 4),
            part_bitmaps=view(e.part_bitmaps, st["n_partial"] * 64,
                              torch.int64, 8).view(-1, 64),
            row_order=view(e.row_order, n, torch.int32, 4),
            row_info=view(e.row_info, 16 * n, torch.int32, 4).view(-1, 16),
            part_pop=view(e.part_pop, st["n_partial"], torch.int32, 4),
            row_ent_cnt=view(e.row_ent_cnt, 4 * n, torch.int32, 4).view(-1, 4),
            row_ent=view(e.row_ent, 256 * st["n_partial"], torch.int32, 4))


def encode_mask(mask, workspace=None):
    """Encode a device mask (bool or uint8, nonzero = attend): one [S, S]
    mask, or a stack [mask_b, mask_h, S, S] whose mask (b', h') serves
    batch b and head h with b' = b if mask_b > 1 else 0 and h' likewise."""
    if mask.dtype not in (torch.bool, torch.uint8):
        raise TypeError("mask must be bool or uint8")
    if not mask.is_cuda:
        raise ValueError("mask must be a device tensor")
    if mask.dim() not in (2, 4) or mask.shape[-1] != mask.shape[-2]:
        raise ValueError("mask must be [S, S] or [mask_b, mask_h, S, S]")
    mask = mask.contiguous()
    if mask.data_ptr() % 16:
        mask = mask.clone()
    S = int(mask.shape[-1])
    mb, mh = (1, 1) if mask.dim() == 2 else (int(mask.shape[0]),
                                              int(mask.shape[1]))
    nbytes = encode_workspace_bytes(S, mb, mh)
    if nbytes == 0:
        check(lib().smh_encode_masks(None, mb, mh, S, None, 0,
                                     ctypes.byref(MaskEnc()), None),
              "smh_encode_masks")
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=mask.device)
    enc = MaskEnc()
    st = lib().smh_encode_masks(
        ctypes.c_void_p(mask.data_ptr()), mb, mh, S,
        ctypes.c_void_p(workspace.data_ptr()), workspace.numel(),
        ctypes.byref(enc), _stream(mask.device))
    check(st, "smh_encode_masks")
    return MaskEncoding(workspace, enc, S, mb, mh)


def encode_masks_noalloc(mask, out=None):
    """encode_mask through smh_encode_masks_noalloc: the library allocates
    nothing (its encoder scratch is a static device array) and the
    encoding goes to `out` (a device uint8 tensor of at least
    encode_noalloc_bytes(...) bytes; allocated here when None)."""
    if mask.dtype not in (torch.bool, torch.uint8) or not mask.is_cuda:
        raise TypeError("mask must be a bool or uint8 device tensor")
    if mask.dim() not in (2, 4) or mask.shape[-1] != mask.shape[-2]:
        raise ValueError("mask must be [S, S] or [mask_b, mask_h, S, S]")
    mask = mask.contiguous()
    if mask.data_ptr() % 16:
        mask = mask.clone()
    S = int(mask.shape[-1])
    mb, mh = (1, 1) if mask.dim() == 2 else (int(mask.shape[0]),
                                              int(mask.shape[1]))
    need = encode_noalloc_bytes(S, mb, mh)
    if out is None:
        out = torch.empty(max(need, 1), dtype=torch.uint8, device=mask.device)
    cap = ctypes.c_size_t(out.numel())
    enc = MaskEnc()
    check(lib().smh_encode_masks_noalloc(
        ctypes.c_void_p(mask.data_ptr()), mb, mh, S,
        ctypes.c_void_p(out.data_ptr()), ctypes.byref(cap),
        ctypes.byref(enc), _stream(mask.device)), "smh_encode_masks_noalloc")
    return MaskEncoding(out, enc, S, mb, mh)


def encode_noalloc_bytes(S, mask_b=1, mask_h=1):
    """Bytes of the encoding buffer smh_encode_masks_noalloc writes (its
    size query: nothing is enqueued)."""
    n = ctypes.c_size_t(0)
    check(lib().smh_encode_masks_noalloc(None, int(mask_b), int(mask_h),
                                         int(S), None, ctypes.byref(n), None,
                                         None), "smh_encode_masks_noalloc")
    return int(n.value)


def encode_pattern(S, causal=False, window=-1, global_rows=0, global_cols=0,
                   blocks=None, block_keep=1.0, random_p=0.0, seed=0,
                   device=None, workspace=None):
    """Encode the mask a pattern describes (include/smh.h, smh_pattern),
    without a dense mask: causal limit, band |i - j| <= window, global rows
    and columns, a [n_ot, n_ot] uint8 device block map (1: block valid,
    other nonzero: its elements kept with probability block_keep), and
    other elements valid with probability random_p (SplitMix64 draws from
    `seed`)."""
    S = int(S)
    if blocks is not None:
        n = -(-S // 64)
        if blocks.dtype != torch.uint8 or tuple(blocks.shape) != (n, n) or \
                not blocks.is_cuda:
            raise ValueError(f"blocks must be a device uint8 [{n}, {n}] map")
        blocks = blocks.contiguous()
        device = blocks.device
    device = torch.device("cuda", torch.cuda.current_device()) \
        if device is None else torch.device(device)
    pat = Pattern(int(bool(causal)), int(window), int(global_rows),
                  int(global_cols),
                  ctypes.c_void_p(blocks.data_ptr()) if blocks is not None
                  else None, float(block_keep), float(random_p),
                  int(seed) & ((1 << 64) - 1))
    nbytes = encode_workspace_bytes(S)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8,
                                device=device)
    enc = MaskEnc()
    check(lib().smh_encode_pattern(
        ctypes.byref(pat), S, ctypes.c_void_p(workspace.data_ptr()),
        workspace.numel(), ctypes.byref(enc), _stream(device)),
        "smh_encode_pattern")
    enc_obj = MaskEncoding(workspace, enc, S)
    enc_obj.blocks = blocks          # the map must outlive the launches
    return enc_obj


def mask_stats_get(enc):
    """Host statistics of an encoding (synchronises the current stream)."""
    out = MaskStats()
    check(lib().smh_mask_stats_get(ctypes.byref(enc.enc), ctypes.byref(out),
                                   _stream(enc.device)), "smh_mask_stats_get")
    return out.as_dict()


def _stats_struct(st):
    s = MaskStats()
    for k, _ in MaskStats._fields_:
        # a dict without the stack shape describes one mask, one without the
        # sparse-tile counts a mask with no sparse tile
        dflt = {"mask_b": 1, "mask_h": 1, "n_sparse": 0, "sparse_nnz": 0,
                "row_entries": 0}
        setattr(s, k, int(st[k] if k in st else dflt[k]))
    return s


def select_kernel(stats, B, H, d, dtype):
    """'rowwise' or 'blockwise' for this mask and shape (host only)."""
    out = ctypes.c_int()
    check(lib().smh_select_kernel(ctypes.byref(_stats_struct(stats)), B, H, d,
                                  _dt(dtype), ctypes.byref(out)),
          "smh_select_kernel")
    return _KNAME[out.value]


def select_costs(stats, B, H, d, dtype):
    """The selector's predicted (rowwise_us, blockwise_us)."""
    a, b = ctypes.c_double(), ctypes.c_double()
    check(lib().smh_select_costs(ctypes.byref(_stats_struct(stats)), B, H, d,
                                 _dt(dtype), ctypes.byref(a), ctypes.byref(b)),
          "smh_select_costs")
    return a.value, b.value


def sparse_mha_fwd(q, k, v, enc, kernel="auto", out_dtype=None, scale=0.0,
                   stats=None, out=None):
    """Masked attention forward over [B, H, S, d] device tensors.

    kernel="auto" with stats=None lets the device decide from the
    encoding's statistics (no host synchronisation); with host stats the
    host decides.  kernel="rowwise" / "blockwise" forces one kernel."""
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share a [B, H, S, d] shape")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share a dtype")
    for t in (q, k, v):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous device tensors")
    B, H, S, d = (int(x) for x in q.shape)
    out_dtype = q.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((B, H, S, d), dtype=out_dtype, device=q.device)
    elif out.shape != q.shape or out.dtype != out_dtype or \
            not out.is_contiguous():
        raise ValueError("out must be a contiguous [B, H, S, d] tensor of "
                         "out_dtype")
    if kernel not in KERNELS:
        raise ValueError(f"kernel must be one of {sorted(KERNELS)}")
    st = ctypes.byref(_stats_struct(stats)) if stats is not None else None
    rc = lib().smh_sparse_mha_fwd(
        ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
        ctypes.c_void_p(v.data_ptr()), ctypes.c_void_p(out.data_ptr()),
        B, H, S, d, _dt(q.dtype), _dt(out_dtype), float(scale),
        ctypes.byref(enc.enc), KERNELS[kernel], st, _stream(q.device))
    check(rc, "smh_sparse_mha_fwd")
    return out


def out_proj(o, w, bias=None, residual=None, out=None):
    """out[b, s, :] = sum_h o[b, h, s, :] @ w[:, h*d:(h+1)*d].T + bias +
    residual[b, s, :] in one fused launch.  o: [B, H, S, d] (the attention
    output), w: [D, H*d] (a linear layer's weight), bias: [D], residual and
    out: [B, S, D]; one dtype (fp16 or bf16); out may be residual."""
    if o.dim() != 4:
        raise ValueError("o must be [B, H, S, d]")
    B, H, S, d = (int(x) for x in o.shape)
    if w.dim() != 2 or w.shape[1] != H * d:
        raise ValueError("w must be [D, H*d]")
    D = int(w.shape[0])
    for name, t, shape in (("bias", bias, (D,)), ("residual", residual,
                                                 (B, S, D))):
        if t is not None and (tuple(t.shape) != shape or t.dtype != o.dtype
                              or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous {shape} tensor "
                             f"of o's dtype")
    if not (o.is_contiguous() and w.is_contiguous()) or w.dtype != o.dtype:
        raise ValueError("o and w must be contiguous and share a dtype")
    if out is None:
        out = torch.empty((B, S, D), dtype=o.dtype, device=o.device)
    elif tuple(out.shape) != (B, S, D) or out.dtype != o.dtype or \
            not out.is_contiguous():
        raise ValueError("out must be a contiguous [B, S, D] tensor")

    def ptr(t):
        return ctypes.c_void_p(t.data_ptr()) if t is not None else None
    check(lib().smh_out_proj(ptr(o), ptr(w), ptr(bias), ptr(residual),
                             ptr(out), B, H, S, d, D, _dt(o.dtype),
                             _stream(o.device)), "smh_out_proj")
    return out
