"""The C-ABI library loads, exports every symbol include/smh.h declares, and
rejects bad arguments on the host before touching a device (no GPU needed:
every call below returns from validation, which makes no HIP call)."""
import ctypes
import os
import re

import pytest

from sparse_masked_head_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "smh.h")


def declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(smh_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = L.lib()
    names = declared()
    assert names == sorted(L.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_version():
    assert L.status_string(L.SMH_OK) == "ok"
    assert "workspace" in L.status_string(L.SMH_ENOSPACE)
    assert L.lib().smh_version().decode().startswith("smh")
    assert L.status_string(99) == "unknown status"


def test_workspace_bytes():
    f = L.lib().smh_encode_workspace_bytes
    assert f(-64) == 0 and f(L.SMH_MAX_S + 64) == 0
    assert f(0) > 0 and f(65) >= f(128) > f(64)    # ragged S rounds up
    small, big = f(64), f(16384)
    assert 0 < small < big
    n = 16384 // 64
    # encoding + scratch: at least two bitmap areas of n^2 * 512 bytes
    assert big >= 2 * n * n * 512
    g = L.lib().smh_encode_masks_workspace_bytes
    assert g(1, 1, 512) == f(512)
    assert g(2, 3, 512) >= 6 * 8 * 8 * 512 * 2 > f(512)
    assert g(0, 1, 64) == 0 and g(1, -1, 64) == 0
    assert g(32, 32, 512) > 0 and g(32, 33, 512) == 0   # 8192 rows at most


FAKE = ctypes.c_void_p(1 << 20)      # never dereferenced: validation fails first


def encode(mask, S, ws, nbytes, enc=True):
    e = L.MaskEnc()
    return L.lib().smh_encode_mask(mask, S, ws, nbytes,
                                   ctypes.byref(e) if enc else None, None)


def encode_stack(masks, mb, mh, S, ws, nbytes):
    e = L.MaskEnc()
    return L.lib().smh_encode_masks(masks, mb, mh, S, ws, nbytes,
                                    ctypes.byref(e), None)


def test_encode_validation():
    f = L.lib().smh_encode_workspace_bytes
    g = L.lib().smh_encode_masks_workspace_bytes
    assert encode(FAKE, -64, FAKE, 1 << 30) == L.SMH_EINVAL
    assert encode(FAKE, L.SMH_MAX_S + 64, FAKE, 1 << 40) == L.SMH_EINVAL
    assert encode(FAKE, 128, FAKE, f(128), enc=False) == L.SMH_EINVAL
    assert encode(None, 128, FAKE, f(128)) == L.SMH_EINVAL
    assert encode(FAKE, 128, None, f(128)) == L.SMH_EINVAL
    assert encode(FAKE, 128, FAKE, f(128) - 1) == L.SMH_ENOSPACE
    assert encode(ctypes.c_void_p((1 << 20) + 8), 128, FAKE, f(128)) \
        == L.SMH_EINVAL                       # mask not 16-byte aligned
    assert encode(FAKE, 128, ctypes.c_void_p((1 << 20) + 16), f(128)) \
        == L.SMH_EINVAL                       # workspace not 256-byte aligned
    # mask inside the workspace
    ws = 1 << 24
    assert encode(ctypes.c_void_p(ws + 4096), 128, ctypes.c_void_p(ws),
                  f(128)) == L.SMH_EINVAL
    # stacks
    assert encode_stack(FAKE, 0, 1, 128, FAKE, 1 << 30) == L.SMH_EINVAL
    assert encode_stack(FAKE, 1, 8193, 64, FAKE, 1 << 40) == L.SMH_EINVAL
    assert encode_stack(FAKE, 2, 3, 128, FAKE, g(2, 3, 128) - 1) \
        == L.SMH_ENOSPACE
    assert encode_stack(FAKE, 2, 3, 128, FAKE, f(128)) == L.SMH_ENOSPACE
    # the last mask of the stack reaches into the workspace
    assert encode_stack(ctypes.c_void_p(ws - 6 * 128 * 128 + 16), 2, 3, 128,
                        ctypes.c_void_p(ws), g(2, 3, 128)) == L.SMH_EINVAL


def stats(**kw):
    s = L.MaskStats()
    base = dict(nnz=61888, S=512, n_full=8, n_partial=14, n_empty_rows=0,
                max_row_tiles=3, mask_b=1, mask_h=1)
    base.update(kw)
    for k, v in base.items():
        setattr(s, k, v)
    return s


def select(st, B=8, H=12, d=64, dt=L.SMH_F16):
    out = ctypes.c_int(-1)
    rc = L.lib().smh_select_kernel(ctypes.byref(st) if st is not None else
                                   None, B, H, d, dt, ctypes.byref(out))
    return rc, out.value


def test_select_validation_and_choice():
    rc, k = select(stats())
    assert rc == L.SMH_OK and k in (L.SMH_ROWWISE, L.SMH_BLOCKWISE)
    assert select(None)[0] == L.SMH_EINVAL
    assert select(stats(), d=96)[0] == L.SMH_EUNSUPPORTED
    assert select(stats(), dt=L.SMH_F32)[0] == L.SMH_EUNSUPPORTED
    assert select(stats(), B=-1)[0] == L.SMH_EINVAL
    assert select(stats(S=500))[0] == L.SMH_OK                # ragged S
    assert select(stats(n_full=100))[0] == L.SMH_EINVAL       # > n_ot^2
    assert select(stats(mask_b=0))[0] == L.SMH_EINVAL
    assert select(stats(mask_b=8))[0] == L.SMH_OK             # B = 8
    assert select(stats(mask_b=8, n_full=100))[0] == L.SMH_OK
    assert select(stats(mask_b=4))[0] == L.SMH_EINVAL         # B = 8
    assert select(stats(mask_h=12, mask_b=8))[0] == L.SMH_OK
    assert select(stats(mask_h=5))[0] == L.SMH_EINVAL
    assert select(stats(nnz=512 * 512 + 1))[0] == L.SMH_EINVAL
    assert select(stats(max_row_tiles=9))[0] == L.SMH_EINVAL
    a, b = ctypes.c_double(), ctypes.c_double()
    assert L.lib().smh_select_costs(ctypes.byref(stats()), 8, 12, 64,
                                    L.SMH_F16, ctypes.byref(a),
                                    ctypes.byref(b)) == L.SMH_OK
    assert a.value > 0 and b.value > 0
    assert L.lib().smh_select_costs(ctypes.byref(stats()), 8, 12, 64,
                                    L.SMH_F16, None, None) == L.SMH_OK


def test_select_cost_model_monotone():
    def costs(st, B=8, H=12, d=64):
        a, b = ctypes.c_double(), ctypes.c_double()
        assert L.lib().smh_select_costs(ctypes.byref(st), B, H, d, L.SMH_F16,
                                        ctypes.byref(a), ctypes.byref(b)) == 0
        return a.value, b.value
    r1, b1 = costs(stats())
    r2, b2 = costs(stats(), B=16)
    assert r2 >= r1 and b2 >= b1
    r3, b3 = costs(stats(), d=128)
    assert r3 >= r1 and b3 >= b1
    # 12 per-head copies of the mask (totals x 12) cost what one shared
    # mask costs: the same work
    r4, b4 = costs(stats(mask_h=12, nnz=12 * 61888, n_full=96,
                         n_partial=168))
    assert r4 == pytest.approx(r1, rel=1e-12)
    assert b4 == pytest.approx(b1, rel=1e-12)


def fwd(q=FAKE, k=FAKE, v=FAKE, o=ctypes.c_void_p(1 << 30), B=1, H=1, S=128,
        d=64, in_dt=L.SMH_F16, out_dt=L.SMH_F16, scale=0.0, enc="ok",
        which=L.SMH_BLOCKWISE, st=None, mb=1, mh=1, enc_S=128):
    e = L.MaskEnc()
    e.S, e.n_ot, e.mask_b, e.mask_h = enc_S, -(-enc_S // 64), mb, mh
    for name in ("full_row_ptr", "full_col_idx", "part_row_ptr",
                 "part_col_idx", "part_bitmaps", "stats", "row_order",
                 "row_info"):
        setattr(e, name, 1 << 28)
    return L.lib().smh_sparse_mha_fwd(
        q, k, v, o, B, H, S, d, in_dt, out_dt, scale,
        ctypes.byref(e) if enc == "ok" else None, which,
        ctypes.byref(st) if st is not None else None, None)


def test_fwd_validation():
    assert fwd(enc=None) == L.SMH_EINVAL
    assert fwd(S=256) == L.SMH_EINVAL                 # enc->S mismatch
    assert fwd(S=100) == L.SMH_EINVAL                 # enc->S mismatch
    assert fwd(S=100, enc_S=100, B=0) == L.SMH_OK     # ragged S accepted
    assert fwd(mb=2) == L.SMH_EINVAL                  # B = 1
    assert fwd(mh=2, H=3) == L.SMH_EINVAL
    assert fwd(mh=3, H=3, B=0) == L.SMH_OK
    assert fwd(mb=0) == L.SMH_EINVAL
    assert fwd(d=96) == L.SMH_EUNSUPPORTED
    assert fwd(in_dt=L.SMH_F32, out_dt=L.SMH_F32) == L.SMH_EUNSUPPORTED
    assert fwd(out_dt=L.SMH_BF16) == L.SMH_EUNSUPPORTED
    assert fwd(scale=float("nan")) == L.SMH_EINVAL
    assert fwd(scale=-1.0) == L.SMH_EINVAL
    assert fwd(which=7) == L.SMH_EINVAL
    assert fwd(which=L.SMH_AUTO, st=stats()) == L.SMH_EINVAL   # S differs
    assert fwd(B=-1) == L.SMH_EINVAL
    assert fwd(q=None) == L.SMH_EINVAL
    assert fwd(q=ctypes.c_void_p((1 << 20) + 2)) == L.SMH_EINVAL  # alignment
    assert fwd(o=FAKE) == L.SMH_EINVAL                # o overlaps q, k, v
    # empty batch: a valid no-op that enqueues nothing
    assert fwd(B=0) == L.SMH_OK and fwd(H=0, q=None) == L.SMH_OK


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(L, "_lib", None)
    monkeypatch.setattr(L, "LIB_PATH", str(tmp_path / "libsmh.so"))
    with pytest.raises(ImportError):
        L.lib()


def test_calibration_model_is_the_library_model():
    """The Python restatement the coefficients are fitted with
    (sparse_masked_head_amd.calibrate.model) computes the same times as the
    library's cost model (smh_select_costs), and the library picks row-wise
    exactly when t_row < ROW_MARGIN * t_blk, the rule the fit scores: a
    fit is then a fit of the model the library runs."""
    import numpy as np
    from sparse_masked_head_amd import calibrate as cal
    text = open(os.path.join(ROOT, "sparse_masked_head_amd", "csrc",
                             "select_model.h")).read()
    coef = {}
    for d in (64, 128):
        body = re.search(r"k%d\s*=\s*\{([^}]*)\}" % d, text).group(1)
        coef[d] = np.array([float(x) for x in body.split(",")])
        assert len(coef[d]) == 12
    margin = float(re.search(r"kRowMargin\s*=\s*([0-9.]+)", text).group(1))
    assert margin == cal.ROW_MARGIN
    rng = np.random.default_rng(5)
    picks = set()
    for _ in range(300):
        S = int(rng.choice([256, 512, 1024, 4096, 16384]))
        n = S // 64
        tiles = int(rng.integers(1, n * n + 1))
        if rng.random() < 0.5:   # dense-ish: any mix of full and partial
            n_full = int(rng.integers(0, tiles + 1))
            n_part = tiles - n_full
            nnz = 4096 * n_full + int(rng.integers(n_part, 4095 * n_part + 1))
        else:                    # very sparse: partial tiles, 0.1-1% dense
            n_full, n_part = 0, tiles
            nnz = max(n_part, int(n_part * 4096 * rng.uniform(0.001, 0.01)))
        max_row = int(rng.integers(-(-tiles // n), min(n, tiles) + 1))
        B, H, d = int(rng.integers(1, 9)), int(rng.integers(1, 65)), int(rng.choice([64, 128]))
        # sparse partial tiles and their row-wise entries (none, some, all)
        n_sp = int(rng.choice([0, n_part // 2, n_part]))
        sp_nnz = int(n_sp * rng.integers(1, L.SMH_SPARSE_TILE_MAX + 1)) if n_sp else 0
        ents = int(rng.integers(n_sp, sp_nnz + 1)) if n_sp else 0
        if rng.random() < 0.2:   # S > 65536 keeps no entries
            ents = 0
        st = L.MaskStats(nnz=nnz, S=S, n_full=n_full, n_partial=n_part,
                         n_empty_rows=0, max_row_tiles=max_row, mask_b=1,
                         mask_h=1, n_sparse=n_sp, sparse_nnz=sp_nnz,
                         row_entries=ents)
        a, b = ctypes.c_double(), ctypes.c_double()
        assert L.lib().smh_select_costs(ctypes.byref(st), B, H, d, L.SMH_F16,
                                        ctypes.byref(a), ctypes.byref(b)) == 0
        p = dict(S=S, BH=B * H, stats=dict(nnz=nnz, n_full=n_full,
                                           n_partial=n_part,
                                           max_row_tiles=max_row,
                                           n_sparse=n_sp, row_entries=ents))
        tr, tb = cal.model(coef[d], p)
        assert a.value == pytest.approx(tr, rel=1e-9)
        assert b.value == pytest.approx(tb, rel=1e-9)
        out = ctypes.c_int()
        assert L.lib().smh_select_kernel(ctypes.byref(st), B, H, d, L.SMH_F16,
                                         ctypes.byref(out)) == 0
        want = L.SMH_ROWWISE if a.value < margin * b.value else L.SMH_BLOCKWISE
        assert out.value == want
        picks.add(out.value)
    assert picks == {L.SMH_ROWWISE, L.SMH_BLOCKWISE}   # both sides exercised


def _header_struct_fields(name):
    """(field, is_pointer, base type) of `typedef struct { ... } name;` in
    smh.h, one declaration per field."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    end = text.index("} " + name + ";")
    body = text[text.rindex("typedef struct {", 0, end) + len("typedef struct {"):end]
    out = []
    for decl in body.split(";"):
        toks = decl.replace("*", " * ").split()
        if not toks:
            continue
        fname = toks[-1]
        ptr = "*" in toks
        base = [t for t in toks[:-1] if t not in ("*", "const")][-1]
        out.append((fname, ptr, base))
    return out


@pytest.mark.parametrize("cname,pyname", [("smh_mask_enc", "MaskEnc"),
                                          ("smh_mask_stats", "MaskStats"),
                                          ("smh_pattern", "Pattern")])
def test_ctypes_structs_match_header(cname, pyname):
    """The ctypes structures the binding passes by pointer have the header
    struct's fields in the same order with the same widths (a shorter
    structure would let the library write past it)."""
    width = {"int32_t": 4, "int64_t": 8, "uint64_t": 8, "float": 4}
    fields = _header_struct_fields(cname)
    cls = getattr(L, pyname)
    assert [f for f, _, _ in fields] == [f for f, _ in cls._fields_]
    for (f, ptr, ctype), (_, pytype) in zip(fields, cls._fields_):
        want = 8 if ptr else width[ctype.split()[-1]]
        assert ctypes.sizeof(pytype) == want, f
