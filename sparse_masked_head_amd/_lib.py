"""ctypes declarations of libsmh.so (include/smh.h).  Marshalling only."""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsmh.so")

SMH_OK, SMH_EINVAL, SMH_EUNSUPPORTED, SMH_ENOSPACE, SMH_EHIP = range(5)
SMH_F16, SMH_BF16, SMH_F32 = range(3)
SMH_AUTO, SMH_ROWWISE, SMH_BLOCKWISE, SMH_BLOCKWISE_DENSE = range(4)
SMH_MAX_S = 131072
SMH_MAX_ENC_ROWS = 8192
SMH_STATIC_SCRATCH_BYTES = 40 << 20
SMH_SPARSE_TILE_MAX = 112

# every exported name of include/smh.h
EXPORTS = ("smh_encode_workspace_bytes", "smh_encode_masks_workspace_bytes",
           "smh_encode_mask", "smh_encode_masks", "smh_encode_masks_noalloc",
           "smh_encode_pattern",
           "smh_mask_stats_get",
           "smh_select_kernel", "smh_select_costs", "smh_sparse_mha_fwd",
           "smh_out_proj",
           "smh_status_string", "smh_version")


class MaskEnc(ctypes.Structure):
    _fields_ = [("S", ctypes.c_int32), ("n_ot", ctypes.c_int32),
                ("mask_b", ctypes.c_int32), ("mask_h", ctypes.c_int32),
                ("full_row_ptr", ctypes.c_void_p),
                ("full_col_idx", ctypes.c_void_p),
                ("part_row_ptr", ctypes.c_void_p),
                ("part_col_idx", ctypes.c_void_p),
                ("part_bitmaps", ctypes.c_void_p),
                ("stats", ctypes.c_void_p),
                ("row_order", ctypes.c_void_p),
                ("row_info", ctypes.c_void_p),
                ("part_pop", ctypes.c_void_p),
                ("row_ent", ctypes.c_void_p),
                ("row_ent_cnt", ctypes.c_void_p)]


class Pattern(ctypes.Structure):
    _fields_ = [("causal", ctypes.c_int32), ("window", ctypes.c_int32),
                ("global_rows", ctypes.c_int32),
                ("global_cols", ctypes.c_int32),
                ("blocks", ctypes.c_void_p), ("block_keep", ctypes.c_float),
                ("random_p", ctypes.c_float), ("seed", ctypes.c_uint64)]


class MaskStats(ctypes.Structure):
    _fields_ = [("nnz", ctypes.c_int64), ("S", ctypes.c_int32),
                ("n_full", ctypes.c_int32), ("n_partial", ctypes.c_int32),
                ("n_empty_rows", ctypes.c_int32),
                ("max_row_tiles", ctypes.c_int32),
                ("mask_b", ctypes.c_int32), ("mask_h", ctypes.c_int32),
                ("n_sparse", ctypes.c_int32), ("sparse_nnz", ctypes.c_int64),
                ("row_entries", ctypes.c_int64)]

    def as_dict(self):
        return {k: getattr(self, k) for k, _ in self._fields_}


class SmhError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} ({status})")


_lib = None


def lib():
    """Load libsmh.so; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m sparse_masked_head_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        p, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        L.smh_encode_workspace_bytes.argtypes = [i32]
        L.smh_encode_workspace_bytes.restype = sz
        L.smh_encode_masks_workspace_bytes.argtypes = [i32, i32, i32]
        L.smh_encode_masks_workspace_bytes.restype = sz
        L.smh_encode_mask.argtypes = [p, i32, p, sz, ctypes.POINTER(MaskEnc),
                                      p]
        L.smh_encode_mask.restype = ctypes.c_int
        L.smh_encode_masks.argtypes = [p, i32, i32, i32, p, sz,
                                       ctypes.POINTER(MaskEnc), p]
        L.smh_encode_masks.restype = ctypes.c_int
        L.smh_encode_masks_noalloc.argtypes = [p, i32, i32, i32, p,
                                               ctypes.POINTER(sz),
                                               ctypes.POINTER(MaskEnc), p]
        L.smh_encode_masks_noalloc.restype = ctypes.c_int
        L.smh_encode_pattern.argtypes = [ctypes.POINTER(Pattern), i32, p, sz,
                                         ctypes.POINTER(MaskEnc), p]
        L.smh_encode_pattern.restype = ctypes.c_int
        L.smh_mask_stats_get.argtypes = [ctypes.POINTER(MaskEnc),
                                         ctypes.POINTER(MaskStats), p]
        L.smh_mask_stats_get.restype = ctypes.c_int
        L.smh_select_kernel.argtypes = [ctypes.POINTER(MaskStats), i32, i32,
                                        i32, ctypes.c_int,
                                        ctypes.POINTER(ctypes.c_int)]
        L.smh_select_kernel.restype = ctypes.c_int
        L.smh_select_costs.argtypes = [ctypes.POINTER(MaskStats), i32, i32,
                                       i32, ctypes.c_int,
                                       ctypes.POINTER(ctypes.c_double),
                                       ctypes.POINTER(ctypes.c_double)]
        L.smh_select_costs.restype = ctypes.c_int
        L.smh_sparse_mha_fwd.argtypes = [p, p, p, p, i32, i32, i32, i32,
                                         ctypes.c_int, ctypes.c_int,
                                         ctypes.c_float,
                                         ctypes.POINTER(MaskEnc),
                                         ctypes.c_int,
                                         ctypes.POINTER(MaskStats), p]
        L.smh_sparse_mha_fwd.restype = ctypes.c_int
        L.smh_out_proj.argtypes = [p, p, p, p, p, i32, i32, i32, i32, i32,
                                   ctypes.c_int, p]
        L.smh_out_proj.restype = ctypes.c_int
        L.smh_status_string.argtypes = [ctypes.c_int]
        L.smh_status_string.restype = ctypes.c_char_p
        L.smh_version.argtypes = []
        L.smh_version.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_string(s):
    return lib().smh_status_string(int(s)).decode()


def check(status, what):
    if status != SMH_OK:
        raise SmhError(status, what)
