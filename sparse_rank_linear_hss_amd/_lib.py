"""Loads libhss.so (built in-tree by sparse_rank_linear_hss_amd/build.py) and
declares its C signatures.  There is no fallback: if the library is missing
or does not load, importing the package fails with the reason."""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libhss.so")

HSS_OK = 0
HSS_ERR_INVALID_ARG = 1
HSS_ERR_UNSUPPORTED = 2
HSS_ERR_WORKSPACE = 3
HSS_ERR_NONFINITE = 4
HSS_ERR_HIP = 5

HSS_F32 = 0
HSS_BF16 = 1
HSS_FMT_CSR = 0
HSS_FMT_2OF4 = 1
HSS_MAX_BATCH = 2048
HSS_OPT_BATCH_ROUTE = 0
HSS_OPT_GRAD_DS_ROUTE = 1
HSS_OPT_DECODE_SPIN = 2
HSS_OPT_DECODE_MERGED = 3
HSS_OPT_DECODE_FORCE_LOCAL = 4
HSS_OPT_DECODE_WAVE_PRODUCERS = 5
HSS_OPT_DECODE_RPW = 6
HSS_COL16 = 1  # hss_matrix.flags: CSR col_idx holds uint16 columns
HSS_DQ4 = 2    # hss_matrix.flags: a 4-bit quantised dense part (dq_codes, dq_levels)
HSS_HIER2 = 4  # hss_matrix.flags: compact 2 x 2 block low-rank term (hier_r)

c_int32, c_int64, c_size_t, c_void_p = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p


class HssMatrixStruct(ctypes.Structure):
    """Mirror of struct hss_matrix in include/hss.h."""
    _fields_ = [
        ("fmt", c_int32), ("dtype", c_int32),
        ("m", c_int32), ("n", c_int32), ("r", c_int32), ("flags", c_int32),
        ("nnz", c_int64),
        ("row_ptr", c_void_p), ("col_idx", c_void_p), ("values", c_void_p),
        ("nm_values", c_void_p), ("nm_meta", c_void_p),
        ("U", c_void_p), ("Vt", c_void_p),
        ("dq_codes", c_void_p), ("dq_levels", c_void_p),
        ("hier_r", c_int32 * 4),
    ]


class HSSError(RuntimeError):
    def __init__(self, code, where=""):
        self.code = code
        super().__init__(f"{where}: {status_string(code)} (code {code})")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python sparse_rank_linear_hss_amd/build.py` "
            "(hipcc, gfx950). There is no non-HIP fallback.")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    sig = {
        "hss_version": (ctypes.c_int, []),
        "hss_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "hss_topk_count": (c_int64, [c_int64, c_int64, c_int64, c_int64]),
        "hss_split_workspace_size": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, c_int32, c_int32, P(c_size_t)]),
        "hss_split": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, c_int32, c_int32, c_void_p, c_int64,
                                     c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                     c_void_p, c_size_t, c_void_p]),
        "hss_get_error": (ctypes.c_int, [c_void_p, c_void_p]),
        "hss_set_option": (ctypes.c_int, [ctypes.c_int, c_int32]),
        "hss_get_option": (c_int32, [ctypes.c_int]),
        "hss_apply_workspace_init": (ctypes.c_int, [c_void_p, c_size_t, c_void_p]),
        "hss_apply_noalloc": (ctypes.c_int, [P(HssMatrixStruct), c_int32, c_void_p, c_void_p, c_void_p]),
        "hss_noalloc_scratch_bytes": (c_size_t, []),
        "hss_apply_workspace_size": (ctypes.c_int, [P(HssMatrixStruct), c_int32, P(c_size_t)]),
        "hss_apply": (ctypes.c_int, [P(HssMatrixStruct), c_int32, c_void_p, c_void_p, c_void_p,
                                     c_size_t, c_void_p]),
        "hss_csr_cols_to_u16": (ctypes.c_int, [c_void_p, c_int64, c_int32, c_void_p, c_void_p]),
        "hss_apply_group_workspace_size": (ctypes.c_int, [P(P(HssMatrixStruct)), c_int32, c_int32,
                                                          P(c_size_t)]),
        "hss_apply_group": (ctypes.c_int, [P(P(HssMatrixStruct)), c_int32, c_int32, c_void_p, P(c_void_p),
                                           c_void_p, c_size_t, c_void_p]),
        "hss_rcm_order": (ctypes.c_int, [c_int32, c_void_p, c_void_p, c_void_p]),
        "hss_concentration_workspace_size": (ctypes.c_int, [c_int32, c_int32, P(c_size_t)]),
        "hss_concentration": (ctypes.c_int, [ctypes.c_int, c_int32, c_int32, c_void_p, c_void_p, c_void_p,
                                             c_void_p, c_size_t, c_void_p]),
        "hss_hier_pack": (ctypes.c_int, [ctypes.c_int, c_int32, c_int32, P(c_int32), P(c_void_p), P(c_void_p),
                                         c_void_p, c_void_p, c_void_p, c_void_p]),
        "hss_grad_workspace_size": (ctypes.c_int, [P(HssMatrixStruct), c_int32, P(c_size_t)]),
        "hss_grad": (ctypes.c_int, [P(HssMatrixStruct), c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                    c_void_p, c_size_t, c_void_p]),
        "hss_csr_transpose": (ctypes.c_int, [c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
        "hss_hier_pack_compact": (ctypes.c_int, [ctypes.c_int, c_int32, c_int32, P(c_int32), P(c_void_p),
                                                 P(c_void_p), c_void_p, c_void_p, c_void_p]),
        "hss_csr_permute": (ctypes.c_int, [c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
        "hss_gather_values": (ctypes.c_int, [ctypes.c_int, c_int64, c_void_p, c_void_p, c_void_p, c_void_p]),
        "hss_transpose": (ctypes.c_int, [ctypes.c_int, c_int32, c_int32, c_void_p, c_void_p, c_void_p]),
        "hss_nm24_to_csr": (ctypes.c_int, [c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def status_string(code: int) -> str:
    return lib.hss_status_string(int(code)).decode()


def check(code: int, where: str = "hss"):
    if code != HSS_OK:
        raise HSSError(code, where)
