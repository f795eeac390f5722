"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects bad arguments on the host before any device work."""
import ctypes
import os
import re

import pytest

from conftest import ROOT

H = os.path.join(ROOT, "include", "hss.h")


def _declared():
    text = open(H).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hss_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def hl():
    import sparse_rank_linear_hss_amd as h
    return h


def test_header_declares_the_boundary():
    names = _declared()
    for must in ("hss_split", "hss_apply", "hss_split_workspace_size", "hss_apply_workspace_size",
                 "hss_apply_group", "hss_apply_group_workspace_size",
                 "hss_get_error", "hss_topk_count", "hss_status_string", "hss_version",
                 "hss_rcm_order", "hss_concentration", "hss_concentration_workspace_size", "hss_hier_pack",
                 "hss_grad", "hss_grad_workspace_size", "hss_csr_transpose", "hss_gather_values", "hss_transpose",
                 "hss_nm24_to_csr", "hss_set_option", "hss_get_option", "hss_apply_workspace_init"):
        assert must in names


def test_library_exports_every_declared_symbol(hl):
    raw = ctypes.CDLL(hl.LIB_PATH)
    for name in _declared():
        assert hasattr(raw, name), name


def test_version_and_strings(hl):
    assert hl.hss_version() == 107
    for code in range(6):
        assert hl.status_string(code).startswith("HSS_")


def test_topk_count_matches_worked_example(hl):
    lib = hl._lib.lib
    assert lib.hss_topk_count(1024, 1024, 5, 100) == 52428
    assert lib.hss_topk_count(8192, 8192, 3, 100) == 2013265
    assert lib.hss_topk_count(-1, 4, 1, 2) == -1
    assert lib.hss_topk_count(4, 4, 1, 0) == -1
    assert lib.hss_topk_count(2**40, 2**40, 2**20, 1) == -1     # int64 overflow


FAKE = 0x10000  # never dereferenced: every call below fails validation first


def _split(lib, fmt=0, dt=1, m=8, n=8, W=FAKE, k=3, rp=FAKE, ci=FAKE, val=FAKE, nmv=None, nmm=None,
           res=None, ws=FAKE, wsb=1 << 20):
    return lib.hss_split(fmt, dt, m, n, W, k, rp, ci, val, nmv, nmm, res, ws, wsb, None)


def test_split_rejects_bad_arguments(hl):
    lib = hl._lib.lib
    INV, WS = hl._lib.HSS_ERR_INVALID_ARG, hl._lib.HSS_ERR_WORKSPACE
    assert _split(lib, fmt=7) == INV
    assert _split(lib, dt=9) == INV
    assert _split(lib, m=0) == INV
    assert _split(lib, n=-1) == INV
    assert _split(lib, m=65536, n=32768) == INV                  # m*n >= 2^31
    assert _split(lib, W=None) == INV
    assert _split(lib, k=-1) == INV
    assert _split(lib, k=65) == INV                               # k > m*n
    assert _split(lib, rp=None) == INV
    assert _split(lib, ci=None) == INV
    assert _split(lib, nmv=FAKE) == INV                           # 2:4 output given for CSR
    assert _split(lib, res=FAKE) == INV                           # residual aliases W
    assert _split(lib, ws=None) == WS
    assert _split(lib, wsb=16) == WS
    # 2:4
    assert _split(lib, fmt=1, rp=None, ci=None, val=None, nmv=FAKE, nmm=FAKE, n=6, k=-1) == INV
    assert _split(lib, fmt=1, rp=None, ci=None, val=None, nmv=FAKE, nmm=FAKE, k=5) == INV
    assert _split(lib, fmt=1, rp=FAKE, ci=None, val=None, nmv=FAKE, nmm=FAKE, k=-1) == INV
    assert _split(lib, fmt=1, rp=None, ci=None, val=None, nmv=None, nmm=FAKE, k=-1) == INV
    assert _split(lib, fmt=1, rp=None, ci=None, val=None, nmv=FAKE, nmm=FAKE, k=-1, wsb=8) == WS


def test_split_workspace_size(hl):
    assert hl.hss_split_workspace_size("csr", 1, 100, 7) >= 4 * 2 * 100
    assert hl.hss_split_workspace_size("2:4", 1, 100, 8) > 0
    with pytest.raises(hl.HSSError):
        hl.hss_split_workspace_size("csr", 1, 0, 7)


def _matrix(hl, **kw):
    s = hl._lib.HssMatrixStruct()
    s.fmt, s.dtype, s.m, s.n, s.r, s.flags, s.nnz = 0, 1, 16, 32, 4, 0, 10
    s.row_ptr = s.col_idx = s.values = FAKE
    s.U, s.Vt = FAKE, FAKE + 4096
    for k, v in kw.items():
        setattr(s, k, v)
    return s


def _apply(hl, s, b=1, X=FAKE + 8192, Y=FAKE + 65536, ws=FAKE * 16, wsb=1 << 20):
    return hl._lib.lib.hss_apply(ctypes.byref(s), b, X, Y, ws, wsb, None)


def test_apply_rejects_bad_arguments(hl):
    INV, WS = hl._lib.HSS_ERR_INVALID_ARG, hl._lib.HSS_ERR_WORKSPACE
    lib = hl._lib.lib
    assert lib.hss_apply(None, 1, FAKE, FAKE * 2, FAKE * 3, 1 << 20, None) == INV
    assert _apply(hl, _matrix(hl, fmt=5)) == INV
    assert _apply(hl, _matrix(hl, dtype=3)) == INV
    assert _apply(hl, _matrix(hl, flags=8)) == INV                  # unknown flag
    # compact 2 x 2 block term (HSS_HIER2): CSR only, ranks >= 0 summing to r, equal per row half
    H4 = (ctypes.c_int32 * 4)
    assert _apply(hl, _matrix(hl, flags=4, hier_r=H4(1, 1, 1, 1)), wsb=0) == WS  # valid: only the workspace short
    assert _apply(hl, _matrix(hl, flags=4, hier_r=H4(1, 1, 1, 0))) == INV          # sum != r
    assert _apply(hl, _matrix(hl, flags=4, hier_r=H4(2, 1, 0, 1))) == INV          # 3 != 1 per row half
    assert _apply(hl, _matrix(hl, flags=4, hier_r=H4(3, -1, 1, 1))) == INV         # negative rank
    assert _apply(hl, _matrix(hl, flags=4, hier_r=H4(1, 1, 1, 1), fmt=1, nm_values=FAKE, nm_meta=FAKE)) == INV
    assert _apply(hl, _matrix(hl, flags=6, hier_r=H4(0, 0, 0, 0), r=0, U=None, Vt=None, dq_codes=FAKE,
                              dq_levels=FAKE)) == INV                   # not with the dense part
    assert _apply(hl, _matrix(hl, flags=4, hier_r=H4(1, 1, 1, 1), m=1)) == INV     # both halves need rows
    hsz = ctypes.c_size_t(0)
    for b in (1, 2, 8, 64, 300):
        assert lib.hss_apply_workspace_size(ctypes.byref(_matrix(hl, flags=4, hier_r=H4(1, 1, 1, 1))), b,
                                            ctypes.byref(hsz)) == 0 and hsz.value > 0
    g_ok = ctypes.c_size_t(0)
    assert lib.hss_grad_workspace_size(ctypes.byref(_matrix(hl, flags=4, hier_r=H4(1, 1, 1, 1))), 4,
                                       ctypes.byref(g_ok)) == hl._lib.HSS_ERR_UNSUPPORTED
    # dense-and-sparse (HSS_DQ4): arrays required, CSR only, n even, no low-rank term
    assert _apply(hl, _matrix(hl, flags=2, r=0, U=None, Vt=None)) == INV
    assert _apply(hl, _matrix(hl, flags=2, r=0, U=None, Vt=None, dq_codes=FAKE)) == INV
    assert _apply(hl, _matrix(hl, flags=2, r=0, U=None, Vt=None, dq_codes=FAKE, dq_levels=FAKE, fmt=1,
                              nm_values=FAKE, nm_meta=FAKE)) == INV
    assert _apply(hl, _matrix(hl, flags=2, r=0, U=None, Vt=None, dq_codes=FAKE, dq_levels=FAKE, n=31)) == INV
    assert _apply(hl, _matrix(hl, flags=2, dq_codes=FAKE, dq_levels=FAKE)) == hl._lib.HSS_ERR_UNSUPPORTED
    dq_sz = ctypes.c_size_t(1)
    assert lib.hss_apply_workspace_size(ctypes.byref(_matrix(hl, flags=2, r=0, U=None, Vt=None, dq_codes=FAKE,
                                                             dq_levels=FAKE)), 7, ctypes.byref(dq_sz)) == 0
    assert dq_sz.value == 0                                         # the dense-and-sparse kernel needs none
    assert _apply(hl, _matrix(hl, fmt=1, flags=1, nm_values=FAKE, nm_meta=FAKE)) == INV  # COL16 on 2:4
    assert _apply(hl, _matrix(hl, flags=1, n=65537)) == INV         # COL16 needs n <= 65536
    assert _apply(hl, _matrix(hl, m=0)) == INV
    assert _apply(hl, _matrix(hl, r=-1)) == INV
    assert _apply(hl, _matrix(hl), b=0) == INV
    assert _apply(hl, _matrix(hl), b=hl.HSS_MAX_BATCH + 1) == INV   # batch beyond the contract
    assert _apply(hl, _matrix(hl, m=1 << 20), b=2048) == INV      # b*m >= 2^31
    assert _apply(hl, _matrix(hl, U=None)) == INV
    assert _apply(hl, _matrix(hl, Vt=None)) == INV
    assert _apply(hl, _matrix(hl, nnz=-2)) == INV
    assert _apply(hl, _matrix(hl, row_ptr=None)) == INV
    assert _apply(hl, _matrix(hl, values=None)) == INV
    assert _apply(hl, _matrix(hl, fmt=1, n=30, nm_values=FAKE, nm_meta=FAKE)) == INV
    assert _apply(hl, _matrix(hl, fmt=1, nm_values=None, nm_meta=FAKE)) == INV
    assert _apply(hl, _matrix(hl), X=None) == INV
    assert _apply(hl, _matrix(hl), X=FAKE, Y=FAKE + 2) == INV      # X overlaps Y
    assert _apply(hl, _matrix(hl), ws=None) == WS
    assert _apply(hl, _matrix(hl), wsb=8) == WS
    # r = 0 needs no factors
    sz = ctypes.c_size_t(0)
    assert lib.hss_apply_workspace_size(ctypes.byref(_matrix(hl, r=0, U=None, Vt=None)), 1,
                                        ctypes.byref(sz)) == 0
    assert sz.value >= 256


def test_batch_range_is_1_to_2048(hl):
    """b in [1, HSS_MAX_BATCH]: the sizing calls agree with the apply."""
    INV = hl._lib.HSS_ERR_INVALID_ARG
    lib = hl._lib.lib
    sz = ctypes.c_size_t(0)
    assert hl.HSS_MAX_BATCH == 2048
    assert lib.hss_apply_workspace_size(ctypes.byref(_matrix(hl)), 2048, ctypes.byref(sz)) == 0
    assert lib.hss_apply_workspace_size(ctypes.byref(_matrix(hl)), 2049, ctypes.byref(sz)) == INV
    assert lib.hss_apply_workspace_size(ctypes.byref(_matrix(hl)), 0, ctypes.byref(sz)) == INV
    arr = (ctypes.POINTER(hl._lib.HssMatrixStruct) * 1)(ctypes.pointer(_matrix(hl)))
    assert lib.hss_apply_group_workspace_size(arr, 1, 2049, ctypes.byref(sz)) == INV
    assert lib.hss_grad_workspace_size(ctypes.byref(_matrix(hl)), 2049, ctypes.byref(sz)) == INV


def test_options_set_get_and_reject(hl):
    """The diagnostic switches: each round-trips, bad ones are refused, and
    the env-derived defaults are what the header states (no env set here)."""
    INV = hl._lib.HSS_ERR_INVALID_ARG
    lib = hl._lib.lib
    L = hl._lib
    defaults = {L.HSS_OPT_BATCH_ROUTE: 0, L.HSS_OPT_GRAD_DS_ROUTE: 0, L.HSS_OPT_DECODE_SPIN: 4096,
                L.HSS_OPT_DECODE_MERGED: 1, L.HSS_OPT_DECODE_FORCE_LOCAL: 0, L.HSS_OPT_DECODE_WAVE_PRODUCERS: 1,
                L.HSS_OPT_DECODE_RPW: 0}
    for k in ("HSS_CSR_BATCH_ROUTE", "HSS_GRAD_DS_ROUTE", "HSS_DECODE_SPIN", "HSS_DECODE_MERGED",
              "HSS_DECODE_WAVE_PRODUCERS", "HSS_DECODE_RPW"):
        assert k not in os.environ
    for opt, v in defaults.items():
        assert lib.hss_get_option(opt) == v
    assert lib.hss_get_option(7) == -1 and lib.hss_get_option(-1) == -1
    for opt, bad in ((L.HSS_OPT_BATCH_ROUTE, 5), (L.HSS_OPT_GRAD_DS_ROUTE, 3), (L.HSS_OPT_DECODE_SPIN, -1),
                     (L.HSS_OPT_DECODE_MERGED, 2), (L.HSS_OPT_DECODE_FORCE_LOCAL, -1),
                     (L.HSS_OPT_DECODE_WAVE_PRODUCERS, 2), (L.HSS_OPT_DECODE_RPW, 3),
                     (L.HSS_OPT_DECODE_RPW, 8), (7, 0)):
        assert lib.hss_set_option(opt, bad) == INV
    with hl.option("batch_route", "densify"):
        assert hl.hss_get_option("batch_route") == 3
        with hl.option("batch_route", "smfmac"):
            assert hl.hss_get_option("batch_route") == 4
        assert hl.hss_get_option("batch_route") == 3
    assert hl.hss_get_option("batch_route") == 0
    with hl.option("decode_spin", 7), hl.option("grad_ds_route", "dense"):
        assert lib.hss_get_option(L.HSS_OPT_DECODE_SPIN) == 7 and hl.hss_get_option("grad_ds_route") == 2
    for opt, v in defaults.items():
        assert lib.hss_get_option(opt) == v


def test_options_read_from_the_environment_once(hl):
    """A fresh process takes the switches' first values from the environment."""
    import subprocess
    import sys
    code = ("import sparse_rank_linear_hss_amd as h, os;"
            "print(h.hss_get_option('batch_route'), h.hss_get_option('grad_ds_route'),"
            " h.hss_get_option('decode_spin'), h.hss_get_option('decode_merged'));"
            "os.environ['HSS_DECODE_SPIN'] = '5'; print(h.hss_get_option('decode_spin'))")
    env = dict(os.environ, HSS_CSR_BATCH_ROUTE="spmm", HSS_GRAD_DS_ROUTE="dense", HSS_DECODE_SPIN="12",
               HSS_DECODE_MERGED="0")
    out = subprocess.run([sys.executable, "-c", code], env=env, cwd=ROOT, capture_output=True, text=True, check=True)
    assert out.stdout.split() == ["2", "2", "12", "0", "12"]


def test_apply_noalloc_checks_on_the_host(hl):
    """The no-allocation apply refuses bad arguments, and routes whose
    workspace exceeds its scratch, before any device work."""
    INV, WS = hl._lib.HSS_ERR_INVALID_ARG, hl._lib.HSS_ERR_WORKSPACE
    lib = hl._lib.lib
    assert lib.hss_noalloc_scratch_bytes() == 16 << 20
    assert lib.hss_apply_noalloc(None, 1, FAKE, FAKE * 2, None) == INV
    s = _matrix(hl)
    assert lib.hss_apply_noalloc(ctypes.byref(s), 0, FAKE, FAKE * 2, None) == INV
    assert lib.hss_apply_noalloc(ctypes.byref(s), 1, None, FAKE * 2, None) == INV
    assert lib.hss_apply_noalloc(ctypes.byref(s), 1, FAKE, FAKE + 2, None) == INV      # X overlaps Y
    big = _matrix(hl, m=8192, n=8192, r=8)                                               # densified at b = 2048
    assert lib.hss_apply_noalloc(ctypes.byref(big), 2048, FAKE * 1024, FAKE * 1024 + (1 << 26), None) == WS


def test_workspace_init_rejects_bad_arguments(hl):
    lib = hl._lib.lib
    assert lib.hss_apply_workspace_init(None, 16, None) == hl._lib.HSS_ERR_INVALID_ARG
    assert lib.hss_apply_workspace_init(None, 0, None) == 0           # nothing to do


def _group(hl, mats, b=1, X=FAKE + 8192, Ys=None, ws=FAKE * 16, wsb=1 << 20):
    lib = hl._lib.lib
    arr = (ctypes.POINTER(hl._lib.HssMatrixStruct) * max(1, len(mats)))(*[ctypes.pointer(m) for m in mats])
    if Ys is None:
        Ys = [FAKE * 32 + i * 65536 for i in range(len(mats))]
    yp = (ctypes.c_void_p * max(1, len(Ys)))(*Ys)
    return lib.hss_apply_group(arr, len(mats), b, X, yp, ws, wsb, None)


def test_apply_group_rejects_bad_arguments(hl):
    INV, WS = hl._lib.HSS_ERR_INVALID_ARG, hl._lib.HSS_ERR_WORKSPACE
    lib = hl._lib.lib
    a, b2 = _matrix(hl), _matrix(hl, m=40)
    assert lib.hss_apply_group(None, 1, 1, FAKE, None, FAKE, 1 << 20, None) == INV
    assert _group(hl, []) == INV                                        # G = 0
    assert _group(hl, [a] * 5) == INV                                   # G > HSS_MAX_GROUP
    assert _group(hl, [a, _matrix(hl, n=64)]) == INV                    # n differs
    assert _group(hl, [a, _matrix(hl, dtype=0)]) == INV                 # dtype differs
    assert _group(hl, [a, _matrix(hl, fmt=1, nm_values=FAKE, nm_meta=FAKE)]) == INV  # format differs
    assert _group(hl, [a, _matrix(hl, r=-1)]) == INV                    # an invalid member
    assert _group(hl, [a, b2], X=None) == INV
    assert _group(hl, [a, b2], Ys=[FAKE * 32, None]) == INV
    assert _group(hl, [a, b2], Ys=[FAKE * 32, FAKE * 32 + 8]) == INV    # outputs overlap
    assert _group(hl, [a, b2], X=FAKE * 32 + 4) == INV                  # X overlaps an output
    assert _group(hl, [a, b2], ws=None) == WS
    assert _group(hl, [a, b2], wsb=8) == WS
    sz1, sz2 = ctypes.c_size_t(0), ctypes.c_size_t(0)
    arr = (ctypes.POINTER(hl._lib.HssMatrixStruct) * 2)(ctypes.pointer(a), ctypes.pointer(b2))
    assert lib.hss_apply_group_workspace_size(arr, 2, 1, ctypes.byref(sz2)) == 0
    assert lib.hss_apply_workspace_size(ctypes.byref(a), 1, ctypes.byref(sz1)) == 0
    assert sz2.value >= sz1.value


def test_hierarchical_entry_points_reject_bad_arguments(hl):
    INV, WS = hl._lib.HSS_ERR_INVALID_ARG, hl._lib.HSS_ERR_WORKSPACE
    lib = hl._lib.lib
    sz = ctypes.c_size_t(0)
    assert lib.hss_concentration_workspace_size(16, 24, ctypes.byref(sz)) == 0 and sz.value >= 4 * 24
    assert lib.hss_concentration_workspace_size(0, 24, ctypes.byref(sz)) == INV
    big = 1 << 22

    def conc(dt=1, m=16, n=16, W=FAKE, perm=None, out=FAKE * 2, ws=FAKE * 3, wsb=big):
        return lib.hss_concentration(dt, m, n, W, perm, out, ws, wsb, None)
    assert conc(dt=7) == INV
    assert conc(m=0) == INV
    assert conc(W=None) == INV
    assert conc(out=None) == INV
    assert conc(n=24, perm=FAKE * 4) == INV                    # a permutation needs a square matrix
    assert conc(ws=None) == WS
    assert conc(wsb=64) == WS

    def pack(dt=1, m=16, n=16, r=(2, 1, 1, 2), U=(FAKE,) * 4, Vt=(FAKE,) * 4, perm=None, Uc=FAKE * 5, Vc=FAKE * 6):
        ra = (ctypes.c_int32 * 4)(*r)
        ua = (ctypes.c_void_p * 4)(*U)
        va = (ctypes.c_void_p * 4)(*Vt)
        return lib.hss_hier_pack(dt, m, n, ra, ua, va, perm, Uc, Vc, None)
    assert pack(dt=5) == INV
    assert pack(m=1) == INV
    assert pack(r=(9, 0, 0, 0)) == INV                         # rank above the block's smaller side
    assert pack(r=(-1, 0, 0, 0)) == INV
    assert pack(U=(None, FAKE, FAKE, FAKE)) == INV             # block 0 has rank 2 but no factor
    assert pack(Uc=None) == INV
    assert pack(n=20, perm=FAKE) == INV
    assert pack(r=(0, 0, 0, 0), U=(None,) * 4, Vt=(None,) * 4, Uc=None, Vc=None) == 0   # nothing to pack


def test_backward_entry_points_reject_bad_arguments(hl):
    INV, WS, UNS = hl._lib.HSS_ERR_INVALID_ARG, hl._lib.HSS_ERR_WORKSPACE, hl._lib.HSS_ERR_UNSUPPORTED
    lib = hl._lib.lib

    def grad(s, b=4, X=FAKE * 64, G=FAKE * 96, dS=FAKE * 128, dU=FAKE * 160, dVt=FAKE * 192, ws=FAKE * 224,
             wsb=1 << 24):
        return lib.hss_grad(ctypes.byref(s), b, X, G, dS, dU, dVt, ws, wsb, None)
    assert grad(_matrix(hl, dtype=0)) == UNS                            # fp32 layer
    assert grad(_matrix(hl, flags=2, r=0, U=None, Vt=None, dq_codes=FAKE, dq_levels=FAKE)) == UNS  # D + S
    assert grad(_matrix(hl, m=0)) == INV
    assert grad(_matrix(hl), b=0) == INV
    assert grad(_matrix(hl), X=None) == INV
    assert grad(_matrix(hl), G=None) == INV
    assert grad(_matrix(hl), dU=FAKE * 64 + 8) == INV                   # output overlaps X
    assert grad(_matrix(hl), dVt=FAKE * 128 + 4) == INV                 # two outputs overlap
    assert grad(_matrix(hl), ws=None) == WS
    assert grad(_matrix(hl), wsb=64) == WS
    sz = ctypes.c_size_t(0)
    assert lib.hss_grad_workspace_size(ctypes.byref(_matrix(hl)), 4, ctypes.byref(sz)) == 0 and sz.value > 0
    assert lib.hss_gather_values(1, -1, FAKE, FAKE * 2, FAKE * 3, None) == INV
    assert lib.hss_gather_values(7, 4, FAKE, FAKE * 2, FAKE * 3, None) == INV
    assert lib.hss_gather_values(1, 4, FAKE, None, FAKE * 3, None) == INV
    assert lib.hss_gather_values(1, 4, FAKE, FAKE * 2, FAKE + 2, None) == INV   # overlapping values
    assert lib.hss_gather_values(1, 0, None, None, None, None) == 0             # nothing to do
    assert lib.hss_transpose(1, 0, 4, FAKE, FAKE * 2, None) == INV
    assert lib.hss_transpose(9, 4, 4, FAKE, FAKE * 2, None) == INV
    assert lib.hss_transpose(1, 4, 4, FAKE, FAKE + 8, None) == INV             # overlapping
    assert lib.hss_transpose(1, 2_200_000, 2, FAKE, FAKE * 64, None) == INV    # too many rows for the grid
    assert lib.hss_nm24_to_csr(0, 8, FAKE, FAKE * 2, FAKE * 3, None) == INV
    assert lib.hss_nm24_to_csr(4, 6, FAKE, FAKE * 2, FAKE * 3, None) == INV     # n % 4 != 0
    assert lib.hss_nm24_to_csr(4, 8, None, FAKE * 2, FAKE * 3, None) == INV
    assert lib.hss_nm24_to_csr(4, 8, FAKE, FAKE * 2, FAKE * 2 + 8, None) == INV  # overlapping outputs
