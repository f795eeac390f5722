"""Host-only calls of a sanitizer build of libhss.so (path in HSS_SANITIZED_LIB),
run by tests/test_host_sanitizers.py in a process with the AddressSanitizer
runtime preloaded.  Every call here stays on the host: argument checks that
fail before any device work, the diagnostic switches, the workspace sizing
arithmetic, the Reverse Cuthill-McKee order and the CSR transpose -- the
last two compared with the oracle on random patterns."""
import ctypes
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import oracle as O  # noqa: E402

lib = ctypes.CDLL(os.environ["HSS_SANITIZED_LIB"])
c_i32, c_i64, c_sz, c_vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p


class M(ctypes.Structure):  # struct hss_matrix
    _fields_ = [("fmt", c_i32), ("dtype", c_i32), ("m", c_i32), ("n", c_i32), ("r", c_i32), ("flags", c_i32),
                ("nnz", c_i64), ("row_ptr", c_vp), ("col_idx", c_vp), ("values", c_vp), ("nm_values", c_vp),
                ("nm_meta", c_vp), ("U", c_vp), ("Vt", c_vp), ("dq_codes", c_vp), ("dq_levels", c_vp),
                ("hier_r", c_i32 * 4)]


P = ctypes.POINTER
for name, res, args in [
        ("hss_rcm_order", ctypes.c_int, [c_i32, c_vp, c_vp, c_vp]),
        ("hss_csr_transpose", ctypes.c_int, [c_i32, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp]),
        ("hss_csr_permute", ctypes.c_int, [c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]),
        ("hss_apply", ctypes.c_int, [P(M), c_i32, c_vp, c_vp, c_vp, c_sz, c_vp]),
        ("hss_apply_noalloc", ctypes.c_int, [P(M), c_i32, c_vp, c_vp, c_vp]),
        ("hss_apply_workspace_size", ctypes.c_int, [P(M), c_i32, P(c_sz)]),
        ("hss_apply_group_workspace_size", ctypes.c_int, [P(P(M)), c_i32, c_i32, P(c_sz)]),
        ("hss_grad_workspace_size", ctypes.c_int, [P(M), c_i32, P(c_sz)]),
        ("hss_grad", ctypes.c_int, [P(M), c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]),
        ("hss_apply_workspace_init", ctypes.c_int, [c_vp, c_sz, c_vp]),
        ("hss_split", ctypes.c_int, [c_i32, c_i32, c_i32, c_i32, c_vp, c_i64, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                     c_vp, c_sz, c_vp]),
        ("hss_transpose", ctypes.c_int, [c_i32, c_i32, c_i32, c_vp, c_vp, c_vp]),
        ("hss_gather_values", ctypes.c_int, [c_i32, c_i64, c_vp, c_vp, c_vp, c_vp]),
        ("hss_set_option", ctypes.c_int, [c_i32, c_i32]),
        ("hss_get_option", c_i32, [c_i32]),
        ("hss_status_string", ctypes.c_char_p, [c_i32])]:
    fn = getattr(lib, name)
    fn.restype, fn.argtypes = res, args
lib.hss_topk_count.restype = c_i64
lib.hss_topk_count.argtypes = [c_i64] * 4
FAKE = 0x10000
INV, WS, UNS = 1, 3, 2


def mat(**kw):
    s = M(fmt=0, dtype=1, m=16, n=32, r=4, flags=0, nnz=10, row_ptr=FAKE, col_idx=FAKE, values=FAKE,
          U=FAKE, Vt=FAKE + 4096)
    for k, v in kw.items():
        setattr(s, k, v)
    return s


def expect(code, want, what):
    if code != want:
        raise SystemExit(f"{what}: returned {code}, expected {want}")


# counts, strings, switches
assert lib.hss_version() == 107
for code in range(-1, 8):
    assert lib.hss_status_string(code).startswith(b"HSS")
assert lib.hss_topk_count(1024, 1024, 5, 100) == 52428
assert lib.hss_topk_count(2 ** 40, 2 ** 40, 2 ** 20, 1) == -1 and lib.hss_topk_count(1, 1, 1, 0) == -1
for opt, val, want in [(0, 3, 0), (0, 5, INV), (1, 2, 0), (2, 0, 0), (3, 1, 0), (4, 1, 0), (4, 2, INV), (5, 0, 0), (5, 2, INV), (5, 1, 0), (9, 0, INV),
                       (-1, 0, INV), (0, 0, 0), (1, 0, 0), (2, 4096, 0), (4, 0, 0)]:
    expect(lib.hss_set_option(opt, val), want, f"set_option({opt}, {val})")
assert lib.hss_get_option(99) == -1

# workspace sizing over many shapes and batches (host arithmetic only)
sz = c_sz(0)
for fmt in (0, 1):
    for m, n, r in [(1, 4, 0), (7, 128, 3), (4096, 4096, 409), (11008, 4096, 64), (8192, 8192, 512)]:
        for b in (1, 2, 3, 16, 64, 129, 2048):
            s = mat(fmt=fmt, m=m, n=n, r=r, nnz=min(10, m * n), nm_values=FAKE, nm_meta=FAKE, U=FAKE if r else None,
                    Vt=FAKE if r else None)
            expect(lib.hss_apply_workspace_size(ctypes.byref(s), b, ctypes.byref(sz)), 0, "apply_workspace_size")
            arr = (ctypes.POINTER(M) * 2)(ctypes.pointer(s), ctypes.pointer(s))
            expect(lib.hss_apply_group_workspace_size(arr, 2, b, ctypes.byref(sz)), 0, "group_workspace_size")
            expect(lib.hss_grad_workspace_size(ctypes.byref(s), b, ctypes.byref(sz)), 0, "grad_workspace_size")
        expect(lib.hss_apply_workspace_size(ctypes.byref(mat(m=m, n=n)), 2049, ctypes.byref(sz)), INV, "b > max")
# the compact 2 x 2 block form: flat factors for the batched routes counted in
for m, n, hr in [(2, 2, (1, 0, 0, 1)), (130, 131, (8, 3, 3, 8)), (4096, 4096, (96, 32, 32, 96))]:
    for b in (1, 2, 3, 64, 129, 2048):
        s = mat(m=m, n=n, r=sum(hr), nnz=min(10, m * n), flags=4, hier_r=(c_i32 * 4)(*hr))
        expect(lib.hss_apply_workspace_size(ctypes.byref(s), b, ctypes.byref(sz)), 0, "hier workspace_size")
        assert b == 1 or sz.value >= sum(hr) * (m + n) * 2, (m, n, b, sz.value)

# argument checks that fail before any device work
expect(lib.hss_apply(None, 1, c_vp(FAKE), c_vp(2 * FAKE), c_vp(3 * FAKE), c_sz(1 << 20), None), INV, "apply null")
for kw in [dict(fmt=5), dict(dtype=3), dict(flags=8), dict(m=0), dict(r=-1), dict(U=None), dict(nnz=-1),
           dict(row_ptr=None), dict(m=1 << 20, n=1 << 12)]:
    expect(lib.hss_apply(ctypes.byref(mat(**kw)), 1, c_vp(FAKE), c_vp(1 << 30), c_vp(3 * FAKE), c_sz(1 << 20), None),
           INV, f"apply {kw}")
expect(lib.hss_apply(ctypes.byref(mat()), 1, c_vp(FAKE), c_vp(FAKE + 2), c_vp(3 * FAKE), c_sz(1 << 20), None),
       INV, "apply overlap")
expect(lib.hss_apply(ctypes.byref(mat()), 1, c_vp(FAKE), c_vp(1 << 30), c_vp(3 * FAKE), c_sz(8), None), WS, "apply ws")
expect(lib.hss_apply_noalloc(ctypes.byref(mat(m=8192, n=8192, r=8)), 2048, c_vp(FAKE * 1024),
                             c_vp(FAKE * 1024 + (1 << 26)), None), WS, "noalloc oversized")
expect(lib.hss_apply_workspace_init(None, c_sz(16), None), INV, "init null")
expect(lib.hss_split(0, 1, 8, 8, None, c_i64(3), c_vp(FAKE), c_vp(FAKE), c_vp(FAKE), None, None, None, c_vp(FAKE),
                     c_sz(1 << 20), None), INV, "split null W")
expect(lib.hss_split(1, 1, 8, 6, c_vp(FAKE), c_i64(-1), None, None, None, c_vp(FAKE), c_vp(FAKE), None, c_vp(FAKE),
                     c_sz(1 << 20), None), INV, "split 2:4 n % 4")
expect(lib.hss_grad(ctypes.byref(mat(dtype=0)), 4, c_vp(FAKE * 64), c_vp(FAKE * 96), None, None, None, c_vp(FAKE),
                    c_sz(1 << 24), None), UNS, "grad fp32")
expect(lib.hss_transpose(1, 2_200_000, 2, c_vp(FAKE), c_vp(FAKE * 64), None), INV, "transpose rows")
expect(lib.hss_gather_values(1, c_i64(4), c_vp(FAKE), c_vp(2 * FAKE), c_vp(FAKE + 2), None), INV, "gather overlap")

# Reverse Cuthill-McKee order and CSR transpose: host code, against the oracle
rng = np.random.default_rng(7)
for n, density in [(1, 0.0), (6, 0.0), (40, 0.1), (257, 0.02), (1000, 0.004), (64, 0.6)]:
    mask = rng.random((n, n)) < density
    if n > 5:
        mask[3, 3] = True
    rows, cols = np.nonzero(mask)
    rp = np.zeros(n + 1, dtype=np.int32)
    np.add.at(rp, rows + 1, 1)
    rp = np.cumsum(rp).astype(np.int32)
    ci = cols.astype(np.int32)
    if ci.size > 2:
        ci = np.concatenate([ci[:1], ci]).astype(np.int32)   # a duplicate entry in row 0 or later
        rp[1 + int(rows[0]):] += 1
    perm = np.zeros(n, dtype=np.int32)
    expect(lib.hss_rcm_order(n, rp.ctypes.data, ci.ctypes.data if ci.size else None, perm.ctypes.data), 0, "rcm")
    assert np.array_equal(perm, O.rcm_order(n, rp, ci)), f"rcm differs at n={n}"
    m2 = n
    nnz = int(rp[-1])
    rpt = np.zeros(n + 1, dtype=np.int32)
    cit = np.zeros(max(nnz, 1), dtype=np.int32)
    pt = np.zeros(max(nnz, 1), dtype=np.int32)
    expect(lib.hss_csr_transpose(m2, n, rp.ctypes.data, ci.ctypes.data if nnz else None, rpt.ctypes.data,
                                 cit.ctypes.data, pt.ctypes.data), 0, "csr_transpose")
    ert, ect, ept = O.csr_transpose(m2, n, rp, ci)
    assert np.array_equal(rpt, ert) and np.array_equal(cit[:nnz], ect) and np.array_equal(pt[:nnz], ept)
    # P S P^T of the duplicate-free pattern, for the RCM order and a random one
    keep = np.ones(len(ci), dtype=bool)
    rr = np.repeat(np.arange(n), np.diff(rp))
    if len(ci) > 1:
        keep[1:] = ~((rr[1:] == rr[:-1]) & (ci[1:] == ci[:-1]))
    ci_u = ci[keep].astype(np.int32)
    rp_u = np.concatenate([[0], np.cumsum(np.bincount(rr[keep], minlength=n))]).astype(np.int32) if n else rp
    nnz_u = int(rp_u[-1])
    for pm in (perm, rng.permutation(n).astype(np.int32)):
        prp = np.zeros(n + 1, dtype=np.int32)
        pci = np.zeros(max(nnz_u, 1), dtype=np.int32)
        src = np.zeros(max(nnz_u, 1), dtype=np.int32)
        expect(lib.hss_csr_permute(n, rp_u.ctypes.data, ci_u.ctypes.data if nnz_u else None, pm.ctypes.data,
                                   prp.ctypes.data, pci.ctypes.data, src.ctypes.data), 0, "csr_permute")
        orp, oci, osrc = O.csr_permute(n, rp_u, ci_u, pm)
        assert np.array_equal(prp, orp) and np.array_equal(pci[:nnz_u], oci) and np.array_equal(src[:nnz_u], osrc)
bad_rp = np.array([0, 2, 1], dtype=np.int32)
bad_ci = np.array([0, 5], dtype=np.int32)
perm = np.zeros(2, dtype=np.int32)
expect(lib.hss_rcm_order(2, bad_rp.ctypes.data, bad_ci.ctypes.data, perm.ctypes.data), INV, "rcm decreasing row_ptr")
print("host sanitizer driver ok", flush=True)
