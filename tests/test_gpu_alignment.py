"""GPU parity with operands that are not 16-byte aligned.

Every kernel checks the alignment its vector loads need and takes an
element-wise path, or another route, otherwise: the 2:4 split's 16-byte
loads and stores, the decode kernel's vector X, Vt, CSR chunk and U piece
loads, the gather SpMM, the sparse matrix cores (16-byte X and values) and the
matrix-core GEMMs.  Each operand here is a view one element past a 16-byte
boundary of a larger device buffer (2 bytes for bf16, 4 for fp32 and the
32-bit index arrays).  Bars as elsewhere: splits bit-exact against the oracle;
applies within tol * sum_j |A_ij X_cj| of the oracle's fp64 result."""
import numpy as np
import pytest

import hss_synth as syn
import oracle as O
from _cases import to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def H():
    import sparse_rank_linear_hss_amd as h
    return h


def _shifted(t):
    """t's values in a new device buffer, starting one element past a 16-byte
    boundary (contiguous, so the library accepts it)."""
    import torch
    flat = torch.empty(t.numel() + 16, dtype=t.dtype, device=t.device)
    base = (-flat.data_ptr() % 16) // t.element_size()  # elements to the next 16-byte boundary
    v = flat[base + 1:base + 1 + t.numel()].view(t.shape)
    v.copy_(t)
    assert v.data_ptr() % 16 != 0 and v.is_contiguous()
    return v


def _raw(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _tdt(dtype):
    import torch
    return torch.float32 if dtype == O.F32 else torch.bfloat16


@pytest.mark.parametrize("dtype", [O.F32, O.BF16])
@pytest.mark.parametrize("fmt,shape", [("csr", (37, 200)), ("csr", (64, 4096)), ("2:4", (33, 128)),
                                       ("2:4", (64, 4096)), ("2:4", (9, 100))])
def test_split_from_unaligned_w(H, dtype, fmt, shape):
    m, n = shape
    W = syn.random_matrix(m, n, dtype, seed=m + n, kind="ties")
    Wd = _shifted(to_dev(W, dtype))
    if fmt == "csr":
        k = O.topk_count(m, n, 5, 100)
        ref = O.split_csr(W, dtype, k)
        sp = H.hss_split(Wd, "csr", k=k, residual=True)
        assert np.array_equal(to_host(sp.row_ptr), ref["row_ptr"])
        assert np.array_equal(to_host(sp.col_idx), ref["col_idx"])
        assert O.bits_equal(to_host(sp.values), ref["values"])
    else:
        ref = O.split_24(W, dtype)
        sp = H.hss_split(Wd, "2:4", residual=True)
        assert O.bits_equal(to_host(sp.nm_values), ref["nm_values"])
        assert np.array_equal(to_host(sp.nm_meta).view(np.uint32), ref["nm_meta"])
    assert O.bits_equal(to_host(sp.residual), ref["residual"])


# (fmt, m, n, r, b): one column (fused decode), a few (decode passes or gather
# / sparse matrix cores), 64 (gather / sparse matrix cores) and 300 (matrix cores)
APPLY = [("csr", 300, 512, 24, 1), ("csr", 2050, 256, 41, 1), ("csr", 300, 512, 24, 4), ("csr", 130, 1024, 16, 16),
         ("csr", 257, 512, 32, 64), ("csr", 300, 640, 128, 300),
         ("2:4", 200, 512, 16, 1), ("2:4", 200, 512, 16, 8), ("2:4", 128, 512, 64, 64), ("2:4", 100, 256, 16, 300)]
WHICH = ["X", "U", "Vt", "S", "all"]


@pytest.mark.parametrize("dtype", [O.F32, O.BF16])
@pytest.mark.parametrize("which", WHICH)
@pytest.mark.parametrize("case", APPLY, ids=[f"{c[0]}-{c[1]}x{c[2]}-r{c[3]}-b{c[4]}" for c in APPLY])
def test_apply_unaligned_operands(H, dtype, which, case):
    fmt, m, n, r, b = case
    seed = 11 * m + n + r + b
    W = syn.random_matrix(m, n, dtype, seed=seed, kind="t3")
    ref = O.split_csr(W, dtype, O.topk_count(m, n, 5, 100)) if fmt == "csr" else O.split_24(W, dtype)
    U, V = syn.factors(m, n, r, dtype, seed)
    X = syn.random_matrix(b, n, dtype, seed=seed + 1, kind="normal", scale=1.0)
    if fmt == "csr":
        S64 = O.dense_from_csr(m, n, ref["row_ptr"], ref["col_idx"], ref["values"], dtype)
    else:
        S64 = O.dense_from_24(m, n, ref["nm_values"], ref["nm_meta"], dtype)
    U64, V64, X64 = O.widen(U, dtype), O.widen(V, dtype), O.widen(X, dtype)
    Yref, N = O.apply_factored(S64, U64, V64, X64), O.normaliser(S64, U64, V64, X64)

    def sh(t, key):
        return _shifted(t) if which in (key, "all") else t

    Ud, Vtd = sh(to_dev(U, dtype), "U"), sh(to_dev(np.ascontiguousarray(V.T), dtype), "Vt")
    if fmt == "csr":
        A = H.HSSMatrix("csr", m, n, _tdt(dtype), U=Ud, Vt=Vtd, row_ptr=sh(_raw(ref["row_ptr"]), "S"),
                        col_idx=sh(_raw(ref["col_idx"]), "S"), values=sh(to_dev(ref["values"], dtype), "S"),
                        nnz=len(ref["col_idx"]))
    else:
        A = H.HSSMatrix("2:4", m, n, _tdt(dtype), U=Ud, Vt=Vtd, nm_values=sh(to_dev(ref["nm_values"], dtype), "S"),
                        nm_meta=sh(_raw(ref["nm_meta"].view(np.int32)), "S"))
    Y = H.hss_apply(A, sh(to_dev(X, dtype), "X"))
    err = O.max_normalised_error(O.widen(to_host(Y), dtype), Yref, N)
    assert err <= O.TOL[dtype], f"max normalised error {err:.3e} > {O.TOL[dtype]}"
