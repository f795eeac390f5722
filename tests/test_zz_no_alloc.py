"""hss_apply_noalloc (the library's own per-GPU scratch in place of a caller
workspace) against hss_apply, through the C ABI.

Calls in a row on one GPU, the second with a smaller input, then the whole
sequence again (the scratch keeps the decode kernel's state from call to
call): every output bit-equal to hss_apply's on the same inputs (the same
kernels and route run) and within the apply bound of the fp64 oracle."""
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


def _raw(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _case(H, fmt, dtype, m, n, r, b, seed):
    import torch
    W = syn.random_matrix(m, n, dtype, seed=seed, kind="t3")
    ref = O.split_csr(W, dtype, O.topk_count(m, n, 5, 100)) if fmt == "csr" else O.split_24(W, dtype)
    U, V = syn.factors(m, n, r, dtype, seed)
    X = syn.random_matrix(b, n, dtype, seed=seed + 1, kind="normal", scale=1.0)
    td = torch.float32 if dtype == O.F32 else torch.bfloat16
    Ud, Vtd = to_dev(U, dtype), to_dev(np.ascontiguousarray(V.T), dtype)
    if fmt == "csr":
        A = H.HSSMatrix("csr", m, n, td, U=Ud, Vt=Vtd, row_ptr=_raw(ref["row_ptr"]), col_idx=_raw(ref["col_idx"]),
                        values=to_dev(ref["values"], dtype), nnz=len(ref["col_idx"]))
        S64 = O.dense_from_csr(m, n, ref["row_ptr"], ref["col_idx"], ref["values"], dtype)
    else:
        A = H.HSSMatrix("2:4", m, n, td, U=Ud, Vt=Vtd, nm_values=to_dev(ref["nm_values"], dtype),
                        nm_meta=_raw(ref["nm_meta"].view(np.int32)))
        S64 = O.dense_from_24(m, n, ref["nm_values"], ref["nm_meta"], dtype)
    U64, V64, X64 = O.widen(U, dtype), O.widen(V, dtype), O.widen(X, dtype)
    return A, to_dev(X, dtype), O.apply_factored(S64, U64, V64, X64), O.normaliser(S64, U64, V64, X64), dtype


CASES = [
    # (fmt, dtype, m, n, r, b): the first is the largest; each route keeps its own data in the scratch
    ("csr", O.BF16, 2048, 1024, 64, 16),    # gather SpMM: T^T, X^T in the scratch
    ("csr", O.BF16, 1030, 512, 41, 1),      # fused decode, T rows made in the row blocks (epoch, T words)
    ("2:4", O.BF16, 300, 512, 24, 8),       # sparse matrix cores: T in the scratch
    ("csr", O.F32, 200, 256, 16, 1),        # fused decode, separate T producer blocks
    ("csr", O.BF16, 96, 64, 40, 300),       # matrix cores (CSR densified into the scratch)
]


def test_noalloc_equals_apply_in_sequence(H):
    import torch
    assert H._lib.lib.hss_noalloc_scratch_bytes() == 16 << 20
    cases = [_case(H, *c, seed=101 + 7 * i) for i, c in enumerate(CASES)]
    for rep in range(2):
        for i, (A, Xd, Yref, N, dtype) in enumerate(cases):
            td = torch.float32 if dtype == O.F32 else torch.bfloat16
            Y_na = torch.empty((Xd.shape[0], A.m), dtype=td, device="cuda")
            H.hss_apply_noalloc(A, Xd, Y_na)
            Y_ws = H.hss_apply(A, Xd)
            got = to_host(Y_na)
            assert O.bits_equal(got, to_host(Y_ws)), (rep, i)
            err = O.max_normalised_error(O.widen(got, dtype), Yref, N)
            assert err <= O.TOL[dtype], (rep, i, err)


def test_noalloc_refuses_a_route_larger_than_its_scratch(H):
    """8192 x 8192 CSR at b = 2048 runs densified on the matrix cores (m n 2
    bytes of workspace): refused on the host, nothing launched."""
    import ctypes
    import torch
    m = n = 8192
    A = H.HSSMatrix("csr", m, n, torch.bfloat16, U=torch.zeros((m, 8), dtype=torch.bfloat16, device="cuda"),
                    Vt=torch.zeros((8, n), dtype=torch.bfloat16, device="cuda"),
                    row_ptr=torch.zeros(m + 1, dtype=torch.int32, device="cuda"),
                    col_idx=torch.zeros(1, dtype=torch.int32, device="cuda"),
                    values=torch.zeros(1, dtype=torch.bfloat16, device="cuda"), nnz=1)
    X = torch.zeros((2048, n), dtype=torch.bfloat16, device="cuda")
    Y = torch.empty((2048, m), dtype=torch.bfloat16, device="cuda")
    code = H._lib.lib.hss_apply_noalloc(ctypes.byref(A.struct), 2048, X.data_ptr(), Y.data_ptr(),
                                        torch.cuda.current_stream().cuda_stream)
    assert code == H._lib.HSS_ERR_WORKSPACE
