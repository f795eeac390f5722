"""GPU parity of the dense-and-sparse apply (HSS_DQ4) against the CPU oracle.

Y = X (S + D)^T with S the 0.5 % outliers (CSR, the oracle's own split) and D
the residual quantised to 4-bit per-row levels by the oracle.  Bar: every
output within tol * N[c, i], N = sum_j |A_ij X_cj| with A = S + D rebuilt in
fp64 from the stored codes and levels; tol = 1e-5 for fp32, 8e-3 for bf16
inputs with fp32 accumulation and bf16 output."""
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


def _tdt(dtype):
    import torch
    return torch.float32 if dtype == O.F32 else torch.bfloat16


def _raw(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _dq_matrix(H, dtype, m, n, d, col16=False):
    k = len(d["col_idx"])
    A = H.HSSMatrix("csr", m, n, _tdt(dtype), row_ptr=_raw(d["row_ptr"]),
                    col_idx=_raw(d["col_idx"]) if k else None,
                    values=to_dev(d["values"], dtype) if k else None, nnz=k,
                    dq_codes=_raw(d["codes_packed"]), dq_levels=to_dev(d["lut"], dtype))
    return A.with_col16() if col16 else A


def _reference(dtype, m, n, d, X):
    S = O.dense_from_csr(m, n, d["row_ptr"], d["col_idx"], d["values"], dtype)
    A = S + O.dense_from_codes(d["codes"], d["lut"], dtype)
    X64 = O.widen(X, dtype)
    zero = np.zeros((m, 0)), np.zeros((n, 0))
    return O.apply_factored(A, zero[0], zero[1], X64), O.normaliser(A, zero[0], zero[1], X64)


def _check(Y_dev, dtype, Yref, N):
    err = O.max_normalised_error(O.widen(to_host(Y_dev), dtype), Yref, N)
    assert err <= O.TOL[dtype], f"max normalised error {err:.3e} > {O.TOL[dtype]}"


CASES = [
    # (m, n, b, k): n % 32 == 0 (16-byte code chunks) and not (bytes one at a time), n % 8 != 0
    # (one column per pass), several passes of 8 columns, ragged rows at 1 and 2 rows per wave
    # (m >= 2048: one column, several), no outliers
    (64, 64, 1, None), (130, 96, 3, None), (257, 512, 8, None), (300, 1024, 17, None),
    (2050, 256, 1, None), (2051, 256, 3, None), (40, 38, 2, None), (96, 4096, 1, None), (33, 128, 5, 0),
]


@pytest.mark.parametrize("dtype", [O.F32, O.BF16])
@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}x{c[1]}-b{c[2]}-k{c[3]}" for c in CASES])
def test_dq_apply(H, dtype, case):
    m, n, b, k = case
    seed = m * 5 + n + b
    W = syn.random_matrix(m, n, dtype, seed=seed, kind="t3")
    d = O.split_dense_sparse(W, dtype, k=k)
    X = syn.random_matrix(b, n, dtype, seed=seed + 1, kind="normal", scale=1.0)
    Yref, N = _reference(dtype, m, n, d, X)
    A = _dq_matrix(H, dtype, m, n, d)
    assert H.hss_apply_workspace_size(A, b) == 0
    Xd = to_dev(X, dtype)
    Y1 = H.hss_apply(A, Xd)
    _check(Y1, dtype, Yref, N)
    Y2 = H.hss_apply(A, Xd)
    assert O.bits_equal(to_host(Y1), to_host(Y2))                   # deterministic


def test_dq_apply_col16_bitwise_equal(H):
    dtype, m, n, b = O.BF16, 200, 256, 4
    W = syn.random_matrix(m, n, dtype, seed=9, kind="t3")
    d = O.split_dense_sparse(W, dtype)
    X = to_dev(syn.random_matrix(b, n, dtype, seed=10, kind="normal", scale=1.0), dtype)
    Y32 = to_host(H.hss_apply(_dq_matrix(H, dtype, m, n, d), X))
    Y16 = to_host(H.hss_apply(_dq_matrix(H, dtype, m, n, d, col16=True), X))
    assert O.bits_equal(Y32, Y16)


def test_dq_apply_group_equals_single(H):
    dtype, n, b = O.BF16, 128, 2
    mats, ds = [], []
    for i, m in enumerate((100, 64, 130)):
        W = syn.random_matrix(m, n, dtype, seed=20 + i, kind="t3")
        d = O.split_dense_sparse(W, dtype)
        mats.append(_dq_matrix(H, dtype, m, n, d))
        ds.append((m, d))
    X = syn.random_matrix(b, n, dtype, seed=30, kind="normal", scale=1.0)
    Xd = to_dev(X, dtype)
    Ys = H.hss_apply_group(mats, Xd)
    for (m, d), A, Y in zip(ds, mats, Ys):
        assert O.bits_equal(to_host(Y), to_host(H.hss_apply(A, Xd)))
        _check(Y, dtype, *_reference(dtype, m, n, d, X))


def test_dq_apply_full_size_sampled(H):
    """4096 x 4096 bf16 with 0.5 % outliers (the oracle's split of the 4096^2
    weight) and stand-in 4-bit codes and levels; rows checked one by one."""
    import torch
    cfg = syn.WORKLOADS["csr4096"]
    m, n = cfg.shapes[0]
    W = syn.weight(cfg)
    s = O.split_csr(W, O.BF16, O.outlier_count(m, n))
    codes, lut = syn.quantised_standin(m, n, O.BF16, cfg.seed)
    A = H.HSSMatrix("csr", m, n, torch.bfloat16, row_ptr=_raw(s["row_ptr"]), col_idx=_raw(s["col_idx"]),
                    values=to_dev(s["values"], O.BF16), nnz=len(s["col_idx"]),
                    dq_codes=_raw(codes), dq_levels=to_dev(lut, O.BF16))
    for b in (1, 8):
        X = syn.activations(cfg, b, 0, 0)
        Y = O.widen(to_host(H.hss_apply(A, to_dev(X, O.BF16))), O.BF16)
        rows = np.sort(np.random.default_rng(b).choice(m, size=256, replace=False))
        S_rows = O.csr_rows_dense(rows, n, s["row_ptr"], s["col_idx"], s["values"], O.BF16)
        D_rows = O.dense_from_codes(O.unpack_nibbles(codes[rows], n), lut[rows], O.BF16)
        A_rows = S_rows + D_rows
        X64 = O.widen(X, O.BF16)
        Yref, N = X64 @ A_rows.T, np.abs(X64) @ np.abs(A_rows).T
        err = O.max_normalised_error(Y[:, rows], Yref, N)
        assert err <= O.TOL[O.BF16], f"b={b}: max normalised error {err:.3e}"
