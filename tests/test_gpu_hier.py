"""GPU side of the hierarchical variant against the CPU oracle: the
concentration ratio, the packing of 2 x 2 block factors, and the apply of a
layer S + (block low-rank term) built from the library's RCM order."""
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


@pytest.mark.parametrize("dtype", [O.F32, O.BF16])
@pytest.mark.parametrize("shape,permuted", [((64, 64), False), ((97, 131), False), ((150, 150), True),
                                            ((1, 5), False)])
def test_concentration_matches_oracle(H, dtype, shape, permuted):
    m, n = shape
    W = syn.random_matrix(m, n, dtype, seed=m + n, kind="t3")
    perm = np.random.default_rng(3).permutation(n).astype(np.int32) if permuted else None
    out = H.hss_concentration(to_dev(W, dtype), None if perm is None else _raw(perm)).cpu().numpy()
    a = np.abs(O.widen(W, dtype))
    assert abs(out[2] - a.sum()) <= 1e-12 * a.sum()
    assert abs(out[0] - O.concentration_ratio(W, dtype, perm)) <= 1e-12
    again = H.hss_concentration(to_dev(W, dtype), None if perm is None else _raw(perm)).cpu().numpy()
    assert np.array_equal(out.view(np.uint64), again.view(np.uint64))       # same bits


def _pack_reference(U, Vt, perm, m, n):
    """U_cat / Vt_cat from the definition (stored bits moved, zeros elsewhere)."""
    r = [u.shape[1] for u in U]
    off = np.cumsum([0] + r)
    R = off[-1]
    m1, n1 = m // 2, n // 2
    p = np.arange(m) if perm is None else perm
    Ucat = np.zeros((m, R), dtype=U[0].dtype)
    Vtcat = np.zeros((R, n), dtype=U[0].dtype)
    for b in range(4):
        bi, bj = b >> 1, b & 1
        rows = range(0, m1) if bi == 0 else range(m1, m)
        cols = range(0, n1) if bj == 0 else range(n1, n)
        for t, i in enumerate(rows):
            Ucat[p[i], off[b]:off[b + 1]] = U[b][t]
        for t, j in enumerate(cols):
            Vtcat[off[b]:off[b + 1], p[j]] = Vt[b][:, t]
    return Ucat, Vtcat


@pytest.mark.parametrize("dtype", [O.F32, O.BF16])
@pytest.mark.parametrize("m,n,r,permuted", [(12, 12, (3, 1, 2, 4), False), (13, 13, (2, 2, 1, 3), True),
                                            (40, 26, (8, 0, 2, 5), False), (9, 9, (0, 2, 0, 1), True)])
def test_hier_pack_bit_exact(H, dtype, m, n, r, permuted):
    rng = np.random.default_rng(m + sum(r))
    m1, n1 = m // 2, n // 2
    rows = [m1, m - m1]
    cols = [n1, n - n1]
    st = np.float32 if dtype == O.F32 else np.uint16
    U = [O.narrow(rng.standard_normal((rows[b >> 1], r[b])), dtype).astype(st) for b in range(4)]
    Vt = [O.narrow(rng.standard_normal((r[b], cols[b & 1])), dtype).astype(st) for b in range(4)]
    perm = rng.permutation(n).astype(np.int32) if permuted else None
    Ucat, Vtcat = H.hss_hier_pack([to_dev(u, dtype) if u.size else None for u in U],
                                  [to_dev(v, dtype) if v.size else None for v in Vt], m, n,
                                  None if perm is None else _raw(perm))
    eU, eV = _pack_reference(U, Vt, perm, m, n)
    assert O.bits_equal(to_host(Ucat), eU) and O.bits_equal(to_host(Vtcat), eV)


@pytest.mark.parametrize("dtype,b", [(O.F32, 1), (O.BF16, 1), (O.BF16, 8), (O.BF16, 64)])
@pytest.mark.parametrize("permuted", [False, True])
def test_hier_layer_apply(H, dtype, b, permuted):
    """W -> S (top 5 %) -> RCM order of S's support (the library's, equal to
    the oracle's) -> per-block truncated SVD of the permuted residual (ranks
    8 diagonal, 3 off) -> packed flat factors -> hss_apply, against the
    oracle's block-form apply of the same stored factors."""
    import torch
    m = n = 130
    W = syn.random_matrix(m, n, dtype, seed=50 + b, kind="t3")
    s = O.split_csr(W, dtype, O.topk_count(m, n, 5, 100))
    perm = None
    if permuted:
        perm = H.hss_rcm_order(s["row_ptr"], s["col_idx"], n)
        assert np.array_equal(perm, O.rcm_order(n, s["row_ptr"], s["col_idx"]))
    R64 = O.widen(s["residual"], dtype)
    Rp = R64 if perm is None else R64[perm][:, perm]
    blocks = O.hier_factors(Rp, 8, 3)
    keys = [(0, 0), (0, 1), (1, 0), (1, 1)]
    st = {k: (O.narrow(blocks[k][0], dtype), O.narrow(np.ascontiguousarray(blocks[k][1].T), dtype)) for k in keys}
    stored = {k: (O.widen(st[k][0], dtype), O.widen(st[k][1], dtype).T) for k in keys}
    Ucat, Vtcat = H.hss_hier_pack([to_dev(st[k][0], dtype) for k in keys], [to_dev(st[k][1], dtype) for k in keys],
                                  m, n, None if perm is None else _raw(perm.astype(np.int32)))
    k = len(s["col_idx"])
    A = H.HSSMatrix("csr", m, n, _tdt(dtype), U=Ucat, Vt=Vtcat, row_ptr=_raw(s["row_ptr"]),
                    col_idx=_raw(s["col_idx"]), values=to_dev(s["values"], dtype), nnz=k)
    X = syn.random_matrix(b, n, dtype, seed=60 + b, kind="normal", scale=1.0)
    Y = to_host(H.hss_apply(A, to_dev(X, dtype)))
    S64 = O.dense_from_csr(m, n, s["row_ptr"], s["col_idx"], s["values"], dtype)
    X64 = O.widen(X, dtype)
    Yref = O.hier_apply(S64, stored, perm, X64)
    Afull = S64 + O.hier_lowrank_dense(stored, perm, m, n)
    N = np.abs(X64) @ np.abs(Afull).T
    err = O.max_normalised_error(O.widen(Y, dtype), Yref, N)
    assert err <= O.TOL[dtype], f"max normalised error {err:.3e}"
