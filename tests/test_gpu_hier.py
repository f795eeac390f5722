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


# ---------------------------------------------------------------------------
# The compact block form (HSS_HIER2): the layer held in the permuted order,
# S' = P S P^T, x' = x[perm], y[perm] = y', and only the blocks' factors.
# ---------------------------------------------------------------------------

def _compact_reference(blocks_st, m, n):
    """U_c and Vt_c as the header lays them out, from the stored blocks."""
    keys = [(0, 0), (0, 1), (1, 0), (1, 1)]
    m1, n1 = m // 2, n // 2
    r = [blocks_st[k][0].shape[1] for k in keys]
    ru, ld = r[0] + r[1], n - n1
    dt = blocks_st[keys[0]][0].dtype
    Uc = np.zeros((m, ru), dtype=dt)
    Uc[:m1] = np.concatenate([blocks_st[(0, 0)][0], blocks_st[(0, 1)][0]], axis=1)
    Uc[m1:] = np.concatenate([blocks_st[(1, 0)][0], blocks_st[(1, 1)][0]], axis=1)
    Vtc = np.zeros((sum(r), ld), dtype=dt)
    o = 0
    for k in keys:
        vt = blocks_st[k][1]
        Vtc[o:o + vt.shape[0], :vt.shape[1]] = vt
        o += vt.shape[0]
    return Uc, Vtc


def _hier_compact_case(H, dtype, m, seed, ranks, permuted, svd=True):
    """S (top 5 %), the RCM order of its support (or none), the block factors
    of the permuted residual (oracle SVDs, or seeded stand-ins), the layer in
    the permuted order: (A, perm, S64, stored blocks, Uc, Vtc, blocks_st)."""
    n = m
    W = syn.random_matrix(m, n, dtype, seed=seed, kind="t3")
    s = O.split_csr(W, dtype, O.topk_count(m, n, 5, 100))
    perm = H.hss_rcm_order(s["row_ptr"], s["col_idx"], n) if permuted else np.arange(n, dtype=np.int32)
    keys = [(0, 0), (0, 1), (1, 0), (1, 1)]
    rows, cols = (m // 2, m - m // 2), (n // 2, n - n // 2)
    if svd:
        R64 = O.widen(s["residual"], dtype)[perm][:, perm]
        res = {}
        for bi in range(2):
            for bj in range(2):
                blk = R64[(0 if bi == 0 else m // 2):(m // 2 if bi == 0 else m),
                          (0 if bj == 0 else n // 2):(n // 2 if bj == 0 else n)]
                U, V, _ = O.truncated_svd(blk, ranks[2 * bi + bj])
                res[(bi, bj)] = (U, V)
        st = {k: (O.narrow(res[k][0], dtype), O.narrow(np.ascontiguousarray(res[k][1].T), dtype)) for k in keys}
    else:
        st = {}
        for b, k in enumerate(keys):
            U, V = syn.factors(rows[k[0]], cols[k[1]], ranks[b], dtype, seed + 7, b)
            st[k] = (U, np.ascontiguousarray(V.T))
    stored = {k: (O.widen(st[k][0], dtype), O.widen(st[k][1], dtype).T) for k in keys}
    # S' = P S P^T: the library's host permutation (equal to the oracle's), values moved on the device
    prp, pci, src = H.hss_csr_permute(s["row_ptr"], s["col_idx"], perm, n)
    orp, oci, osrc = O.csr_permute(n, s["row_ptr"], s["col_idx"], perm)
    assert np.array_equal(prp, orp) and np.array_equal(pci, oci) and np.array_equal(src, osrc)
    k = len(s["col_idx"])
    vals = to_dev(s["values"], dtype)
    pvals = H.hss_gather_values(vals, _raw(src.astype(np.int32))) if k else vals
    Uc, Vtc = H.hss_hier_pack_compact([to_dev(st[kk][0], dtype) for kk in keys],
                                      [to_dev(st[kk][1], dtype) for kk in keys], m, n)
    A = H.HSSMatrix("csr", m, n, _tdt(dtype), U=Uc, Vt=Vtc, row_ptr=_raw(prp), col_idx=_raw(pci),
                    values=pvals, nnz=k, hier_r=ranks)
    S64 = O.dense_from_csr(m, n, s["row_ptr"], s["col_idx"], s["values"], dtype)
    return A, perm, S64, stored, st


def _check_hier_apply(H, A, perm, S64, stored, dtype, X):
    """hss_apply in the permuted order against the oracle's block-form apply
    in the original order: x' = x[perm], y[perm] = y'."""
    m, n = S64.shape
    Xp = np.ascontiguousarray(X[:, perm])
    Yp = to_host(H.hss_apply(A, to_dev(Xp, dtype)))
    Y = np.empty_like(Yp)
    Y[:, perm] = Yp
    X64 = O.widen(X, dtype)
    Yref = O.hier_apply(S64, stored, perm, X64)
    N = np.abs(X64) @ np.abs(S64 + O.hier_lowrank_dense(stored, perm, m, n)).T
    err = O.max_normalised_error(O.widen(Y, dtype), Yref, N)
    assert err <= O.TOL[dtype], f"max normalised error {err:.3e}"
    return Yp


@pytest.mark.parametrize("dtype,b", [(O.F32, 1), (O.F32, 3), (O.BF16, 1), (O.BF16, 2), (O.BF16, 5),
                                     (O.BF16, 64), (O.BF16, 300)])
@pytest.mark.parametrize("m,ranks,permuted", [(130, (8, 3, 3, 8), True), (131, (8, 3, 5, 6), False),
                                              (2050, (40, 8, 8, 40), True), (2064, (32, 16, 16, 32), True)])
def test_hier_compact_apply(H, dtype, b, m, ranks, permuted):
    """The compact block form through every route (b = 1, 2: fused decode
    kernel on the compact factors; 3 fp32: decode; 5, 64: gather SpMM and 300:
    matrix cores on factors expanded in the workspace) against the oracle;
    half widths off the 16-byte grid (65 / 66 / 1025: element-wise V^T
    rows; 2050: two rows per wave, one in each row half) and on it (1032:
    the vector path), unequal block ranks, the RCM order; compact factors
    bit-exact to their layout."""
    if m > 1000 and b > 5:
        pytest.skip("large shape: decode batches only")
    A, perm, S64, stored, st = _hier_compact_case(H, dtype, m, 70 + m % 7 + b, ranks, permuted, svd=m < 1000)
    eU, eV = _compact_reference(st, m, m)
    assert O.bits_equal(to_host(A.U), eU) and O.bits_equal(to_host(A.Vt), eV)
    X = syn.random_matrix(b, m, dtype, seed=80 + b, kind="normal", scale=1.0)
    _check_hier_apply(H, A, perm, S64, stored, dtype, X)


def test_hier_compact_local_fallback_and_group(H, hss_opt):
    """Every T row recomputed by every block (the fallback path's column
    halves) gives the same bits as the hand-off; two compact matrices in one
    grouped call equal their single applies within the bar and repeat bit
    for bit; a graph replay matches."""
    import torch
    dtype = O.BF16
    A1, perm, S64, stored, _ = _hier_compact_case(H, dtype, 272, 91, (16, 4, 4, 16), True)
    X = syn.random_matrix(1, 272, dtype, seed=92, kind="normal", scale=1.0)
    Xp = to_dev(np.ascontiguousarray(X[:, perm]), dtype)
    y0 = to_host(H.hss_apply(A1, Xp))
    hss_opt("decode_force_local", 1)
    y1 = to_host(H.hss_apply(A1, Xp))
    hss_opt("decode_force_local", 0)
    assert O.bits_equal(y0, y1)
    _check_hier_apply(H, A1, perm, S64, stored, dtype, X)
    # a second compact matrix in the same (permuted) basis: same S pattern, other blocks
    A2 = H.HSSMatrix("csr", 272, 272, torch.bfloat16, U=(A1.U * 2).contiguous(), Vt=A1.Vt, row_ptr=A1.row_ptr,
                     col_idx=A1.col_idx, values=A1.values, nnz=A1.nnz, hier_r=A1.hier_r)
    ys = [torch.empty((1, 272), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    ws = H.apply_workspace(H.hss_apply_group_workspace_size([A1, A2], 1), "cuda")
    H.hss_apply_group([A1, A2], Xp, ys, ws)
    g0 = [to_host(y) for y in ys]
    H.hss_apply_group([A1, A2], Xp, ys, ws)
    assert all(O.bits_equal(to_host(y), g) for y, g in zip(ys, g0))
    single = [y0, to_host(H.hss_apply(A2, Xp))]
    for g, s_ in zip(g0, single):
        d = np.abs(O.widen(g, dtype) - O.widen(s_, dtype))
        assert np.all(d <= 8e-3 * (np.abs(O.widen(s_, dtype)) + 1e-2))
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        H.hss_apply_group([A1, A2], Xp, ys, ws)
    for _ in range(2):
        for y in ys:
            y.zero_()
        gr.replay()
        torch.cuda.synchronize()
        assert all(O.bits_equal(to_host(y), g) for y, g in zip(ys, g0))
