"""GPU parity of the batched CSR routes (bf16): the gather SpMM, the fused
decode passes and the densified matrix-core GEMM, each forced through
HSS_CSR_BATCH_ROUTE and checked against the CPU oracle with the apply bar
(every output within 8e-3 * sum_j |A_ij X_cj|)."""
import numpy as np
import pytest

import hss_synth as syn
import oracle as O
from _cases import oracle_split, to_dev, to_host

pytestmark = pytest.mark.gpu

DT = O.BF16


@pytest.fixture(scope="module")
def H():
    import sparse_rank_linear_hss_amd as h
    return h


def _raw(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _layer(H, m, n, r, seed, frac=(5, 100), col16=False):
    import torch
    W = syn.random_matrix(m, n, DT, seed=seed, kind="t3")
    ref = O.split_csr(W, DT, O.topk_count(m, n, *frac))
    if r:
        U, V = syn.factors(m, n, r, DT, seed)
    else:
        U, V = np.zeros((m, 0), np.uint16), np.zeros((n, 0), np.uint16)
    k = len(ref["col_idx"])
    cols = ref["col_idx"].astype(np.uint16) if col16 else ref["col_idx"]
    A = H.HSSMatrix("csr", m, n, torch.bfloat16, U=to_dev(U, DT) if r else None,
                    Vt=to_dev(np.ascontiguousarray(V.T), DT) if r else None, row_ptr=_raw(ref["row_ptr"]),
                    col_idx=_raw(cols.view(np.int16) if col16 else cols) if k else None,
                    values=to_dev(ref["values"], DT) if k else None, nnz=k)
    S64 = O.dense_from_csr(m, n, ref["row_ptr"], ref["col_idx"], ref["values"], DT)
    return A, S64, O.widen(U, DT), O.widen(V, DT)


def _check(Y, S64, U64, V64, X64):
    err = O.max_normalised_error(O.widen(to_host(Y), DT), O.apply_factored(S64, U64, V64, X64),
                                 O.normaliser(S64, U64, V64, X64))
    assert err <= O.TOL[DT], f"max normalised error {err:.3e}"


CASES = [
    # (m, n, r, b): ragged rows, columns and batch tiles of 8 / 16 / 32 / 64 columns
    (1, 1, 0, 2), (5, 13, 2, 3), (65, 129, 7, 9), (130, 1000, 64, 16), (257, 512, 1, 17),
    (300, 640, 128, 33), (300, 640, 256, 64), (100, 77, 5, 65), (520, 512, 256, 130),
    (200, 256, 300, 8), (64, 4100, 33, 300), (2053, 256, 16, 5), (90, 200, 0, 40),
    # a rank whose T tile only fits 16 columns: four batch tiles
    (64, 2048, 2048, 64),
]


@pytest.mark.parametrize("route", ["spmm", "decode", "densify"])
@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}x{c[1]}-r{c[2]}-b{c[3]}" for c in CASES])
def test_route_matches_oracle(H, hss_opt, route, case):
    m, n, r, b = case
    seed = m + 3 * n + r + b
    A, S64, U64, V64 = _layer(H, m, n, r, seed)
    X = syn.random_matrix(b, n, DT, seed=seed + 1, kind="normal", scale=1.0)
    hss_opt("batch_route", route)
    Xd = to_dev(X, DT)
    Y1 = H.hss_apply(A, Xd)
    _check(Y1, S64, U64, V64, O.widen(X, DT))
    assert O.bits_equal(to_host(Y1), to_host(H.hss_apply(A, Xd)))     # deterministic


@pytest.mark.parametrize("b,r", [(7, 6), (16, 0), (64, 32)])
def test_spmm_empty_sparse_part_and_empty_rows(H, hss_opt, b, r):
    """k = 0 (a pure low-rank product, or exact zeros with r = 0), and a
    split so sparse that most rows are empty."""
    hss_opt("batch_route", "spmm")
    for frac in ((0, 100), (1, 1000)):
        A, S64, U64, V64 = _layer(H, 150, 96, r, 7 + b, frac=frac)
        X = syn.random_matrix(b, 96, DT, seed=8, kind="normal", scale=1.0)
        _check(H.hss_apply(A, to_dev(X, DT)), S64, U64, V64, O.widen(X, DT))


@pytest.mark.parametrize("b", [3, 16, 40])
def test_spmm_col16_bit_equal_to_int32(H, hss_opt, b):
    hss_opt("batch_route", "spmm")
    A32, S64, U64, V64 = _layer(H, 140, 300, 24, 30 + b)
    A16, _, _, _ = _layer(H, 140, 300, 24, 30 + b, col16=True)
    Xd = to_dev(syn.random_matrix(b, 300, DT, seed=31, kind="normal", scale=1.0), DT)
    Y32 = to_host(H.hss_apply(A32, Xd))
    assert O.bits_equal(Y32, to_host(H.hss_apply(A16, Xd)))


@pytest.mark.parametrize("b", [16, 64])
def test_spmm_graph_replay_matches_eager(H, hss_opt, b):
    import torch
    hss_opt("batch_route", "spmm")
    m, n = 300, 256
    A, _, _, _ = _layer(H, m, n, 48, 61)
    xs = [to_dev(syn.random_matrix(b, n, DT, seed=62 + i, kind="normal", scale=1.0), DT) for i in range(3)]
    ys = [torch.empty((b, m), dtype=torch.bfloat16, device="cuda") for _ in range(3)]
    ws = A.workspace(b)
    expect = [to_host(H.hss_apply(A, x, ws=ws)) for x in xs]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for x, y in zip(xs, ys):
            H.hss_apply(A, x, y, ws)
    for rep in range(3):
        for y in ys:
            y.zero_()
        g.replay()
        torch.cuda.synchronize()
        for i in range(3):
            assert O.bits_equal(to_host(ys[i]), expect[i]), (rep, i)
        assert O.bits_equal(to_host(H.hss_apply(A, xs[rep % 3], ws=ws)), expect[rep % 3])


@pytest.mark.parametrize("b", [12, 48])
def test_spmm_group_equals_single_applies(H, hss_opt, b):
    hss_opt("batch_route", "spmm")
    n = 256
    layers = [_layer(H, m, n, r, 70 + m) for m, r in ((200, 16), (64, 0), (301, 40))]
    X = syn.random_matrix(b, n, DT, seed=71, kind="normal", scale=1.0)
    Xd = to_dev(X, DT)
    Ys = H.hss_apply_group([L[0] for L in layers], Xd)
    for (A, S64, U64, V64), Y in zip(layers, Ys):
        assert O.bits_equal(to_host(Y), to_host(H.hss_apply(A, Xd)))
        _check(Y, S64, U64, V64, O.widen(X, DT))


def _full(H, wl, b, rows, route, hss_opt):
    c = syn.WORKLOADS[wl]
    m, n = c.shapes[0]
    r = c.rank[0]
    ref = oracle_split(wl)
    U, V = syn.factors(m, n, r, DT, c.seed)
    import torch
    A = H.HSSMatrix("csr", m, n, torch.bfloat16, U=to_dev(U, DT), Vt=to_dev(np.ascontiguousarray(V.T), DT),
                    row_ptr=_raw(ref["row_ptr"]), col_idx=_raw(ref["col_idx"]),
                    values=to_dev(ref["values"], DT), nnz=len(ref["col_idx"]))
    X = syn.activations(c, b, 0, 0)
    hss_opt("batch_route", route)
    Y = to_host(H.hss_apply(A, to_dev(X, DT)))
    S_rows = O.csr_rows_dense(rows, n, ref["row_ptr"], ref["col_idx"], ref["values"], DT)
    Yref, N = O.apply_rows(S_rows, O.widen(U, DT)[rows], O.widen(V, DT), O.widen(X, DT))
    err = O.max_normalised_error(O.widen(Y[:, rows], DT), Yref, N)
    assert err <= O.TOL[DT], f"max normalised error {err:.3e}"


@pytest.mark.parametrize("b", [4, 64, 256])
def test_spmm_4096_layer_sampled(H, hss_opt, b):
    """The 4096 x 4096 top-5 % rank-256 layer on the gather route."""
    rows = np.sort(np.random.default_rng(b).choice(4096, size=256, replace=False))
    _full(H, "csr4096", b, rows, "spmm", hss_opt)


def test_spmm_8192_prefill_sampled(H, hss_opt):
    """The 8192 x 8192 top-3 % rank-512 layer at b = 2048 on the gather route
    (32 batch tiles of 64 columns)."""
    rows = np.sort(np.random.default_rng(9).choice(8192, size=64, replace=False))
    _full(H, "csr8192_prefill", 2048, rows, "spmm", hss_opt)
