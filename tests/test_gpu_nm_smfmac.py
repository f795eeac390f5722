"""GPU parity of the 2:4 route on the sparse matrix cores (bf16, 2..64
columns): S's values and metadata go to v_smfmac as stored, T = X V comes
from a vector-unit prologue (up to 16 columns) or a matrix-core one.  Checked against the CPU oracle with the apply
bar (every output within 8e-3 * sum_j |A_ij X_cj|), forced through
HSS_CSR_BATCH_ROUTE=smfmac and through the default route."""
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


def _layer(H, m, n, r, seed):
    import torch
    W = syn.random_matrix(m, n, DT, seed=seed, kind="t3")
    ref = O.split_24(W, DT)
    if r:
        U, V = syn.factors(m, n, r, DT, seed)
    else:
        U, V = np.zeros((m, 0), np.uint16), np.zeros((n, 0), np.uint16)
    A = H.HSSMatrix("2:4", m, n, torch.bfloat16, U=to_dev(U, DT) if r else None,
                    Vt=to_dev(np.ascontiguousarray(V.T), DT) if r else None,
                    nm_values=to_dev(ref["nm_values"], DT), nm_meta=_raw(ref["nm_meta"].view(np.int32)))
    S64 = O.dense_from_24(m, n, ref["nm_values"], ref["nm_meta"], DT)
    return A, S64, O.widen(U, DT), O.widen(V, DT)


def _check(Y, S64, U64, V64, X64):
    err = O.max_normalised_error(O.widen(to_host(Y), DT), O.apply_factored(S64, U64, V64, X64),
                                 O.normaliser(S64, U64, V64, X64))
    assert err <= O.TOL[DT], f"max normalised error {err:.3e}"


CASES = [
    # (m, n, r, b): one 32-row tile and ragged ones; 1 .. 32 stages of 128
    # columns (fewer stages than waves, and a last wave with a partial range);
    # rank 0, ranks ending mid-step (r % 16 == 8) and off the 16-byte grid
    # (r % 8 != 0), ranks needing several steps per wave (r > 128); 1 and 2
    # column tiles
    (32, 128, 0, 2), (1, 128, 3, 3), (33, 384, 8, 8), (100, 256, 16, 17), (257, 1152, 24, 31),
    (64, 4096, 64, 32), (300, 512, 200, 33), (129, 1024, 13, 63), (70, 640, 272, 64),
    (2053, 128, 40, 5),
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}x{c[1]}-r{c[2]}-b{c[3]}" for c in CASES])
def test_smfmac_matches_oracle(H, hss_opt, case):
    m, n, r, b = case
    seed = 5 * m + n + 3 * r + b
    A, S64, U64, V64 = _layer(H, m, n, r, seed)
    X = syn.random_matrix(b, n, DT, seed=seed + 1, kind="normal", scale=1.0)
    Xd = to_dev(X, DT)
    hss_opt("batch_route", "smfmac")
    Y1 = H.hss_apply(A, Xd)
    _check(Y1, S64, U64, V64, O.widen(X, DT))
    assert O.bits_equal(to_host(Y1), to_host(H.hss_apply(A, Xd)))      # deterministic
    hss_opt("batch_route", "auto")
    if b >= 3:
        assert O.bits_equal(to_host(Y1), to_host(H.hss_apply(A, Xd)))  # the default route for 3..64 columns


@pytest.mark.parametrize("b", [2, 16, 64])
def test_smfmac_agrees_with_decode_and_densify(H, hss_opt, b):
    """The other routes of the same call stay within the bar (they differ in
    rounding: T is bf16 on the matrix-core routes, fp32 in the decode)."""
    m, n, r = 200, 512, 48
    A, S64, U64, V64 = _layer(H, m, n, r, 90 + b)
    X = syn.random_matrix(b, n, DT, seed=91 + b, kind="normal", scale=1.0)
    Xd = to_dev(X, DT)
    for route in ("smfmac", "decode", "densify"):
        hss_opt("batch_route", route)
        _check(H.hss_apply(A, Xd), S64, U64, V64, O.widen(X, DT))


def test_smfmac_unaligned_x_takes_another_route(H):
    """X one element past a 16-byte boundary: the call still runs (on a route
    without the alignment need) and meets the bar."""
    import torch
    m, n, r, b = 96, 256, 16, 4
    A, S64, U64, V64 = _layer(H, m, n, r, 77)
    X = syn.random_matrix(b, n, DT, seed=78, kind="normal", scale=1.0)
    buf = torch.empty(b * n + 8, dtype=torch.bfloat16, device="cuda")
    Xs = buf[1:1 + b * n].view(b, n)
    Xs.copy_(to_dev(X, DT))
    assert Xs.data_ptr() % 16 != 0
    _check(H.hss_apply(A, Xs), S64, U64, V64, O.widen(X, DT))


def test_smfmac_graph_replay_matches_eager(H):
    import torch
    m, n, r, b = 300, 512, 40, 24
    A, _, _, _ = _layer(H, m, n, r, 81)
    xs = [to_dev(syn.random_matrix(b, n, DT, seed=82 + i, kind="normal", scale=1.0), DT) for i in range(3)]
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


def test_smfmac_group_equals_single_applies(H):
    n, b = 256, 8
    layers = [_layer(H, m, n, r, 60 + m) for m, r in ((200, 16), (64, 0), (301, 40))]
    X = syn.random_matrix(b, n, DT, seed=61, kind="normal", scale=1.0)
    Xd = to_dev(X, DT)
    Ys = H.hss_apply_group([L[0] for L in layers], Xd)
    for (A, S64, U64, V64), Y in zip(layers, Ys):
        assert O.bits_equal(to_host(Y), to_host(H.hss_apply(A, Xd)))
        _check(Y, S64, U64, V64, O.widen(X, DT))


@pytest.mark.parametrize("b", [2, 33])
def test_smfmac_11008x4096_sampled(H, hss_opt, b):
    """The 11008 x 4096 2:4 rank-64 layer on this route (rows sampled; every
    row at b = 8 and 64, through the default route, in the full-size tests)."""
    hss_opt("batch_route", "smfmac")
    c = syn.WORKLOADS["nm24_11008x4096"]
    m, n = c.shapes[0]
    r = c.rank[0]
    ref = oracle_split("nm24_11008x4096")
    U, V = syn.factors(m, n, r, DT, c.seed)
    import torch
    A = H.HSSMatrix("2:4", m, n, torch.bfloat16, U=to_dev(U, DT), Vt=to_dev(np.ascontiguousarray(V.T), DT),
                    nm_values=to_dev(ref["nm_values"], DT), nm_meta=_raw(ref["nm_meta"].view(np.int32)))
    X = syn.activations(c, b, 0, 0)
    Y = to_host(H.hss_apply(A, to_dev(X, DT)))
    rows = np.sort(np.random.default_rng(b).choice(m, size=384, replace=False))
    S_rows = O.dense_from_24(len(rows), n, ref["nm_values"][rows], ref["nm_meta"][rows], DT)
    Yref, N = O.apply_rows(S_rows, O.widen(U, DT)[rows], O.widen(V, DT), O.widen(X, DT))
    err = O.max_normalised_error(O.widen(Y[:, rows], DT), Yref, N)
    assert err <= O.TOL[DT], f"max normalised error {err:.3e}"


def test_smfmac_shared_workspace_across_routes(H, hss_opt):
    """One workspace, calls alternating between this route, the fused decode
    and the densified GEMM (whose scratch overlaps the T partials): every
    result equals the one from a fresh workspace (the T tile counters live in
    the control region and are cleared by the call that used them)."""
    import torch
    m, n, r = 260, 512, 72
    A, _, _, _ = _layer(H, m, n, r, 101)
    calls = [(b, route) for b in (8, 40, 16) for route in ("smfmac", "decode", "densify")]
    xs = {b: to_dev(syn.random_matrix(b, n, DT, seed=102 + b, kind="normal", scale=1.0), DT) for b in (8, 16, 40)}
    expect = {}
    for b, route in calls:
        hss_opt("batch_route", route)
        expect[(b, route)] = to_host(H.hss_apply(A, xs[b]))
    size = max(H.hss_apply_workspace_size(A, b) for b in xs)
    ws = H.apply_workspace(size, "cuda")
    for it in range(3):
        for b, route in calls:
            hss_opt("batch_route", route)
            assert O.bits_equal(to_host(H.hss_apply(A, xs[b], ws=ws)), expect[(b, route)]), (it, b, route)
