"""GPU parity of the backward pass (bf16 CSR layers) against the CPU oracle.

Bar: every gradient entry within 8e-3 of its scale, the same sum with every
term's magnitude (|G|^T |X| |V| for dU, |X|^T |G| |U| for dV, sum_c |G_ci
X_cj| for dS, |G| |S + U V^T| for dX): the GEMM path rounds X V and G U to
bf16 once and accumulates in fp32, as the forward does.  Inputs are the
seeded layers of the apply tests, S from the oracle's own split."""
import numpy as np
import pytest

import hss_synth as syn
import oracle as O
from _cases import oracle_split, to_dev, to_host

pytestmark = pytest.mark.gpu

DT = O.BF16
TOL = O.TOL[O.BF16]


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
    cols = ref["col_idx"].astype(np.uint16).view(np.int16) if col16 else ref["col_idx"]
    A = H.HSSMatrix("csr", m, n, torch.bfloat16, U=to_dev(U, DT) if r else None,
                    Vt=to_dev(np.ascontiguousarray(V.T), DT) if r else None, row_ptr=_raw(ref["row_ptr"]),
                    col_idx=_raw(cols) if k else None, values=to_dev(ref["values"], DT) if k else None, nnz=k)
    S64 = O.dense_from_csr(m, n, ref["row_ptr"], ref["col_idx"], ref["values"], DT)
    return A, ref, S64, O.widen(U, DT), O.widen(V, DT)


def _within(got, ref, scale, what):
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - ref)
    zero = scale == 0
    assert np.all(err[zero] == 0), what
    if np.any(~zero):
        worst = float(np.max(err[~zero] / scale[~zero]))
        assert worst <= TOL, f"{what}: max normalised error {worst:.3e}"


CASES = [
    # (m, n, r, b): ragged shapes, batches below / at / across the 8-column padding and K tails
    (5, 13, 2, 3), (65, 129, 7, 9), (130, 1000, 64, 16), (257, 512, 1, 33), (300, 640, 128, 64),
    (100, 77, 5, 65), (520, 512, 256, 130), (64, 256, 16, 600), (2053, 256, 16, 5),
    # one column: the reductions over the batch are GEMMs with K = 1
    (40, 64, 4, 1),
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}x{c[1]}-r{c[2]}-b{c[3]}" for c in CASES])
def test_backward_matches_oracle(H, case):
    m, n, r, b = case
    seed = 3 * m + n + r + b
    A, ref, S64, U64, V64 = _layer(H, m, n, r, seed)
    X = syn.random_matrix(b, n, DT, seed=seed + 1, kind="normal", scale=1.0)
    G = syn.random_matrix(b, m, DT, seed=seed + 2, kind="normal", scale=1.0)
    X64, G64 = O.widen(X, DT), O.widen(G, DT)
    g = O.backward(m, n, ref["row_ptr"], ref["col_idx"], S64, U64, V64, X64, G64)
    N = O.backward_normalisers(m, n, ref["row_ptr"], ref["col_idx"], S64, U64, V64, X64, G64)
    out = H.hss_backward(A, to_dev(X, DT), to_dev(G, DT))
    _within(out["dS"].cpu().numpy(), g["dS"], N["dS"], "dS")
    _within(out["dU"].cpu().numpy(), g["dU"], N["dU"], "dU")
    _within(out["dVt"].cpu().numpy().T, g["dV"], N["dV"], "dV")
    _within(O.widen(to_host(out["dX"]), DT), g["dX"], N["dX"], "dX")
    again = H.hss_grad(A, to_dev(X, DT), to_dev(G, DT))
    for k in ("dS", "dU", "dVt"):                                      # deterministic
        assert np.array_equal(again[k].cpu().numpy().view(np.uint32), out[k].cpu().numpy().view(np.uint32)), k


def test_backward_skips_and_degenerate_layers(H):
    """Outputs may be skipped; an empty S and r = 0 are handled."""
    m, n, b = 90, 64, 12
    X = syn.random_matrix(b, n, DT, seed=1, kind="normal", scale=1.0)
    G = syn.random_matrix(b, m, DT, seed=2, kind="normal", scale=1.0)
    X64, G64 = O.widen(X, DT), O.widen(G, DT)
    for r, frac in ((8, (0, 100)), (0, (5, 100))):
        A, ref, S64, U64, V64 = _layer(H, m, n, r, 40 + r, frac=frac)
        g = O.backward(m, n, ref["row_ptr"], ref["col_idx"], S64, U64, V64, X64, G64)
        N = O.backward_normalisers(m, n, ref["row_ptr"], ref["col_idx"], S64, U64, V64, X64, G64)
        out = H.hss_grad(A, to_dev(X, DT), to_dev(G, DT))
        if r:
            _within(out["dU"].cpu().numpy(), g["dU"], N["dU"], "dU")
            _within(out["dVt"].cpu().numpy().T, g["dV"], N["dV"], "dV")
        if len(ref["col_idx"]):
            _within(out["dS"].cpu().numpy(), g["dS"], N["dS"], "dS")
        dX = H.hss_apply(H.hss_transposed_layer(A), to_dev(G, DT))
        _within(O.widen(to_host(dX), DT), g["dX"], N["dX"], "dX")
    A, ref, S64, U64, V64 = _layer(H, m, n, 8, 48)
    only_u = H.hss_grad(A, to_dev(X, DT), to_dev(G, DT), dS=False, dVt=False)
    full = H.hss_grad(A, to_dev(X, DT), to_dev(G, DT))
    assert set(only_u) == {"dU"}
    assert np.array_equal(only_u["dU"].cpu().numpy(), full["dU"].cpu().numpy())


def test_grad_col16_bit_equal_to_int32(H):
    m, n, b = 140, 300, 24
    A32, *_ = _layer(H, m, n, 16, 77)
    A16, *_ = _layer(H, m, n, 16, 77, col16=True)
    X = to_dev(syn.random_matrix(b, n, DT, seed=5, kind="normal", scale=1.0), DT)
    G = to_dev(syn.random_matrix(b, m, DT, seed=6, kind="normal", scale=1.0), DT)
    a, c = H.hss_grad(A32, X, G), H.hss_grad(A16, X, G)
    for k in a:
        assert np.array_equal(a[k].cpu().numpy(), c[k].cpu().numpy()), k


def test_transposed_layer_is_exact(H):
    """S^T's pattern and permutation equal the oracle's; values and the two
    factors are moved bit for bit."""
    m, n, r = 77, 130, 12
    A, ref, S64, U64, V64 = _layer(H, m, n, r, 91)
    At = H.hss_transposed_layer(A)
    rpt, cit, perm = O.csr_transpose(m, n, ref["row_ptr"], ref["col_idx"])
    assert np.array_equal(At.row_ptr.cpu().numpy(), rpt) and np.array_equal(At.col_idx.cpu().numpy(), cit)
    assert np.array_equal(to_host(At.values), ref["values"][perm])
    assert np.array_equal(to_host(At.U), to_host(A.Vt).T) and np.array_equal(to_host(At.Vt), to_host(A.U).T)
    f = to_dev(syn.random_matrix(33, 50, O.F32, seed=3, kind="normal", scale=1.0), O.F32)
    assert np.array_equal(H.hss_transpose(f).cpu().numpy(), f.cpu().numpy().T)


def test_backward_8192_layer_sampled(H):
    """The 8192 x 8192 top-3 % rank-512 layer at b = 2048 (the training-size
    shape): dU and dV on sampled rows, dS on sampled entries, dX on sampled
    columns."""
    import torch
    c = syn.WORKLOADS["csr8192_prefill"]
    m, n = c.shapes[0]
    r = c.rank[0]
    ref = oracle_split("csr8192_prefill")
    U, V = syn.factors(m, n, r, DT, c.seed)
    A = H.HSSMatrix("csr", m, n, torch.bfloat16, U=to_dev(U, DT), Vt=to_dev(np.ascontiguousarray(V.T), DT),
                    row_ptr=_raw(ref["row_ptr"]), col_idx=_raw(ref["col_idx"]), values=to_dev(ref["values"], DT),
                    nnz=len(ref["col_idx"]))
    b = 2048
    X = syn.activations(c, b, 0, 0)
    G = syn.random_matrix(b, m, DT, seed=17, kind="normal", scale=1.0)
    out = H.hss_backward(A, to_dev(X, DT), to_dev(G, DT))
    rng = np.random.default_rng(4)
    rows = np.sort(rng.choice(m, 48, replace=False))
    cols = np.sort(rng.choice(n, 48, replace=False))
    pick = np.sort(rng.choice(len(ref["col_idx"]), 256, replace=False))
    er = O.csr_row_of_entry(m, ref["row_ptr"])[pick]
    ec = ref["col_idx"][pick]
    U64, V64, X64, G64 = O.widen(U, DT), O.widen(V, DT), O.widen(X, DT), O.widen(G, DT)
    smp = O.backward_sampled(rows, cols, er, ec, U64, V64, X64, G64)
    _within(out["dU"].cpu().numpy()[rows], smp["dU"], smp["NU"], "dU")
    _within(out["dVt"].cpu().numpy()[:, cols].T, smp["dV"], smp["NV"], "dV")
    _within(out["dS"].cpu().numpy()[pick], smp["dS"], smp["NS"], "dS")
    # dX columns j: G (S + U V^T)[:, j]
    S_cols = np.zeros((m, len(cols)))
    Sfull_rows = O.csr_row_of_entry(m, ref["row_ptr"])
    vals = O.widen(ref["values"], DT)
    for k, j in enumerate(cols):
        hit = ref["col_idx"] == j
        S_cols[Sfull_rows[hit], k] = vals[hit]
    A_cols = S_cols + U64 @ V64[cols].T
    dX_ref, NX = G64 @ A_cols, np.abs(G64) @ np.abs(A_cols)
    _within(O.widen(to_host(out["dX"]), DT)[:, cols], dX_ref, NX, "dX")


@pytest.mark.parametrize("route,b", [("dense", 16), ("sparse", 600), ("dense", 5)])
def test_ds_routes_forced(H, hss_opt, route, b):
    """Both forms of dS (the sampled product and the dense G^T X plus gather)
    on the other side of their default batch threshold."""
    m, n, r = 130, 264, 8
    A, ref, S64, U64, V64 = _layer(H, m, n, r, 55 + b)
    X = syn.random_matrix(b, n, DT, seed=56, kind="normal", scale=1.0)
    G = syn.random_matrix(b, m, DT, seed=57, kind="normal", scale=1.0)
    X64, G64 = O.widen(X, DT), O.widen(G, DT)
    g = O.backward(m, n, ref["row_ptr"], ref["col_idx"], S64, U64, V64, X64, G64)
    N = O.backward_normalisers(m, n, ref["row_ptr"], ref["col_idx"], S64, U64, V64, X64, G64)
    hss_opt("grad_ds_route", route)
    out = H.hss_grad(A, to_dev(X, DT), to_dev(G, DT))
    _within(out["dS"].cpu().numpy(), g["dS"], N["dS"], "dS")
    _within(out["dU"].cpu().numpy(), g["dU"], N["dU"], "dU")


def _layer24(H, m, n, r, seed):
    import torch
    W = syn.random_matrix(m, n, DT, seed=seed, kind="normal")
    s = O.split_24(W, DT)
    U, V = syn.factors(m, n, r, DT, seed)
    A = H.HSSMatrix("2:4", m, n, torch.bfloat16, U=to_dev(U, DT), Vt=to_dev(np.ascontiguousarray(V.T), DT),
                    nm_values=to_dev(s["nm_values"], DT), nm_meta=_raw(s["nm_meta"].view(np.int32)))
    rp, ci = O.nm24_pattern(m, n, s["nm_meta"])
    S64 = O.dense_from_24(m, n, s["nm_values"], s["nm_meta"], DT)
    return A, s, rp, ci, S64, O.widen(U, DT), O.widen(V, DT)


@pytest.mark.parametrize("m,n,r,b,route", [(40, 64, 8, 5, None), (130, 96, 16, 33, None), (70, 128, 4, 16, "dense"),
                                           (36, 32, 4, 1, None),
                                           (64, 256, 16, 600, None), (64, 256, 16, 600, "sparse")])
def test_backward_2of4_matches_oracle(H, hss_opt, m, n, r, b, route):
    """A 2:4 layer: dS laid out as nm_values, dU, dV, and dX through the
    transposed layer built from the 2:4 positions."""
    if route:
        hss_opt("grad_ds_route", route)
    A, s, rp, ci, S64, U64, V64 = _layer24(H, m, n, r, 100 + m + b)
    X = syn.random_matrix(b, n, DT, seed=101, kind="normal", scale=1.0)
    G = syn.random_matrix(b, m, DT, seed=102, kind="normal", scale=1.0)
    X64, G64 = O.widen(X, DT), O.widen(G, DT)
    g = O.backward(m, n, rp, ci, S64, U64, V64, X64, G64)
    N = O.backward_normalisers(m, n, rp, ci, S64, U64, V64, X64, G64)
    out = H.hss_backward(A, to_dev(X, DT), to_dev(G, DT))
    _within(out["dS"].cpu().numpy(), g["dS"], N["dS"], "dS")
    _within(out["dU"].cpu().numpy(), g["dU"], N["dU"], "dU")
    _within(out["dVt"].cpu().numpy().T, g["dV"], N["dV"], "dV")
    _within(O.widen(to_host(out["dX"]), DT), g["dX"], N["dX"], "dX")


def test_nm24_to_csr_is_the_oracle_pattern(H):
    m, n = 33, 160
    A, s, rp, ci, *_ = _layer24(H, m, n, 4, 7)
    drp, dci = H.hss_nm24_to_csr(A)
    assert np.array_equal(drp.cpu().numpy(), rp) and np.array_equal(dci.cpu().numpy(), ci)


def test_fp32_input_gradient_through_transposed_layer(H):
    """An fp32 CSR layer (hss_grad is bf16-only): dX = G A still comes from
    the transposed layer's apply, within the fp32 bar."""
    import torch
    m, n, r, b = 90, 70, 6, 4
    W = syn.random_matrix(m, n, O.F32, seed=5, kind="t3")
    ref = O.split_csr(W, O.F32, O.topk_count(m, n, 5, 100))
    U, V = syn.factors(m, n, r, O.F32, 5)
    A = H.HSSMatrix("csr", m, n, torch.float32, U=to_dev(U, O.F32), Vt=to_dev(np.ascontiguousarray(V.T), O.F32),
                    row_ptr=_raw(ref["row_ptr"]), col_idx=_raw(ref["col_idx"]), values=to_dev(ref["values"], O.F32),
                    nnz=len(ref["col_idx"]))
    G = syn.random_matrix(b, m, O.F32, seed=6, kind="normal", scale=1.0)
    dX = H.hss_apply(H.hss_transposed_layer(A), to_dev(G, O.F32)).cpu().numpy()
    S64 = O.dense_from_csr(m, n, ref["row_ptr"], ref["col_idx"], ref["values"], O.F32)
    A64 = S64 + O.widen(U, O.F32) @ O.widen(V, O.F32).T
    G64 = O.widen(G, O.F32)
    err = O.max_normalised_error(dX.astype(np.float64), G64 @ A64, np.abs(G64) @ np.abs(A64))
    assert err <= O.TOL[O.F32], f"max normalised error {err:.3e}"
