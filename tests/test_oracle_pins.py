"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Each test ties an oracle function to something other than itself: numbers the
pages print (fixtures under tests/golden/, each with its citation), closed
forms, brute force on tiny inputs, or independent library routines.
"""
import itertools
import json
import os

import numpy as np
import pytest
import scipy.linalg
import scipy.sparse

import hss_synth as syn
import oracle as O
from conftest import GOLDEN


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# Counts: the 1024 x 1024 worked example and the rank rule
# ---------------------------------------------------------------------------

def test_worked_example_counts():
    g = _golden("worked_example_1024.json")
    m, n, r = g["m"], g["n"], g["rank"]
    k = O.topk_count(m, n, *g["kept_fraction"])
    assert m * n == g["dense_params"]
    assert k == g["sparse_kept"]                                   # 52,428: floor, not round
    assert O.param_count(0, m, n, r) == g["lowrank_params"]         # 2 x 1024 x 64
    assert O.param_count(k, m, n, r) == g["total_params"]           # 183,500
    assert round(O.compression_ratio(m, n, k, r), 1) == g["reduction_printed"]
    # 87 % residual footprint reduction: 131,072 factor entries replace the
    # m*n - k residual values.
    assert round(100 * (1 - g["lowrank_params"] / (m * n - k))) == g["residual_footprint_reduction_pct_printed"]
    # The printed residual count is off by 1,000 (typo on the page).
    assert m * n - k == 996148
    assert m * n - k - g["residual_count_printed"] == 1000


def test_rank_rule():
    g = _golden("rank_rule.json")
    assert O.rank_rule(g["dim"], g["dim"], *g["fraction"]) == g["rank"]
    # The decoder-layer workload's rank, 10 % of min(m, n) = 4096, floored.
    assert O.rank_rule(4096, 11008) == 409 == O.rank_rule(11008, 4096)


def test_topk_count_is_floor_in_integers():
    # 0.05 * 1048576 = 52428.8: floor, and exact (no binary 0.05).
    assert O.topk_count(1024, 1024, 5, 100) == 52428
    assert O.topk_count(4096, 4096, 5, 100) == 838860
    assert O.topk_count(4096, 4096, 3, 100) == 503316
    assert O.topk_count(11008, 4096, 3, 100) == 1352663
    assert O.topk_count(8192, 8192, 3, 100) == 2013265
    assert O.topk_count(3, 3, 1, 3) == 3
    assert O.topk_count(7, 1, 0, 100) == 0


def test_csr1024_oracle_reproduces_worked_example():
    """The first workload is the worked example's shape: the oracle's split and
    factor shapes must give the printed parameter total."""
    cfg = syn.WORKLOADS["csr1024_f32"]
    W = syn.weight(cfg)
    m, n = W.shape
    k = O.topk_count(m, n, *cfg.frac)
    s = O.split_csr(W, O.F32, k)
    assert int(s["row_ptr"][-1]) == len(s["col_idx"]) == 52428
    nnz_res = int(np.count_nonzero(~s["mask"]))
    assert nnz_res == 996148
    assert O.param_count(len(s["values"]), m, n, cfg.rank[0]) == 183500


# ---------------------------------------------------------------------------
# Stage 1: top-k by magnitude
# ---------------------------------------------------------------------------

def _brute_topk(W, dtype, k):
    m, n = W.shape
    vals = O.widen(W, dtype).reshape(-1)
    keys = [abs(float(v)) for v in vals]
    order = sorted(range(m * n), key=lambda t: (-keys[t], t))
    mask = np.zeros(m * n, dtype=bool)
    for t in order[:k]:
        mask[t] = True
    return mask.reshape(m, n)


@pytest.mark.parametrize("kind", ["t3", "ties", "equal", "zeros", "ints"])
@pytest.mark.parametrize("dtype", [O.F32, O.BF16])
@pytest.mark.parametrize("shape", [(1, 1), (1, 6), (5, 1), (3, 4), (6, 6)])
def test_topk_matches_brute_force(kind, dtype, shape):
    m, n = shape
    W = syn.random_matrix(m, n, dtype, seed=11, kind=kind)
    for k in range(m * n + 1):
        assert np.array_equal(O.topk_mask(W, dtype, k), _brute_topk(W, dtype, k)), k


def test_topk_invariants_csr1024():
    cfg = syn.WORKLOADS["csr1024_f32"]
    W = syn.weight(cfg)
    k = O.topk_count(*W.shape, *cfg.frac)
    mask = O.topk_mask(W, O.F32, k)
    a = np.abs(W.astype(np.float64))
    assert mask.sum() == k
    assert a[mask].min() >= a[~mask].max()
    T = a[mask].min()
    flat_eq = np.flatnonzero((a == T).reshape(-1))
    kept_eq = np.flatnonzero((mask & (a == T)).reshape(-1))
    assert np.array_equal(kept_eq, flat_eq[: len(kept_eq)])        # lowest linear indices


def test_topk_tie_split_across_rows():
    # Every magnitude equal: S must be the first k row-major positions.
    W = syn.random_matrix(7, 5, O.BF16, seed=3, kind="equal")
    for k in (0, 1, 4, 5, 6, 17, 35):
        mask = O.topk_mask(W, O.BF16, k)
        assert np.array_equal(np.flatnonzero(mask.reshape(-1)), np.arange(k))


def test_topk_signed_zero_and_nonfinite():
    W = np.array([[-0.0, 0.0, 1.0]], dtype=np.float32)
    assert np.array_equal(O.topk_mask(W, O.F32, 2), [[True, False, True]])
    with pytest.raises(ValueError):
        O.topk_mask(np.array([[np.nan, 1.0]], dtype=np.float32), O.F32, 1)
    with pytest.raises(ValueError):
        O.topk_mask(np.array([[np.inf, 1.0]], dtype=np.float32), O.F32, 1)
    with pytest.raises(ValueError):
        O.topk_mask(np.zeros((2, 2), np.float32), O.F32, 5)


# ---------------------------------------------------------------------------
# CSR storage and the residual
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", [O.F32, O.BF16])
def test_csr_matches_scipy(dtype):
    W = syn.random_matrix(37, 53, dtype, seed=5, kind="t3")
    k = O.topk_count(37, 53, 5, 100)
    s = O.split_csr(W, dtype, k)
    dense = O.widen(W, dtype) * s["mask"]
    assert np.count_nonzero(dense) == k          # no kept zero, so scipy keeps all
    ref = scipy.sparse.csr_matrix(dense)
    ref.sort_indices()
    assert np.array_equal(s["row_ptr"], ref.indptr)
    assert np.array_equal(s["col_idx"], ref.indices)
    assert np.array_equal(O.widen(s["values"], dtype), ref.data)


@pytest.mark.parametrize("kind", ["t3", "ties", "zeros"])
def test_csr_roundtrip_and_residual(kind):
    dtype = O.BF16
    W = syn.random_matrix(19, 24, dtype, seed=2, kind=kind)
    k = 57
    s = O.split_csr(W, dtype, k)
    S = O.dense_from_csr(19, 24, s["row_ptr"], s["col_idx"], s["values"], dtype)
    R = O.widen(s["residual"], dtype)
    Wd = O.widen(W, dtype)
    assert np.array_equal(S + R, Wd)                     # R + S == W
    assert np.all(s["residual"][s["mask"]] == 0)         # +0 bits on supp(S)
    assert O.bits_equal(s["residual"][~s["mask"]], W[~s["mask"]])
    assert len(s["values"]) == k
    assert O.bits_equal(s["values"], W[s["mask"]])       # bits copied (sign of zeros too)
    for i in range(19):                                  # ascending columns within rows
        c = s["col_idx"][s["row_ptr"][i]:s["row_ptr"][i + 1]]
        assert np.all(np.diff(c) > 0)


# ---------------------------------------------------------------------------
# Stage 1, 2:4 form
# ---------------------------------------------------------------------------

def _brute_pair(mags):
    """Lexicographically smallest pair (i0 < i1) with every kept |w| >= every dropped |w|."""
    for i0, i1 in itertools.combinations(range(4), 2):
        kept = [mags[i0], mags[i1]]
        dropped = [mags[t] for t in range(4) if t not in (i0, i1)]
        if min(kept) >= max(dropped):
            return i0, i1
    raise AssertionError("no valid pair")


@pytest.mark.parametrize("kind", ["t3", "ties", "equal", "zeros", "ints"])
@pytest.mark.parametrize("dtype", [O.F32, O.BF16])
def test_nm24_matches_brute_force(kind, dtype):
    m, n = 9, 40
    W = syn.random_matrix(m, n, dtype, seed=8, kind=kind)
    s = O.split_24(W, dtype)
    a = np.abs(O.widen(W, dtype))
    for i in range(m):
        for g in range(n // 4):
            i0, i1 = _brute_pair(list(a[i, 4 * g:4 * g + 4]))
            expect = np.zeros(4, bool)
            expect[[i0, i1]] = True
            assert np.array_equal(s["mask"][i, 4 * g:4 * g + 4], expect)
            nib = (int(s["nm_meta"][i, g // 8]) >> (4 * (g % 8))) & 0xF
            assert nib == i0 | (i1 << 2)
    S = O.dense_from_24(m, n, s["nm_values"], s["nm_meta"], dtype)
    assert np.array_equal(S + O.widen(s["residual"], dtype), O.widen(W, dtype))
    assert np.all((S != 0).reshape(m, n // 4, 4).sum(-1) <= 2)


def test_nm24_hand_row():
    g = _golden("nm24_hand_row.json")
    W = np.array([g["row"]], dtype=np.float32)
    s = O.split_24(W, O.F32)
    assert s["nm_meta"].shape == (1, 1)
    assert int(s["nm_meta"][0, 0]) == g["meta_word"] == int(g["meta_word_hex"], 16)
    assert np.array_equal(s["nm_values"][0], np.array(g["values"], dtype=np.float32))


def test_nm24_partial_meta_word():
    # n = 36: 9 groups, two meta words; the unused nibbles of word 1 are zero.
    W = syn.random_matrix(3, 36, O.BF16, seed=1, kind="t3")
    s = O.split_24(W, O.BF16)
    assert s["nm_meta"].shape == (3, 2)
    assert np.all((s["nm_meta"][:, 1] >> 4) == 0)


# ---------------------------------------------------------------------------
# Stage 2: truncated SVD
# ---------------------------------------------------------------------------

def _orthonormal(rng, m, k):
    q, _ = np.linalg.qr(rng.standard_normal((m, k)))
    return q


def test_svd_eckart_young_and_orthonormality():
    W = syn.random_matrix(80, 60, O.F32, seed=4, kind="t3")
    k = O.topk_count(80, 60, 5, 100)
    R = O.widen(O.split_csr(W, O.F32, k)["residual"], O.F32)
    for r in (0, 1, 7, 60):
        U, V, s = O.truncated_svd(R, r)
        assert U.shape == (80, r) and V.shape == (60, r)
        err = np.linalg.norm(R - U @ V.T)
        expect = np.sqrt(np.sum(s[r:] ** 2))
        assert abs(err - expect) <= 1e-10 * max(expect, 1e-300) + 1e-13
        assert np.max(np.abs(V.T @ V - np.eye(r)), initial=0) <= 1e-12
        for l in range(r):                        # sign rule
            j = int(np.argmax(np.abs(V[:, l])))
            assert V[j, l] > 0
    s2 = scipy.linalg.svd(R, compute_uv=False, lapack_driver="gesvd")
    assert np.max(np.abs(s - s2)) <= 1e-12 * s[0]


def test_svd_recovers_known_spectrum():
    rng = np.random.default_rng(0)
    m, n, true = 50, 30, np.array([9.0, 5.0, 4.0, 1.5, 0.25])
    A = _orthonormal(rng, m, 5) @ np.diag(true) @ _orthonormal(rng, n, 5).T
    U, V, s = O.truncated_svd(A, 5)
    assert np.allclose(s[:5], true, rtol=0, atol=1e-12)
    assert np.max(np.abs(s[5:])) <= 1e-12
    assert np.max(np.abs(A - U @ V.T)) <= 1e-12                   # exact for a rank-5 matrix
    U2, V2, _ = O.truncated_svd(A, 2)                              # best rank 2 drops 4.0, 1.5, 0.25
    assert abs(np.linalg.norm(A - U2 @ V2.T) - np.sqrt(4.0**2 + 1.5**2 + 0.25**2)) <= 1e-12


# ---------------------------------------------------------------------------
# Apply: factored vs dense, special cases, hand example
# ---------------------------------------------------------------------------

def _tiny_problem(seed, m=6, n=8, r=3, b=4, k=10):
    rng = np.random.default_rng(seed)
    W = syn.random_matrix(m, n, O.F32, seed=seed, kind="t3")
    s = O.split_csr(W, O.F32, k)
    S = O.dense_from_csr(m, n, s["row_ptr"], s["col_idx"], s["values"], O.F32)
    return s, S, rng.standard_normal((m, r)), rng.standard_normal((n, r)), rng.standard_normal((b, n))


def test_apply_hand_example():
    g = _golden("apply_hand_2x3.json")
    S, U, V, X = (np.array(g[t], dtype=np.float64) for t in ("S", "U", "V", "X"))
    assert np.array_equal(O.apply_factored(S, U, V, X), np.array(g["Y"]))
    assert np.array_equal(O.apply_dense(S, U, V, X), np.array(g["Y"]))
    assert np.array_equal(O.normaliser(S, U, V, X), np.array(g["N"]))


@pytest.mark.parametrize("seed", range(5))
def test_apply_factored_equals_dense(seed):
    _, S, U, V, X = _tiny_problem(seed)
    N = O.normaliser(S, U, V, X)
    d = np.abs(O.apply_factored(S, U, V, X) - O.apply_dense(S, U, V, X))
    assert np.all(d <= 1e-12 * N)


def test_apply_rank0_is_scipy_spmv():
    s, S, U, V, X = _tiny_problem(7)
    U0, V0 = U[:, :0], V[:, :0]
    csr = scipy.sparse.csr_matrix((O.widen(s["values"], O.F32), s["col_idx"], s["row_ptr"]), shape=S.shape)
    ref = np.stack([csr @ x for x in X])
    assert np.allclose(O.apply_factored(S, U0, V0, X), ref, rtol=1e-14, atol=1e-15)


def test_apply_k0_is_pure_low_rank_loops():
    _, S, U, V, X = _tiny_problem(9)
    Z = np.zeros_like(S)
    Y = O.apply_factored(Z, U, V, X)
    b, n = X.shape
    m, r = U.shape
    for c in range(b):
        for i in range(m):
            acc = sum(U[i, l] * sum(V[j, l] * X[c, j] for j in range(n)) for l in range(r))
            assert abs(Y[c, i] - acc) <= 1e-12 * (1 + abs(acc))


def test_apply_unit_vector_returns_column():
    _, S, U, V, _ = _tiny_problem(3)
    A = S + U @ V.T
    n = S.shape[1]
    for j in range(n):
        e = np.zeros((1, n))
        e[0, j] = 1.0
        assert np.allclose(O.apply_factored(S, U, V, e)[0], A[:, j], rtol=1e-14, atol=1e-15)


def test_normaliser_loop_definition():
    _, S, U, V, X = _tiny_problem(2)
    A = S + U @ V.T
    N = O.normaliser(S, U, V, X)
    for c in range(X.shape[0]):
        for i in range(S.shape[0]):
            assert abs(N[c, i] - sum(abs(A[i, j] * X[c, j]) for j in range(S.shape[1]))) <= 1e-13


@pytest.mark.parametrize("seed,r", [(11, 3), (12, 0)])
def test_apply_csr_equals_the_hand_loop(seed, r):
    """The CSR-form apply against the definition written out as loops: for
    each output, the stored entries of row i times X, plus sum_l U[i, l] (V^T x)_l."""
    s, S, U, V, X = _tiny_problem(seed, m=7, n=9, r=max(r, 1), b=2, k=15)
    U, V = U[:, :r], V[:, :r]
    m, n = S.shape
    Y = O.apply_csr(m, n, s["row_ptr"], s["col_idx"], s["values"], O.F32, U, V, X)
    vals = O.widen(s["values"], O.F32)
    for c in range(X.shape[0]):
        for i in range(m):
            acc = sum(vals[p] * X[c, s["col_idx"][p]] for p in range(s["row_ptr"][i], s["row_ptr"][i + 1]))
            acc += sum(U[i, l] * sum(V[j, l] * X[c, j] for j in range(n)) for l in range(r))
            assert abs(Y[c, i] - acc) <= 1e-12 * (1 + abs(acc))


def test_apply_rows_matches_full():
    s, S, U, V, X = _tiny_problem(4, m=9, n=12, r=2, b=3, k=20)
    rows = np.array([0, 4, 8])
    Srows = O.csr_rows_dense(rows, 12, s["row_ptr"], s["col_idx"], s["values"], O.F32)
    Yr, Nr = O.apply_rows(Srows, U[rows], V, X)
    assert np.allclose(Yr, O.apply_factored(S, U, V, X)[:, rows], rtol=1e-13, atol=1e-15)
    assert np.allclose(Nr, O.normaliser(S, U, V, X)[:, rows], rtol=1e-13, atol=1e-15)


def test_max_normalised_error_rules():
    N = np.array([[1.0, 0.0]])
    assert O.max_normalised_error(np.array([[1.5, 0.0]]), np.array([[1.0, 0.0]]), N) == 0.5
    assert O.max_normalised_error(np.array([[1.0, 1e-30]]), np.array([[1.0, 0.0]]), N) == float("inf")


# ---------------------------------------------------------------------------
# Storage narrowing: RNE against an independent implementation (torch)
# ---------------------------------------------------------------------------

def test_bf16_narrowing_matches_torch():
    import torch
    rng = np.random.default_rng(1)
    a = np.concatenate([rng.standard_normal(5000) * 10.0 ** rng.integers(-30, 30, 5000),
                        [0.0, -0.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -9, -1.5,
                         3.0e38, 1e-40]])
    mine = O.narrow(a, O.BF16)
    ref = torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)
    assert np.array_equal(syn.f32_to_bf16_bits(a.astype(np.float32)), ref)
    assert np.array_equal(O.widen(mine, O.BF16), torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).double().numpy())


# ---------------------------------------------------------------------------
# Dense-and-sparse variant (SqueezeLLM explainer, section "3.中核となる技術的要素")
# ---------------------------------------------------------------------------

def test_kmeans_hand_tie_rule():
    g = json.load(open(os.path.join(GOLDEN, "kmeans_hand.json")))
    c, codes = O.kmeans_1d(np.array(g["values"], dtype=np.float64), g["K"])
    assert np.allclose(c, g["centroids"], rtol=0, atol=1e-15)
    assert codes.tolist() == g["codes"]


def test_kmeans_recovers_separated_clusters():
    """16 tight, equally large clusters far apart (all values distinct): each
    starting quantile falls in its own cluster, so the levels are the cluster means and the codes the
    cluster labels (centres ascending).  (With unequal sizes Lloyd's algorithm
    may settle with two levels in one cluster: a local optimum.)"""
    rng = np.random.default_rng(7)
    centres = np.arange(16) * 10.0 - 75.0
    sizes = np.full(16, 7)
    vals, labels = [], []
    for k, (c0, sz) in enumerate(zip(centres, sizes)):
        vals.append(c0 + rng.uniform(-0.1, 0.1, size=sz))
        labels.append(np.full(sz, k))
    vals, labels = np.concatenate(vals), np.concatenate(labels)
    perm = rng.permutation(vals.size)
    vals, labels = vals[perm], labels[perm]
    c, codes = O.kmeans_1d(vals, 16)
    assert np.array_equal(codes, labels)
    for k in range(16):
        assert abs(c[k] - vals[labels == k].sum() / (labels == k).sum()) < 1e-12


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_kmeans_fixed_point_and_not_worse_than_start(seed):
    rng = np.random.default_rng(seed)
    v = rng.standard_t(3, size=300) * 0.02
    K = 16
    c, codes = O.kmeans_1d(v, K)
    d = np.abs(v[:, None] - c[None, :])
    # every value sits at a nearest level, the first one on ties
    assert np.all(d[np.arange(v.size), codes] <= d.min(axis=1))
    first = np.array([int(np.flatnonzero(row == row.min())[0]) for row in d])
    assert np.array_equal(codes, first)
    # every non-empty level is the mean of its values
    for k in range(K):
        if np.any(codes == k):
            assert abs(c[k] - np.sum(v[codes == k]) / np.sum(codes == k)) < 1e-15 + 1e-12 * abs(c[k])
    # Lloyd never increases the squared error of its starting quantiser
    u = np.unique(v)
    c0 = u[[(2 * k + 1) * u.size // (2 * K) for k in range(K)]]
    sse0 = np.sum(np.min((v[:, None] - c0[None, :]) ** 2, axis=1))
    sse = np.sum((v - c[codes]) ** 2)
    assert sse <= sse0 + 1e-18


@pytest.mark.parametrize("dtype", [O.F32, O.BF16])
def test_quantize_rows_codes_are_nearest_stored_level(dtype):
    W = syn.random_matrix(24, 64, dtype, seed=5, kind="t3")
    lut, codes = O.quantize_rows(W, dtype, 4)
    L, D = O.widen(lut, dtype), O.widen(W, dtype)
    for i in range(W.shape[0]):
        d = np.abs(D[i][:, None] - L[i][None, :])
        first = np.array([int(np.flatnonzero(row == row.min())[0]) for row in d])
        assert np.array_equal(codes[i].astype(np.int64), first)


def test_quantize_rows_few_distinct_values_is_exact():
    rng = np.random.default_rng(3)
    levels = np.sort(rng.standard_normal(16)).astype(np.float32)
    W = levels[rng.integers(0, 16, size=(10, 48))]
    W[0, :] = levels[3]                 # a row with one distinct value
    W[1, :] = levels[rng.integers(0, 5, size=48)]
    lut, codes = O.quantize_rows(W, O.F32, 4)
    assert O.bits_equal(O.narrow(O.dense_from_codes(codes, lut, O.F32), O.F32), W)


def test_pack_nibbles_hand_and_roundtrip():
    g = json.load(open(os.path.join(GOLDEN, "dq4_pack_hand.json")))
    packed = O.pack_nibbles(np.array([g["codes"]], dtype=np.uint8))
    assert packed[0].tolist() == g["bytes"]
    rng = np.random.default_rng(1)
    codes = rng.integers(0, 16, size=(5, 38)).astype(np.uint8)
    assert np.array_equal(O.unpack_nibbles(O.pack_nibbles(codes), 38), codes)


def test_dense_sparse_split_invariants():
    assert O.outlier_count(4096, 4096) == 83886     # 0.5 % of 16,777,216, floored
    W = syn.random_matrix(40, 64, O.BF16, seed=11, kind="t3")
    d = O.split_dense_sparse(W, O.BF16)
    k = O.outlier_count(40, 64)
    assert k == 12 and len(d["col_idx"]) == k
    S = O.dense_from_csr(40, 64, d["row_ptr"], d["col_idx"], d["values"], O.BF16)
    R = O.widen(d["residual"], O.BF16)
    assert np.array_equal(S + R, O.widen(W, O.BF16))             # W = S + D exactly
    a = np.abs(O.widen(W, O.BF16))
    assert a[S != 0].min() >= a[S == 0].max() if np.any(S != 0) else True
    assert d["codes"].max() < 16 and d["codes_packed"].shape == (40, 32)


def test_dense_sparse_apply_histogram_form():
    """y_i = sum_k lut[i, k] * (sum of x_j over the columns j coded k) + (S x)_i:
    the grouped sum equals the dense product with the dequantised D."""
    m, n = 12, 40
    W = syn.random_matrix(m, n, O.F32, seed=4, kind="t3")
    d = O.split_dense_sparse(W, O.F32)
    X = syn.random_matrix(3, n, O.F32, seed=6, kind="normal", scale=1.0).astype(np.float64)
    S = O.dense_from_csr(m, n, d["row_ptr"], d["col_idx"], d["values"], O.F32)
    Dq = O.dense_from_codes(d["codes"], d["lut"], O.F32)
    Y = O.apply_factored(S + Dq, np.zeros((m, 0)), np.zeros((n, 0)), X)
    L = O.widen(d["lut"], O.F32)
    for c in range(3):
        for i in range(m):
            grouped = sum(L[i, k] * X[c, d["codes"][i] == k].sum() for k in range(16))
            sparse = sum(S[i, j] * X[c, j] for j in range(n))
            assert abs(Y[c, i] - (grouped + sparse)) <= 1e-12 * (1 + abs(Y[c, i]))


# ---------------------------------------------------------------------------
# Hierarchical variant ([HSS] section "順列と階層的整列")
# ---------------------------------------------------------------------------

def test_concentration_ratio_closed_forms():
    # constant blocks: diagonal quadrants |a|, off-diagonal |b| -> rho = (m1 n1 + m2 n2) a / (that + rest)
    m, n = 7, 5
    m1, n1 = 3, 2
    W = np.full((m, n), -3.0, dtype=np.float32)
    W[:m1, :n1] = 2.0
    W[m1:, n1:] = 2.0
    diag = 2.0 * (m1 * n1 + (m - m1) * (n - n1))
    off = 3.0 * (m1 * (n - n1) + (m - m1) * n1)
    assert abs(O.concentration_ratio(W, O.F32) - diag / (diag + off)) < 1e-15
    # block-diagonal -> 1; all zero -> 0
    B = np.zeros((6, 6), dtype=np.float32)
    B[:3, :3] = 1.5
    B[3:, 3:] = -0.5
    assert O.concentration_ratio(B, O.F32) == 1.0
    assert O.concentration_ratio(np.zeros((4, 4), np.float32), O.F32) == 0.0
    # a scrambled matrix measured in the order that unscrambles it
    sigma = np.random.default_rng(2).permutation(6)
    Wsc = B[np.argsort(sigma)][:, np.argsort(sigma)]   # Wsc[sigma[i], sigma[j]] = B[i, j]
    assert O.concentration_ratio(Wsc, O.F32, perm=sigma) == 1.0


def test_rcm_hand_example():
    g = json.load(open(os.path.join(GOLDEN, "rcm_hand.json")))
    assert O.rcm_order(g["n"], g["row_ptr"], g["col_idx"]).tolist() == g["perm"]


def _csr_of_edges(n, edges):
    rows = [[] for _ in range(n)]
    for a, b in edges:
        rows[a].append(b)
    rp, ci = [0], []
    for i in range(n):
        ci += sorted(rows[i])
        rp.append(len(ci))
    return rp, ci


@pytest.mark.parametrize("seed", range(4))
def test_rcm_recovers_a_scrambled_path(seed):
    n = 9 + seed
    q = np.random.default_rng(seed).permutation(n)
    rp, ci = _csr_of_edges(n, [(int(q[t]), int(q[t + 1])) for t in range(n - 1)])
    perm = O.rcm_order(n, rp, ci)
    assert sorted(perm.tolist()) == list(range(n))
    assert O.bandwidth(n, rp, ci, perm) == 1
    assert O.bandwidth(n, rp, ci) > 1


def test_rcm_keeps_components_contiguous():
    # two scrambled paths on interleaved node sets, plus an isolated node
    n = 11
    a, b = [0, 2, 4, 6, 8], [1, 3, 5, 7, 9]
    rp, ci = _csr_of_edges(n, [(a[t], a[t + 1]) for t in range(4)] + [(b[t + 1], b[t]) for t in range(4)])
    perm = O.rcm_order(n, rp, ci).tolist()
    pos = {v: i for i, v in enumerate(perm)}
    for comp in (a, b, [10]):
        ps = sorted(pos[v] for v in comp)
        assert ps == list(range(ps[0], ps[0] + len(comp)))
    assert O.bandwidth(n, rp, ci, np.array(perm)) == 1


def test_hier_full_rank_reproduces_residual_and_eckart_young():
    rng = np.random.default_rng(4)
    m = n = 13                                   # odd: blocks 6 and 7
    R = rng.standard_normal((m, n))
    full = O.hier_factors(R, 7, 7)
    assert np.max(np.abs(O.hier_lowrank_dense(full, None, m, n) - R)) < 1e-12
    low = O.hier_factors(R, 4, 2)
    rows, cols = [(0, 6), (6, 13)], [(0, 6), (6, 13)]
    for (bi, bj), (U, V) in low.items():
        blk = R[rows[bi][0]:rows[bi][1], cols[bj][0]:cols[bj][1]]
        r = 4 if bi == bj else 2
        assert U.shape == (blk.shape[0], r) and V.shape == (blk.shape[1], r)
        s = np.linalg.svd(blk, compute_uv=False)
        assert abs(np.linalg.norm(blk - U @ V.T) - np.sqrt(np.sum(s[r:] ** 2))) < 1e-10


def test_hier_param_count_hand_counts():
    """Hand-counted fixtures (the page's 512 x 512 block ranks, and odd sides)."""
    with open(os.path.join(GOLDEN, "hier_param_count_hand.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        assert O.hier_param_count(c["k"], c["m"], c["n"], c["r_diag"], c["r_off"]) == c["params"], c["note"]


@pytest.mark.parametrize("m,n,r_diag,r_off", [(9, 9, 3, 1), (7, 12, 2, 2), (12, 7, 3, 0), (2, 3, 1, 1)])
def test_hier_param_count_counts_the_stored_factors(m, n, r_diag, r_off):
    """Brute force: the entries of the factors hier_factors actually returns
    (every block's U and V), plus k, equal the count."""
    R = np.random.default_rng(m * 31 + n).standard_normal((m, n))
    blocks = O.hier_factors(R, r_diag, r_off)
    stored = sum(U.size + V.size for U, V in blocks.values())
    assert O.hier_param_count(5, m, n, r_diag, r_off) == 5 + stored


def test_bits_equal_compares_bit_patterns():
    """bits_equal is the checker behind every bitwise parity assertion, so its
    negative cases are pinned: patterns, not values, decide."""
    f = np.array([1.0, -2.5, 3.0], dtype=np.float32)
    assert O.bits_equal(f, f.copy())
    assert O.bits_equal(f, f.view(np.uint32))                     # same bits, another view
    assert not O.bits_equal(np.array([0.0], np.float32), np.array([-0.0], np.float32))   # +0 vs -0
    qnan = np.array([0x7FC00000], np.uint32).view(np.float32)
    pnan = np.array([0x7FC00001], np.uint32).view(np.float32)
    assert O.bits_equal(qnan, qnan.copy())                         # the same NaN pattern
    assert not O.bits_equal(qnan, pnan)                            # NaN payloads differ
    g = f.copy()
    g.view(np.uint32)[1] ^= 1                                      # one bit of one element
    assert not O.bits_equal(f, g)
    assert not O.bits_equal(f, f[:2])                              # shape
    assert not O.bits_equal(f.reshape(3, 1), f.reshape(1, 3))      # shape, same size
    assert not O.bits_equal(f, f.astype(np.float64))               # element width
    h = np.array([0x3F80, 0x8000], np.uint16)                      # bf16 patterns 1.0, -0
    assert O.bits_equal(h, h.copy())
    assert not O.bits_equal(h, np.array([0x3F80, 0x0000], np.uint16))
    assert not O.bits_equal(h, np.array([0x3F80, 0x8001], np.uint16))


@pytest.mark.parametrize("permuted", [False, True])
def test_hier_apply_equals_dense(permuted):
    rng = np.random.default_rng(8)
    m = n = 11
    S = np.where(rng.random((m, n)) < 0.2, rng.standard_normal((m, n)), 0.0)
    R = rng.standard_normal((m, n))
    perm = rng.permutation(n) if permuted else None
    Rp = R if perm is None else R[perm][:, perm]
    blocks = O.hier_factors(Rp, 3, 1)
    X = rng.standard_normal((4, n))
    A = S + O.hier_lowrank_dense(blocks, perm, m, n)
    Y = O.hier_apply(S, blocks, perm, X)
    assert np.max(np.abs(Y - X @ A.T)) < 1e-12 * (1 + np.max(np.abs(Y)))
    # with full ranks the permuted low-rank term is R itself, back in the original order
    fullb = O.hier_factors(Rp, 6, 6)
    assert np.max(np.abs(O.hier_lowrank_dense(fullb, perm, m, n) - R)) < 1e-12


# ---------------------------------------------------------------------------
# Backward: gradients of S (on its support), U, V and the input
# ---------------------------------------------------------------------------

def _bw_case(m=7, n=9, r=3, b=4, density=0.3, seed=0):
    rng = np.random.default_rng(seed)
    mask = rng.random((m, n)) < density
    S = np.where(mask, rng.standard_normal((m, n)), 0.0)
    rows, cols = np.nonzero(mask)
    row_ptr = np.concatenate([[0], np.cumsum(np.bincount(rows, minlength=m))]).astype(np.int32)
    return (row_ptr, cols.astype(np.int32), S, rng.standard_normal((m, r)), rng.standard_normal((n, r)),
            rng.standard_normal((b, n)), rng.standard_normal((b, m)))


def _loss(G, S, U, V, X):
    return float(np.sum(G * O.apply_factored(S, U, V, X)))


@pytest.mark.parametrize("seed", [0, 1])
def test_backward_matches_exact_finite_differences(seed):
    """L = sum(G * Y) is linear in each of S's stored values, U, V and X, so
    L(theta + E) - L(theta) = <grad, E> exactly (up to rounding), with L
    evaluated through the forward apply."""
    m, n = 7, 9
    rp, ci, S, U, V, X, G = _bw_case(m, n, seed=seed)
    g = O.backward(m, n, rp, ci, S, U, V, X, G)
    rng = np.random.default_rng(100 + seed)
    L0 = _loss(G, S, U, V, X)
    rows = O.csr_row_of_entry(m, rp)
    Es = rng.standard_normal(len(ci))
    S2 = S.copy()
    S2[rows, ci] += Es
    for delta, expect in (
        (_loss(G, S2, U, V, X) - L0, g["dS"] @ Es),
        (_loss(G, S, U + (EU := rng.standard_normal(U.shape)), V, X) - L0, np.sum(g["dU"] * EU)),
        (_loss(G, S, U, V + (EV := rng.standard_normal(V.shape)), X) - L0, np.sum(g["dV"] * EV)),
        (_loss(G, S, U, V, X + (EX := rng.standard_normal(X.shape))) - L0, np.sum(g["dX"] * EX)),
    ):
        assert abs(delta - expect) <= 1e-9 * (1 + abs(expect))


def test_backward_euler_identities():
    """Each part of L is homogeneous of degree 1 in each parameter: <dS, s> is
    the sparse part of L, <dU, U> = <dV, V> its low-rank part, <dX, X> all of it."""
    m, n = 6, 11
    rp, ci, S, U, V, X, G = _bw_case(m, n, r=4, b=5, seed=3)
    g = O.backward(m, n, rp, ci, S, U, V, X, G)
    Ls = float(np.sum(G * (X @ S.T)))
    Ll = float(np.sum(G * ((X @ V) @ U.T)))
    vals = S[O.csr_row_of_entry(m, rp), ci]
    assert np.isclose(g["dS"] @ vals, Ls, rtol=1e-12, atol=1e-12)
    assert np.isclose(np.sum(g["dU"] * U), Ll, rtol=1e-12, atol=1e-12)
    assert np.isclose(np.sum(g["dV"] * V), Ll, rtol=1e-12, atol=1e-12)
    assert np.isclose(np.sum(g["dX"] * X), Ls + Ll, rtol=1e-12, atol=1e-12)


def test_backward_one_hot_upstream_and_full_support_brute_force():
    """G = one entry (c, i): dX is row i of A in batch row c only, dU is X_c V in
    row i only, dV is X_c^T U_i.  With every position stored, dS is the
    brute-force double loop sum_c G_ci X_cj."""
    m, n, b = 5, 4, 3
    rp, ci, S, U, V, X, _ = _bw_case(m, n, b=b, density=1.1, seed=4)   # every position stored
    G = np.zeros((b, m))
    G[1, 3] = 1.0
    g = O.backward(m, n, rp, ci, S, U, V, X, G)
    A = S + U @ V.T
    expect_dX = np.zeros((b, n))
    expect_dX[1] = A[3]
    assert np.allclose(g["dX"], expect_dX, rtol=0, atol=1e-14)
    expect_dU = np.zeros_like(U)
    expect_dU[3] = X[1] @ V
    assert np.allclose(g["dU"], expect_dU, rtol=0, atol=1e-14)
    assert np.allclose(g["dV"], np.outer(X[1], U[3]), rtol=0, atol=1e-14)
    G = np.random.default_rng(5).standard_normal((b, m))
    g = O.backward(m, n, rp, ci, S, U, V, X, G)
    brute = [sum(G[c, i] * X[c, j] for c in range(b)) for i in range(m) for j in range(n)]
    assert np.allclose(g["dS"], brute, rtol=1e-13, atol=1e-13)


def test_backward_normalisers_bound_the_gradients():
    m, n = 8, 6
    rp, ci, S, U, V, X, G = _bw_case(m, n, seed=6)
    g = O.backward(m, n, rp, ci, S, U, V, X, G)
    N = O.backward_normalisers(m, n, rp, ci, S, U, V, X, G)
    for k in g:
        assert np.all(np.abs(g[k]) <= N[k] * (1 + 1e-12) + 1e-15), k
    # with nonnegative inputs there is no cancellation: the bound is attained
    p = [np.abs(a) for a in (S, U, V, X, G)]
    g = O.backward(m, n, rp, ci, *p)
    N = O.backward_normalisers(m, n, rp, ci, *p)
    for k in g:
        assert np.allclose(g[k], N[k], rtol=1e-12), k


def test_csr_transpose_is_the_transposed_matrix():
    m, n = 9, 7
    rp, ci, S, *_ = _bw_case(m, n, density=0.4, seed=7)
    vals = S[O.csr_row_of_entry(m, rp), ci]
    rpt, cit, perm = O.csr_transpose(m, n, rp, ci)
    St = np.zeros((n, m))
    for j in range(n):
        seg = slice(rpt[j], rpt[j + 1])
        assert np.all(np.diff(cit[seg]) > 0)                         # original rows ascending
        St[j, cit[seg]] = vals[perm][seg]
    assert np.array_equal(St, S.T)
    assert sorted(perm.tolist()) == list(range(len(ci)))


def test_csr_permute_hand_example():
    """3 x 3 pattern, perm = [2, 0, 1] (so pos = [1, 2, 0]), worked by hand
    from S'[i][j] = S[perm[i]][perm[j]]: entries p0 (0,0), p1 (0,2), p2 (1,1),
    p3 (2,0), p4 (2,1) of S become row 0 = S's row 2 at columns pos[0] = 1,
    pos[1] = 2; row 1 = S's row 0 at pos[2] = 0, pos[0] = 1; row 2 = S's row
    1 at pos[1] = 2."""
    rp, ci, src = O.csr_permute(3, [0, 2, 3, 5], [0, 2, 1, 0, 1], [2, 0, 1])
    assert rp.tolist() == [0, 2, 4, 5]
    assert ci.tolist() == [1, 2, 0, 1, 2]
    assert src.tolist() == [3, 4, 1, 0, 2]


@pytest.mark.parametrize("n,density,seed", [(1, 1.0, 0), (6, 0.5, 1), (17, 0.2, 2), (40, 0.05, 3), (9, 0.0, 4)])
def test_csr_permute_is_the_permuted_matrix(n, density, seed):
    """Brute force: the permuted pattern with the values moved by src is
    W[perm][:, perm] of the dense matrix; columns ascend in every row; src is
    a permutation; permuting back by the inverse returns S exactly."""
    rng = np.random.default_rng(seed)
    D = np.where(rng.random((n, n)) < density, rng.standard_normal((n, n)), 0.0)
    rp = np.concatenate([[0], np.cumsum((D != 0).sum(axis=1))]).astype(np.int32)
    ci = np.nonzero(D)[1].astype(np.int32)
    vals = D[np.nonzero(D)]
    perm = rng.permutation(n)
    prp, pci, src = O.csr_permute(n, rp, ci, perm)
    Dp = np.zeros((n, n))
    for i in range(n):
        seg = slice(prp[i], prp[i + 1])
        assert np.all(np.diff(pci[seg]) > 0)
        Dp[i, pci[seg]] = vals[src[seg]]
    assert np.array_equal(Dp, D[perm][:, perm])
    assert sorted(src.tolist()) == list(range(len(ci)))
    inv = np.argsort(perm)
    brp, bci, bsrc = O.csr_permute(n, prp, pci, inv)
    assert np.array_equal(brp, rp) and np.array_equal(bci, ci) and np.array_equal(src[bsrc], np.arange(len(ci)))


def test_backward_sampled_equals_full():
    m, n = 10, 8
    rp, ci, S, U, V, X, G = _bw_case(m, n, r=3, b=6, seed=8)
    g = O.backward(m, n, rp, ci, S, U, V, X, G)
    N = O.backward_normalisers(m, n, rp, ci, S, U, V, X, G)
    rows, cols = np.array([0, 3, 9]), np.array([1, 7])
    er = O.csr_row_of_entry(m, rp)
    pick = np.array([0, len(ci) // 2, len(ci) - 1])
    smp = O.backward_sampled(rows, cols, er[pick], ci[pick], U, V, X, G)
    assert np.allclose(smp["dU"], g["dU"][rows], rtol=1e-12, atol=1e-12)
    assert np.allclose(smp["dV"], g["dV"][cols], rtol=1e-12, atol=1e-12)
    assert np.allclose(smp["dS"], g["dS"][pick], rtol=1e-12, atol=1e-12)
    assert np.allclose(smp["NU"], N["dU"][rows]) and np.allclose(smp["NV"], N["dV"][cols])
    assert np.allclose(smp["NS"], N["dS"][pick])


def test_nm24_pattern_is_the_mask_in_storage_order():
    """The 2:4 pattern as CSR: the kept positions row-major (ascending within
    each group), and with the stored values it rebuilds the same matrix."""
    W = syn.random_matrix(6, 40, O.BF16, seed=21, kind="ties")
    s = O.split_24(W, O.BF16)
    rp, ci = O.nm24_pattern(6, 40, s["nm_meta"])
    rows, cols = np.nonzero(s["mask"])
    assert np.array_equal(rp, np.arange(7) * 20)
    assert np.array_equal(ci, cols) and np.array_equal(O.csr_row_of_entry(6, rp), rows)
    assert np.array_equal(O.dense_from_csr(6, 40, rp, ci, s["nm_values"].reshape(-1), O.BF16),
                          O.dense_from_24(6, 40, s["nm_values"], s["nm_meta"], O.BF16))


def test_svd_factor_cache_matches_its_manifest():
    """The full-size factors the GPU parity tests use (written by
    tests/golden/make_svd_factors.py from oracle calls only): each entry's
    Eckart-Young check held when it was written, the singular values it
    recorded are ordered, and the cached files hash to the manifest."""
    import hashlib
    man = _golden("svd_factors_manifest.json")
    cache = os.path.join(os.path.dirname(GOLDEN), "_svd_cache")
    assert len(man["entries"]) == 10
    for name, e in man["entries"].items():
        assert abs(e["eckart_young_lhs"] - e["eckart_young_rhs"]) <= 1e-9 * e["eckart_young_rhs"], name
        assert e["sigma_r_minus_1"] >= e["sigma_r"] > 0, name
        key, which = name.rsplit(".", 1)
        cfg = syn.WORKLOADS[key]
        assert (e["m"], e["n"]) == cfg.shapes[int(which)] and e["r"] == cfg.rank[int(which)]
        if not os.path.isdir(cache):
            continue
        for part, shape in (("U", (e["m"], e["r"])), ("V", (e["n"], e["r"]))):
            a = np.load(os.path.join(cache, f"{name}.{part}.npy"), allow_pickle=False)
            assert a.shape == shape and a.dtype == np.uint16
            if not os.path.exists(os.path.join(cache, f"{name}.rebuilt")):
                assert hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest() == e[f"sha256_{part}"]
