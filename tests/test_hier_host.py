"""The library's Reverse Cuthill-McKee order (host code, no GPU needed) is
bit-identical to the oracle's on hand, structured and random patterns, and
rejects bad arguments before doing anything."""
import json
import os

import numpy as np
import pytest

import hss_synth as syn
import oracle as O
from conftest import GOLDEN


@pytest.fixture(scope="module")
def H():
    import sparse_rank_linear_hss_amd as h
    return h


def _csr(mask):
    rows, cols = np.nonzero(mask)
    rp = np.zeros(mask.shape[0] + 1, dtype=np.int32)
    np.add.at(rp, rows + 1, 1)
    return np.cumsum(rp).astype(np.int32), cols.astype(np.int32)


def test_rcm_hand(H):
    g = json.load(open(os.path.join(GOLDEN, "rcm_hand.json")))
    assert H.hss_rcm_order(g["row_ptr"], g["col_idx"], g["n"]).tolist() == g["perm"]


@pytest.mark.parametrize("n,density,seed", [(1, 0.0, 0), (5, 0.0, 1), (17, 0.1, 2), (60, 0.05, 3), (200, 0.02, 4),
                                            (301, 0.01, 5), (64, 0.5, 6)])
def test_rcm_matches_oracle_on_random_patterns(H, n, density, seed):
    rng = np.random.default_rng(seed)
    mask = rng.random((n, n)) < density
    if n > 3:
        mask[2, 2] = True                         # a self-loop (ignored)
    rp, ci = _csr(mask)
    assert np.array_equal(H.hss_rcm_order(rp, ci, n), O.rcm_order(n, rp, ci))


def test_rcm_matches_oracle_on_topk_support(H):
    W = syn.random_matrix(150, 150, O.BF16, seed=12, kind="t3")
    s = O.split_csr(W, O.BF16, O.topk_count(150, 150, 5, 100))
    perm = H.hss_rcm_order(s["row_ptr"], s["col_idx"], 150)
    assert np.array_equal(perm, O.rcm_order(150, s["row_ptr"], s["col_idx"]))
    assert sorted(perm.tolist()) == list(range(150))


def test_rcm_duplicate_entries_count_once(H):
    rp = np.array([0, 3, 4, 4], dtype=np.int32)
    ci = np.array([1, 1, 2, 2], dtype=np.int32)            # (0,1) twice, (1,2)
    assert np.array_equal(H.hss_rcm_order(rp, ci, 3), O.rcm_order(3, rp, ci))


def test_rcm_rejects_bad_arguments(H):
    import ctypes
    lib, INV = H._lib.lib, H._lib.HSS_ERR_INVALID_ARG
    perm = np.zeros(4, dtype=np.int32)

    def call(rp, ci, n):
        rp = np.asarray(rp, dtype=np.int32)
        ci = np.asarray(ci, dtype=np.int32)
        return lib.hss_rcm_order(n, rp.ctypes.data, ci.ctypes.data if ci.size else None, perm.ctypes.data)
    assert call([0, 1, 1], [1], 2) == 0
    assert call([0, 1, 1], [1], 0) == INV                  # n < 1
    assert call([1, 1, 1], [1], 2) == INV                  # row_ptr[0] != 0
    assert call([0, 2, 1], [1, 0], 2) == INV               # decreasing row_ptr
    assert call([0, 1, 1], [5], 2) == INV                  # column out of range
    assert call([0, 1, 1], [-1], 2) == INV
    assert lib.hss_rcm_order(2, None, None, perm.ctypes.data) == INV


@pytest.mark.parametrize("m,n,density,seed", [(1, 1, 1.0, 0), (7, 5, 0.4, 1), (60, 90, 0.05, 2), (300, 41, 0.2, 3),
                                              (33, 33, 0.0, 4)])
def test_csr_transpose_matches_oracle(H, m, n, density, seed):
    """The library's host transpose of a CSR pattern is the oracle's: same
    S^T pattern, same permutation (bit-exact)."""
    rng = np.random.default_rng(seed)
    mask = rng.random((m, n)) < density
    rp, ci = _csr(mask)
    rpt, cit, perm = H.hss_csr_transpose(rp, ci, m, n)
    ort, oct_, operm = O.csr_transpose(m, n, rp, ci)
    assert np.array_equal(rpt, ort) and np.array_equal(cit, oct_) and np.array_equal(perm, operm)


def test_csr_transpose_rejects_bad_arguments(H):
    lib, INV = H._lib.lib, H._lib.HSS_ERR_INVALID_ARG
    out = np.zeros(8, dtype=np.int32)

    def call(rp, ci, m, n):
        rp = np.asarray(rp, dtype=np.int32)
        ci = np.asarray(ci, dtype=np.int32)
        return lib.hss_csr_transpose(m, n, rp.ctypes.data, ci.ctypes.data, out.ctypes.data, out.ctypes.data,
                                     out.ctypes.data)
    assert call([0, 1, 2], [0, 1], 2, 2) == 0
    assert call([0, 1, 2], [0, 1], 0, 2) == INV
    assert call([0, 1, 2], [0, 1], 2, 0) == INV
    assert call([1, 1, 2], [0, 1], 2, 2) == INV
    assert call([0, 2, 1], [0, 1], 2, 2) == INV
    assert call([0, 1, 2], [0, 2], 2, 2) == INV                  # column outside [0, n)


@pytest.mark.parametrize("n,density,seed", [(1, 1.0, 0), (7, 0.4, 1), (90, 0.05, 2), (300, 0.03, 3), (33, 0.0, 4)])
def test_csr_permute_matches_oracle(H, n, density, seed):
    """The library's host P S P^T of a CSR pattern is the oracle's: same
    pattern, same source indices (bit-exact), for a random and the RCM
    permutation."""
    rng = np.random.default_rng(seed)
    rp, ci = _csr(rng.random((n, n)) < density)
    for perm in (rng.permutation(n).astype(np.int32), H.hss_rcm_order(rp, ci, n)):
        prp, pci, src = H.hss_csr_permute(rp, ci, perm, n)
        orp, oci, osrc = O.csr_permute(n, rp, ci, perm)
        assert np.array_equal(prp, orp) and np.array_equal(pci, oci) and np.array_equal(src, osrc)


def test_csr_permute_rejects_bad_arguments(H):
    lib, INV = H._lib.lib, H._lib.HSS_ERR_INVALID_ARG
    out = np.zeros(8, dtype=np.int32)

    def call(rp, ci, perm, n):
        rp, ci, perm = (np.asarray(a, dtype=np.int32) for a in (rp, ci, perm))
        return lib.hss_csr_permute(n, rp.ctypes.data, ci.ctypes.data, perm.ctypes.data, out.ctypes.data,
                                   out.ctypes.data, out.ctypes.data)
    assert call([0, 1, 2], [1, 0], [1, 0], 2) == 0
    assert call([0, 1, 2], [1, 0], [1, 0], 0) == INV             # n < 1
    assert call([1, 1, 2], [1, 0], [1, 0], 2) == INV             # row_ptr[0] != 0
    assert call([0, 2, 1], [1, 0], [1, 0], 2) == INV             # decreasing row_ptr
    assert call([0, 1, 2], [2, 0], [1, 0], 2) == INV             # column outside [0, n)
    assert call([0, 1, 2], [1, 0], [1, 1], 2) == INV             # not a permutation
    assert call([0, 1, 2], [1, 0], [0, 2], 2) == INV
    assert call([0, 2, 2], [1, 1], [0, 1], 2) == INV             # a repeated column
    assert lib.hss_csr_permute(2, None, None, None, None, None, None) == INV
