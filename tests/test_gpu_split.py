"""GPU parity of hss_split against the CPU oracle: bit-exact row pointers,
column indices, values, 2:4 metadata and residual."""
import numpy as np
import pytest

import hss_synth as syn
import oracle as O
from _cases import (check_topk_properties, dt_of, oracle_split, to_dev, to_host, weight)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def H():
    import sparse_rank_linear_hss_amd as h
    return h


def _assert_csr_equal(sp, ref, dtype):
    assert np.array_equal(to_host(sp.row_ptr), ref["row_ptr"])
    if sp.k > 0:
        assert np.array_equal(to_host(sp.col_idx), ref["col_idx"])
        assert O.bits_equal(to_host(sp.values), ref["values"])
    if sp.residual is not None:
        assert O.bits_equal(to_host(sp.residual), ref["residual"])


SHAPES = [(1, 1), (1, 7), (7, 1), (3, 5), (5, 13), (17, 33), (64, 64), (65, 129), (130, 1000),
          (1000, 37), (96, 4100), (33, 4104)]
KINDS = ["t3", "ties", "equal", "zeros", "ints"]


@pytest.mark.parametrize("dtype", [O.F32, O.BF16])
@pytest.mark.parametrize("shape", SHAPES, ids=[f"{m}x{n}" for m, n in SHAPES])
def test_split_csr_small(H, dtype, shape):
    m, n = shape
    mn = m * n
    for kind in KINDS:
        W = syn.random_matrix(m, n, dtype, seed=m * 131 + n, kind=kind)
        Wd = to_dev(W, dtype)
        for k in sorted({0, 1, mn // 20, mn // 3, mn - 1, mn} - {-1}):
            if k < 0:
                continue
            sp = H.hss_split(Wd, "csr", k=k, residual=True)
            _assert_csr_equal(sp, O.split_csr(W, dtype, k), dtype)


@pytest.mark.parametrize("cfg", ["csr1024_f32", "csr4096"])
def test_split_csr_workload_vs_oracle(H, cfg):
    c = syn.WORKLOADS[cfg]
    W = weight(cfg)
    dtype = dt_of(c.dtype)
    ref = oracle_split(cfg)
    sp = H.hss_split(to_dev(W, dtype), "csr", frac=c.frac, residual=True)
    assert sp.k == len(ref["col_idx"])
    _assert_csr_equal(sp, ref, dtype)
    sp2 = H.hss_split(to_dev(W, dtype), "csr", frac=c.frac, residual=False)   # deterministic
    assert np.array_equal(to_host(sp2.col_idx), ref["col_idx"])


@pytest.mark.parametrize("cfg,which", [("decoder_layer", i) for i in range(7)] + [("csr8192_prefill", 0)])
def test_split_csr_workload_properties(H, cfg, which):
    """Full-size decoder-layer and 8192^2 splits: the defining properties of
    the top-k set (which make it unique) checked on every entry."""
    c = syn.WORKLOADS[cfg]
    W = weight(cfg, which)
    dtype = dt_of(c.dtype)
    m, n = W.shape
    k = O.topk_count(m, n, *c.frac)
    sp = H.hss_split(to_dev(W, dtype), "csr", k=k, residual=True)
    check_topk_properties(W, dtype, k, to_host(sp.row_ptr), to_host(sp.col_idx),
                          to_host(sp.values), to_host(sp.residual))


def _assert_24_equal(sp, ref):
    assert O.bits_equal(to_host(sp.nm_values), ref["nm_values"])
    assert np.array_equal(to_host(sp.nm_meta).view(np.uint32), ref["nm_meta"])
    if sp.residual is not None:
        assert O.bits_equal(to_host(sp.residual), ref["residual"])


@pytest.mark.parametrize("dtype", [O.F32, O.BF16])
@pytest.mark.parametrize("shape", [(1, 4), (3, 8), (5, 36), (17, 32), (33, 100), (64, 4096), (7, 4100)])
def test_split_24_small(H, dtype, shape):
    """n % 32 == 0 takes the 16-byte load / store path, other widths the
    element-wise one; with and without the residual."""
    m, n = shape
    for i, kind in enumerate(KINDS):
        W = syn.random_matrix(m, n, dtype, seed=7 * m + n, kind=kind)
        sp = H.hss_split(to_dev(W, dtype), "2:4", residual=i % 2 == 0)
        _assert_24_equal(sp, O.split_24(W, dtype))


def test_split_24_nm24_11008x4096_vs_oracle(H):
    c = syn.WORKLOADS["nm24_11008x4096"]
    W = weight("nm24_11008x4096")
    sp = H.hss_split(to_dev(W, O.BF16), "2:4", residual=True)
    _assert_24_equal(sp, oracle_split("nm24_11008x4096"))


@pytest.mark.parametrize("fmt,k", [("csr", 10), ("csr", 0), ("csr", 144), ("2:4", None)])
@pytest.mark.parametrize("bad", [float("nan"), float("inf"), -float("inf")])
def test_split_flags_nonfinite(H, fmt, k, bad):
    """A NaN or infinity in W is reported for every k, also k = 0 (nothing
    kept: no threshold search, but the first pass still reads every key) and
    k = m n (everything kept)."""
    W = syn.random_matrix(9, 16, O.F32, seed=1, kind="t3").copy()
    W[4, 5] = bad
    with pytest.raises(H.HSSError) as ei:
        H.hss_split(to_dev(W, O.F32), fmt, k=k)
    assert ei.value.code == 4
    # a finite matrix afterwards (fresh workspace state) is fine
    H.hss_split(to_dev(np.zeros((9, 16), np.float32), O.F32), fmt, k=3 if fmt == "csr" else None)
