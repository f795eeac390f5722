"""GPU parity of hss_apply on the full-size workloads, every output row, with
the factors the workloads name: the oracle's truncated SVD of the stage-1
residual, rounded to bf16 (HSS page, section "2段階階層的スパース+低ランク圧縮",
stage 2; written by tests/golden/make_svd_factors.py, sha256 in its manifest).

The decoder layer runs in the launch configuration the benchmark times: q, k
and v as one grouped call, gate and up as another, o and down alone, several
tokens in sequence, eagerly and replayed from a HIP graph.

Bar: every output within tol * N[c, i], N = sum_j |A_ij X_cj| with A = S +
U V^T in fp64 from the stored operands; tol = 8e-3 for bf16."""
import os
import sys

import numpy as np
import pytest

import hss_synth as syn
import oracle as O
from _cases import dt_of, oracle_split, to_dev, to_host

sys.path.insert(0, os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden"))
import make_svd_factors as svd  # noqa: E402  (oracle-written factors)

pytestmark = pytest.mark.gpu

CHUNK = 1024  # oracle rows per block (bounds its memory at the 8192^2 layer)


@pytest.fixture(scope="module")
def H():
    import sparse_rank_linear_hss_amd as h
    return h


def _raw(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _matrix(H, cfg, which):
    import torch
    c = syn.WORKLOADS[cfg]
    dtype = dt_of(c.dtype)
    m, n = c.shapes[which]
    ref = oracle_split(cfg, which)
    U, V = svd.load(cfg, which)
    Ud, Vtd = to_dev(U, dtype), to_dev(np.ascontiguousarray(V.T), dtype)
    if c.fmt == "csr":
        A = H.HSSMatrix("csr", m, n, torch.bfloat16, U=Ud, Vt=Vtd, row_ptr=_raw(ref["row_ptr"]),
                        col_idx=_raw(ref["col_idx"]), values=to_dev(ref["values"], dtype), nnz=len(ref["col_idx"]))
    else:
        A = H.HSSMatrix("2:4", m, n, torch.bfloat16, U=Ud, Vt=Vtd, nm_values=to_dev(ref["nm_values"], dtype),
                        nm_meta=_raw(ref["nm_meta"].view(np.int32)))
    return A, ref, U, V


def _check_all_rows(cfg, which, ref, U, V, pairs):
    """Every output of each (X, Y) pair (Y: b x m, bf16 bits) against the
    oracle, CHUNK rows of A = S + U V^T at a time."""
    c = syn.WORKLOADS[cfg]
    dtype = dt_of(c.dtype)
    m, n = c.shapes[which]
    U64, V64 = O.widen(U, dtype), O.widen(V, dtype)
    worst = 0.0
    for i0 in range(0, m, CHUNK):
        rows = np.arange(i0, min(m, i0 + CHUNK))
        if c.fmt == "csr":
            S_rows = O.csr_rows_dense(rows, n, ref["row_ptr"], ref["col_idx"], ref["values"], dtype)
        else:
            S_rows = O.dense_from_24(len(rows), n, ref["nm_values"][rows], ref["nm_meta"][rows], dtype)
        for X, Y in pairs:
            Yref, N = O.apply_rows(S_rows, U64[rows], V64, O.widen(X, dtype))
            err = O.max_normalised_error(O.widen(Y, dtype)[:, rows], Yref, N)
            assert err <= O.TOL[dtype], f"{cfg}[{which}] rows {rows[0]}..{rows[-1]}: max normalised error {err:.3e}"
            worst = max(worst, err)
    return worst


@pytest.mark.parametrize("b", [1, 16])
def test_csr4096_every_row(H, b):
    """4096 x 4096, top 5 % CSR, rank 256 (truncated SVD), b = 1 and 16."""
    A, ref, U, V = _matrix(H, "csr4096", 0)
    X = syn.activations(syn.WORKLOADS["csr4096"], b)
    Y = to_host(H.hss_apply(A, to_dev(X, O.BF16)))
    _check_all_rows("csr4096", 0, ref, U, V, [(X, Y)])


@pytest.mark.parametrize("b", [1, 8, 64])
def test_nm24_11008x4096_every_row(H, b):
    """11008 x 4096, 2:4, rank 64 (truncated SVD), b = 1, 8, 64."""
    A, ref, U, V = _matrix(H, "nm24_11008x4096", 0)
    X = syn.activations(syn.WORKLOADS["nm24_11008x4096"], b)
    Y = to_host(H.hss_apply(A, to_dev(X, O.BF16)))
    _check_all_rows("nm24_11008x4096", 0, ref, U, V, [(X, Y)])


def test_csr8192_prefill_every_row(H):
    """8192 x 8192, top 3 % CSR, rank 512 (truncated SVD), prefill b = 2048."""
    A, ref, U, V = _matrix(H, "csr8192_prefill", 0)
    X = syn.activations(syn.WORKLOADS["csr8192_prefill"], 2048)
    Y = to_host(H.hss_apply(A, to_dev(X, O.BF16)))
    _check_all_rows("csr8192_prefill", 0, ref, U, V, [(X, Y)])


# The decoder layer's calls per token, as the benchmark makes them: projections
# that share their input are one grouped call.
LAYER_CALLS = [(0, 1, 2), (3,), (4, 5), (6,)]   # q k v | o | gate up | down


def test_decoder_layer_every_row_grouped_and_graph(H):
    """Seven projections (r = 409: U rows off the 16-byte grid), 3 tokens of
    batch-1 decode through the grouped calls; every output of every
    projection against the oracle, for the grouped calls and for single
    applies of each projection (a lone 4096 x 4096 matrix takes another
    launch plan, so the two may differ in the last bits); the token sequence
    repeated gives the same bits; a HIP graph of the whole sequence replayed
    twice (with eager calls on the same workspace in between) bit-equal to
    the eager run."""
    import torch
    cfg = "decoder_layer"
    c = syn.WORKLOADS[cfg]
    mats = [_matrix(H, cfg, w) for w in range(7)]
    tokens = 3
    xs = {(t, w): syn.activations(c, 1, w, t) for t in range(tokens) for w in range(7)}
    xd = {k: to_dev(v, O.BF16) for k, v in xs.items()}
    ys = {(t, w): torch.empty((1, c.shapes[w][0]), dtype=torch.bfloat16, device="cuda")
          for t in range(tokens) for w in range(7)}
    ws = H.apply_workspace(max(H.hss_apply_group_workspace_size([mats[w][0] for w in call], 1)
                               for call in LAYER_CALLS), "cuda")

    def run_layer():
        for t in range(tokens):
            for call in LAYER_CALLS:
                if len(call) == 1:
                    H.hss_apply(mats[call[0]][0], xd[(t, call[0])], ys[(t, call[0])], ws)
                else:
                    # projections of one group share X; each token's x of the group's first projection
                    H.hss_apply_group([mats[w][0] for w in call], xd[(t, call[0])], [ys[(t, w)] for w in call], ws)

    run_layer()
    eager = {k: to_host(v) for k, v in ys.items()}
    run_layer()
    for k, y in ys.items():
        assert O.bits_equal(to_host(y), eager[k]), k                  # deterministic
    single = {(t, w): to_host(H.hss_apply(mats[w][0], xd[(t, call[0])]))
              for t in range(tokens) for call in LAYER_CALLS for w in call}
    # oracle, every row of every projection (the input of a group is its first projection's x)
    for call in LAYER_CALLS:
        for w in call:
            A, ref, U, V = mats[w]
            _check_all_rows(cfg, w, ref, U, V, [(xs[(t, call[0])], eager[(t, w)]) for t in range(tokens)] +
                            [(xs[(t, call[0])], single[(t, w)]) for t in range(tokens)])
    # graph replay of the whole sequence
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run_layer()
    for rep in range(2):
        for y in ys.values():
            y.zero_()
        g.replay()
        torch.cuda.synchronize()
        for k, y in ys.items():
            assert O.bits_equal(to_host(y), eager[k]), (rep, k)
        H.hss_apply(mats[0][0], xd[(0, 0)], ws=ws)          # eager work on the same workspace
        torch.cuda.synchronize()
