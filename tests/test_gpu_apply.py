"""GPU parity of hss_apply against the CPU oracle.

Bar: every output within tol * N[c, i], N = sum_j |A_ij X_cj| (A = S + U V^T
built in fp64 from the stored operands); tol = 1e-5 for fp32, 8e-3 for bf16
inputs with fp32 accumulation and bf16 output.  The sparse part S always comes
from the oracle's own split of the seeded W (never from the GPU split)."""
import numpy as np
import pytest

import hss_synth as syn
import oracle as O
from _cases import dt_of, oracle_split, to_dev, to_host, weight

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


def _matrix(H, fmt, dtype, m, n, ref, U, V):
    """Device HSSMatrix from the oracle's split arrays and storage-typed U, V."""
    Ud = to_dev(U, dtype) if U.shape[1] > 0 else None
    Vtd = to_dev(np.ascontiguousarray(V.T), dtype) if V.shape[1] > 0 else None
    if fmt == "csr":
        k = len(ref["col_idx"])
        return H.HSSMatrix("csr", m, n, _tdt(dtype), U=Ud, Vt=Vtd, row_ptr=_raw(ref["row_ptr"]),
                           col_idx=_raw(ref["col_idx"]) if k else None,
                           values=to_dev(ref["values"], dtype) if k else None, nnz=k)
    return H.HSSMatrix("2:4", m, n, _tdt(dtype), U=Ud, Vt=Vtd, nm_values=to_dev(ref["nm_values"], dtype),
                       nm_meta=_raw(ref["nm_meta"].view(np.int32)))


def _dense_S(fmt, dtype, m, n, ref):
    if fmt == "csr":
        return O.dense_from_csr(m, n, ref["row_ptr"], ref["col_idx"], ref["values"], dtype)
    return O.dense_from_24(m, n, ref["nm_values"], ref["nm_meta"], dtype)


def _factors(m, n, r, dtype, seed):
    if r == 0:
        st = np.float32 if dtype == O.F32 else np.uint16
        return np.zeros((m, 0), st), np.zeros((n, 0), st)
    return syn.factors(m, n, r, dtype, seed)


def _check(Y_dev, dtype, Yref, N):
    err = O.max_normalised_error(O.widen(to_host(Y_dev), dtype), Yref, N)
    assert err <= O.TOL[dtype], f"max normalised error {err:.3e} > {O.TOL[dtype]}"
    return err


SMALL = [
    # (fmt, m, n, r, b)
    ("csr", 1, 1, 0, 1), ("csr", 5, 13, 2, 3), ("csr", 64, 64, 8, 1), ("csr", 65, 129, 7, 16),
    ("csr", 130, 1000, 64, 17), ("csr", 1000, 37, 5, 2), ("csr", 96, 4100, 33, 8),
    ("csr", 257, 512, 1, 33), ("csr", 300, 640, 128, 64),
    ("2:4", 1, 4, 0, 1), ("2:4", 5, 36, 3, 2), ("2:4", 64, 4096, 16, 1), ("2:4", 65, 128, 7, 9),
    ("2:4", 33, 100, 5, 16), ("2:4", 128, 512, 64, 64),
    # ragged row counts in the 2- and 4-rows-per-wave regimes (m >= 2048, m >= 8192)
    ("csr", 2053, 256, 16, 1), ("csr", 2049, 64, 9, 3), ("csr", 8195, 64, 12, 2),
    ("2:4", 8197, 128, 8, 1), ("2:4", 8197, 128, 8, 5), ("2:4", 2050, 64, 6, 2),
    # large batches: 256 x 128 tiles (ragged M and N, K tails not a multiple of the stage)
    ("csr", 300, 640, 128, 300), ("csr", 257, 1000, 72, 260), ("2:4", 100, 256, 16, 256),
    # 256 x 256 tiles: ragged M and N, split-K ranges across the S | U segment boundary,
    # odd stage counts per split
    ("csr", 520, 512, 256, 512), ("csr", 300, 224, 32, 260), ("csr", 256, 160, 64, 256),
    # one CSR column, bf16: T producers merged into 512-thread row blocks (r <= blocks <= CUs),
    # with a ragged last block, r equal to the block count, blocks past r, 1, 2 and 4 rows per wave
    ("csr", 1030, 512, 40, 1), ("csr", 4096, 1024, 256, 1), ("csr", 100, 128, 4, 1),
    ("csr", 7990, 256, 60, 1), ("csr", 2047, 64, 252, 1), ("2:4", 2100, 256, 16, 1),
    # ... and 2 or 4 T rows per block (r up to 4x the blocks)
    ("csr", 2048, 256, 400, 1), ("csr", 1024, 128, 500, 1),
    # ... with r % 4 != 0 (U rows read as 16-byte pieces straddling row ends)
    ("csr", 1030, 512, 41, 1), ("csr", 2050, 256, 409, 1),
    # inputs wider than 4096 on the one-column fast path: X staged beyond the
    # prologue's two vectors per thread; rows of ~410 entries take both CSR
    # chunks up front, rows of ~820 continue in the consume loop; r > 506
    # (two U pieces per lane)
    ("csr", 300, 8192, 24, 1), ("csr", 70, 16384, 16, 1), ("csr", 2051, 11008, 409, 1),
    ("csr", 200, 4096, 700, 1), ("2:4", 100, 8192, 8, 1),
]


@pytest.mark.parametrize("dtype", [O.F32, O.BF16])
@pytest.mark.parametrize("case", SMALL, ids=[f"{c[0]}-{c[1]}x{c[2]}-r{c[3]}-b{c[4]}" for c in SMALL])
def test_apply_small(H, dtype, case):
    fmt, m, n, r, b = case
    seed = m * 7 + n * 3 + r + b
    W = syn.random_matrix(m, n, dtype, seed=seed, kind="t3")
    ref = O.split_csr(W, dtype, O.topk_count(m, n, 5, 100)) if fmt == "csr" else O.split_24(W, dtype)
    U, V = _factors(m, n, r, dtype, seed)
    X = syn.random_matrix(b, n, dtype, seed=seed + 1, kind="normal", scale=1.0)
    S64 = _dense_S(fmt, dtype, m, n, ref)
    U64, V64, X64 = O.widen(U, dtype), O.widen(V, dtype), O.widen(X, dtype)
    Yref, N = O.apply_factored(S64, U64, V64, X64), O.normaliser(S64, U64, V64, X64)
    A = _matrix(H, fmt, dtype, m, n, ref, U, V)
    Xd = to_dev(X, dtype)
    Y1 = H.hss_apply(A, Xd)
    _check(Y1, dtype, Yref, N)
    Y2 = H.hss_apply(A, Xd)
    assert O.bits_equal(to_host(Y1), to_host(Y2))                  # deterministic


@pytest.mark.parametrize("dtype,b,r", [(O.F32, 5, 6), (O.BF16, 5, 6), (O.BF16, 32, 16), (O.BF16, 300, 0)])
def test_apply_empty_sparse_part(H, dtype, b, r):
    """k = 0: a pure low-rank product (matrix-core batches skip the sparse
    segment); with r = 0 too the output is exactly zero."""
    m, n = 70, 96
    W = syn.random_matrix(m, n, dtype, seed=3, kind="t3")
    ref = O.split_csr(W, dtype, 0)
    U, V = _factors(m, n, r, dtype, 5)
    X = syn.random_matrix(b, n, dtype, seed=4, kind="normal", scale=1.0)
    S64 = np.zeros((m, n))
    U64, V64, X64 = O.widen(U, dtype), O.widen(V, dtype), O.widen(X, dtype)
    Y = H.hss_apply(_matrix(H, "csr", dtype, m, n, ref, U, V), to_dev(X, dtype))
    _check(Y, dtype, O.apply_factored(S64, U64, V64, X64), O.normaliser(S64, U64, V64, X64))


def test_apply_csr1024_f32_true_svd(H):
    """1024 x 1024 fp32 workload end to end on the oracle's side: top 5 %, +0
    residual, rank-64 truncated SVD, factors cast to fp32; GPU apply at b=1."""
    c = syn.WORKLOADS["csr1024_f32"]
    W = weight("csr1024_f32")
    ref = oracle_split("csr1024_f32")
    U64, V64, _ = O.truncated_svd(O.widen(ref["residual"], O.F32), c.rank[0])
    U, V = O.narrow(U64, O.F32), O.narrow(V64, O.F32)
    X = syn.activations(c, 1)
    S64 = _dense_S("csr", O.F32, 1024, 1024, ref)
    Uw, Vw, Xw = O.widen(U, O.F32), O.widen(V, O.F32), O.widen(X, O.F32)
    Yref, N = O.apply_factored(S64, Uw, Vw, Xw), O.normaliser(S64, Uw, Vw, Xw)
    Y = H.hss_apply(_matrix(H, "csr", O.F32, 1024, 1024, ref, U, V), to_dev(X, O.F32))
    _check(Y, O.F32, Yref, N)


@pytest.mark.parametrize("fmt,dtype,b,m", [("csr", O.BF16, 1, 300), ("csr", O.F32, 3, 300), ("2:4", O.BF16, 8, 300),
                                           ("2:4", O.F32, 2, 300), ("csr", O.BF16, 1, 1030),
                                           ("2:4", O.BF16, 1, 1030), ("csr", O.BF16, 1, 100)])
def test_apply_local_fallback_is_bitwise_identical(H, hss_opt, fmt, dtype, b, m):
    """Every block computing every T row itself (decode_force_local: no T word
    is taken from the hand-off) must give the bits of the normal hand-off, and
    so must a zero poll budget (a mix, depending on timing).  One bf16 CSR
    column: the T rows come from the row blocks themselves, 4, 2 and 1 per
    block at m = 100, 300 and 1030.  r = 40 and 41: U rows on and off the
    16-byte grid."""
    n = 512
    hss_opt("batch_route", "decode")   # the fused kernel's hand-off is what is tested
    W = syn.random_matrix(m, n, dtype, seed=21, kind="t3")
    ref = O.split_csr(W, dtype, O.topk_count(m, n, 5, 100)) if fmt == "csr" else O.split_24(W, dtype)
    Xd = None
    for r in (40, 41):
        U, V = _factors(m, n, r, dtype, 22)
        X = syn.random_matrix(b, n, dtype, seed=23, kind="normal", scale=1.0)
        A = _matrix(H, fmt, dtype, m, n, ref, U, V)
        Xd = to_dev(X, dtype)
        Y_normal = to_host(H.hss_apply(A, Xd))
        hss_opt("decode_force_local", 1)
        Y_forced = to_host(H.hss_apply(A, Xd))
        hss_opt("decode_force_local", 0)
        hss_opt("decode_spin", 0)
        Y_spin0 = to_host(H.hss_apply(A, Xd))
        hss_opt("decode_spin", 4096)
        assert O.bits_equal(Y_normal, Y_forced), r
        assert O.bits_equal(Y_normal, Y_spin0), r
        assert O.bits_equal(Y_normal, to_host(H.hss_apply(A, Xd))), r   # the state after forced calls
        S64 = _dense_S(fmt, dtype, m, n, ref)
        U64, V64, X64 = O.widen(U, dtype), O.widen(V, dtype), O.widen(X, dtype)
        err = O.max_normalised_error(O.widen(Y_forced, dtype), O.apply_factored(S64, U64, V64, X64),
                                     O.normaliser(S64, U64, V64, X64))
        assert err <= O.TOL[dtype]


@pytest.mark.parametrize("fmt,n,shapes", [("csr", 128, [(3000, 64), (2000, 63), (700, 1)]),
                                            ("csr", 4096, [(2100, 41), (900, 5)]),
                                            ("csr", 4104, [(2100, 41)]),
                                            ("2:4", 512, [(2500, 9), (1100, 3)])])
def test_decode_producer_layouts_are_bitwise_identical(H, hss_opt, fmt, n, shapes):
    """One bf16 column with separate T producer blocks (merging off): one T row
    per producer wave (four per block; X of at most 4096 elements) and one T
    row per block give the same bits for every rows-per-wave setting, and so
    does every block computing every T row itself.  Ranks that leave the last
    producer block with idle waves (63, 41, 9, ...), several matrices in one
    launch, and X one vector too wide for the wave producers (n = 4104)."""
    dtype = O.BF16
    hss_opt("batch_route", "decode")
    hss_opt("decode_merged", 0)
    X = syn.random_matrix(1, n, dtype, seed=n + 5, kind="normal", scale=1.0)
    Xd = to_dev(X, dtype)
    mats, refs = [], []
    for i, (m, r) in enumerate(shapes):
        W = syn.random_matrix(m, n, dtype, seed=300 + 11 * i + m, kind="t3")
        ref = O.split_csr(W, dtype, O.topk_count(m, n, 3, 100)) if fmt == "csr" else O.split_24(W, dtype)
        U, V = _factors(m, n, r, dtype, 400 + i)
        mats.append(_matrix(H, fmt, dtype, m, n, ref, U, V))
        S64 = _dense_S(fmt, dtype, m, n, ref)
        Uw, Vw, Xw = O.widen(U, dtype), O.widen(V, dtype), O.widen(X, dtype)
        refs.append((O.apply_factored(S64, Uw, Vw, Xw), O.normaliser(S64, Uw, Vw, Xw)))
    Ys = H.hss_apply_group(mats, Xd)
    for Y, (Yref, N) in zip(Ys, refs):
        _check(Y, dtype, Yref, N)
    base = [to_host(Y) for Y in Ys]
    for wave in (0, 1):
        for rpw in (0, 1, 2, 4):
            for local in (0, 1):
                hss_opt("decode_wave_producers", wave)
                hss_opt("decode_rpw", rpw)
                hss_opt("decode_force_local", local)
                got = [to_host(Y) for Y in H.hss_apply_group(mats, Xd)]
                for i, (g, e) in enumerate(zip(got, base)):
                    assert O.bits_equal(g, e), (wave, rpw, local, i)
    hss_opt("decode_force_local", 0)


def test_apply_shared_workspace_many_calls(H):
    """One workspace shared by two matrices of different shape, rank and batch,
    called alternately many times: every result equals the one from a fresh
    workspace (the call tags never let a stale T row through)."""
    import torch
    dtype = O.BF16
    mats, xs, expect = [], [], []
    for (m, n, r, b, seed) in [(200, 256, 24, 1, 31), (96, 512, 70, 5, 32)]:
        W = syn.random_matrix(m, n, dtype, seed=seed, kind="t3")
        ref = O.split_csr(W, dtype, O.topk_count(m, n, 5, 100))
        U, V = _factors(m, n, r, dtype, seed)
        A = _matrix(H, "csr", dtype, m, n, ref, U, V)
        X = [to_dev(syn.random_matrix(b, n, dtype, seed=seed + 100 + i, kind="normal", scale=1.0), dtype)
             for i in range(3)]
        mats.append(A)
        xs.append(X)
        expect.append([to_host(H.hss_apply(A, x)) for x in X])     # each with its own workspace
    size = max(H.hss_apply_workspace_size(A, x[0].shape[0]) for A, x in zip(mats, xs))
    ws = H.apply_workspace(size, "cuda")
    for it in range(40):
        k = it % 2
        i = (it // 2) % 3
        Y = H.hss_apply(mats[k], xs[k][i], ws=ws)
        assert O.bits_equal(to_host(Y), expect[k][i]), (it, k, i)


@pytest.mark.parametrize("fmt,b", [("csr", 1), ("2:4", 1), ("csr", 2), ("csr", 5)])
def test_apply_on_two_streams_at_once(H, fmt, b):
    """One matrix applied from two streams (default priority) with nothing
    ordering the calls of one stream against the other's: the binding gives
    each stream its own workspace, so every result equals the one-stream
    result bit for bit."""
    import torch
    dtype = O.BF16
    m, n, r, calls = 2100, 512, 40, 24
    W = syn.random_matrix(m, n, dtype, seed=51, kind="t3")
    ref = O.split_csr(W, dtype, O.topk_count(m, n, 5, 100)) if fmt == "csr" else O.split_24(W, dtype)
    U, V = _factors(m, n, r, dtype, 52)
    A = _matrix(H, fmt, dtype, m, n, ref, U, V)
    xs = [to_dev(syn.random_matrix(b, n, dtype, seed=53 + i, kind="normal", scale=1.0), dtype) for i in range(4)]
    expect = [to_host(H.hss_apply(A, x)) for x in xs]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    ys = [[torch.empty((b, m), dtype=torch.bfloat16, device="cuda") for _ in range(calls)] for _ in streams]
    wss = []
    for s in streams:
        with torch.cuda.stream(s):
            wss.append(A.workspace(b))
    torch.cuda.synchronize()
    assert wss[0].data_ptr() != wss[1].data_ptr()
    for it in range(calls):
        for si, s in enumerate(streams):
            with torch.cuda.stream(s):
                H.hss_apply(A, xs[(it + si) % 4], ys[si][it])
    torch.cuda.synchronize()
    for si in range(2):
        for it in range(calls):
            assert O.bits_equal(to_host(ys[si][it]), expect[(it + si) % 4]), (si, it)


@pytest.mark.parametrize("fmt,b,m", [("csr", 1, 200), ("csr", 5, 200), ("2:4", 1, 200), ("csr", 32, 200),
                                     ("2:4", 64, 200), ("csr", 1, 1030), ("2:4", 1, 1030)])
def test_apply_graph_replay_matches_eager(H, fmt, b, m):
    """hss_apply captured into a HIP graph: every replay (with eager calls on
    the same workspace in between) reproduces the eager result bit for bit."""
    import torch
    dtype = O.BF16
    n, r = 256, 48
    W = syn.random_matrix(m, n, dtype, seed=41, kind="t3")
    ref = O.split_csr(W, dtype, O.topk_count(m, n, 5, 100)) if fmt == "csr" else O.split_24(W, dtype)
    U, V = _factors(m, n, r, dtype, 42)
    A = _matrix(H, fmt, dtype, m, n, ref, U, V)
    xs = [to_dev(syn.random_matrix(b, n, dtype, seed=43 + i, kind="normal", scale=1.0), dtype) for i in range(3)]
    ys = [torch.empty((b, m), dtype=torch.bfloat16, device="cuda") for _ in range(3)]
    ws = A.workspace(b)
    expect = [to_host(H.hss_apply(A, x, ws=ws)) for x in xs]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for x, y in zip(xs, ys):
            H.hss_apply(A, x, y, ws)
    for rep in range(4):
        for y in ys:
            y.zero_()
        g.replay()
        torch.cuda.synchronize()
        for i in range(3):
            assert O.bits_equal(to_host(ys[i]), expect[i]), (rep, i)
        # eager work on the same workspace between replays
        assert O.bits_equal(to_host(H.hss_apply(A, xs[rep % 3], ws=ws)), expect[rep % 3])


GROUPS = [
    # (fmt, [(m, r), ...], n, b)
    ("csr", [(200, 16), (64, 8), (300, 12)], 256, 1),
    ("csr", [(130, 7), (130, 0), (65, 33)], 96, 3),
    ("csr", [(2100, 16), (333, 4)], 64, 8),
    ("2:4", [(300, 8), (300, 8)], 128, 1),
    ("2:4", [(70, 5), (33, 16), (129, 4)], 64, 5),
    ("csr", [(150, 16), (90, 8)], 256, 16),
    # one bf16 column: T producers merged into the row blocks, 2 and 4 T rows per block (and a
    # group with more blocks than CUs at every row count per wave: separate producers)
    ("csr", [(1000, 200), (600, 100)], 512, 1),
    ("csr", [(512, 200), (256, 100), (300, 4)], 256, 1),
    ("csr", [(4096, 64), (4096, 64), (4090, 64)], 128, 1),
    ("csr", [(1000, 201), (600, 99)], 512, 1),
    # wide inputs: both CSR chunks up front for the long-row matrix only
    ("csr", [(300, 40), (200, 41)], 8192, 1),
]


@pytest.mark.parametrize("dtype", [O.F32, O.BF16])
@pytest.mark.parametrize("case", GROUPS, ids=[f"{c[0]}-g{len(c[1])}-n{c[2]}-b{c[3]}" for c in GROUPS])
def test_apply_group(H, dtype, case):
    """hss_apply_group: every output within the oracle bound, and bit-equal to
    hss_apply of the same matrix on the same X."""
    fmt, shapes, n, b = case
    X = syn.random_matrix(b, n, dtype, seed=n + b, kind="normal", scale=1.0)
    Xd = to_dev(X, dtype)
    mats, refs = [], []
    for i, (m, r) in enumerate(shapes):
        W = syn.random_matrix(m, n, dtype, seed=100 + 7 * i + m, kind="t3")
        ref = O.split_csr(W, dtype, O.topk_count(m, n, 5, 100)) if fmt == "csr" else O.split_24(W, dtype)
        U, V = _factors(m, n, r, dtype, 200 + i)
        mats.append(_matrix(H, fmt, dtype, m, n, ref, U, V))
        S64 = _dense_S(fmt, dtype, m, n, ref)
        Uw, Vw, Xw = O.widen(U, dtype), O.widen(V, dtype), O.widen(X, dtype)
        refs.append((O.apply_factored(S64, Uw, Vw, Xw), O.normaliser(S64, Uw, Vw, Xw)))
    Ys = H.hss_apply_group(mats, Xd)
    for A, Y, (Yref, N) in zip(mats, Ys, refs):
        _check(Y, dtype, Yref, N)
        assert O.bits_equal(to_host(Y), to_host(H.hss_apply(A, Xd)))


@pytest.mark.parametrize("dtype,b", [(O.BF16, 1), (O.F32, 1), (O.BF16, 3)])
def test_apply_group_with_rank0_member_shares_a_workspace(H, dtype, b):
    """A grouped call that includes a matrix with no low-rank term, called
    again and again on one workspace with changing inputs (single calls in
    between): every result equals the one from a fresh workspace.  Every
    block of a launch counts towards the call epoch, so no later call takes
    an earlier call's T words as its own."""
    n = 96
    shapes = [(130, 7), (130, 0), (65, 33)]
    mats = []
    for i, (m, r) in enumerate(shapes):
        W = syn.random_matrix(m, n, dtype, seed=300 + 7 * i + m, kind="t3")
        ref = O.split_csr(W, dtype, O.topk_count(m, n, 5, 100))
        U, V = _factors(m, n, r, dtype, 310 + i)
        mats.append(_matrix(H, "csr", dtype, m, n, ref, U, V))
    xs = [to_dev(syn.random_matrix(b, n, dtype, seed=320 + j, kind="normal", scale=1.0), dtype) for j in range(3)]
    expect = [[to_host(y) for y in H.hss_apply_group(mats, x)] for x in xs]      # fresh workspace each
    expect0 = [to_host(H.hss_apply(mats[2], x, ws=H.apply_workspace(H.hss_apply_workspace_size(mats[2], b), "cuda")))
               for x in xs]
    ws = H.apply_workspace(H.hss_apply_group_workspace_size(mats, b), "cuda")
    for it in range(12):
        j = it % 3
        Ys = H.hss_apply_group(mats, xs[j], ws=ws)
        for g in range(3):
            assert O.bits_equal(to_host(Ys[g]), expect[j][g]), (it, g)
        if it % 4 == 3:
            assert O.bits_equal(to_host(H.hss_apply(mats[2], xs[(j + 1) % 3], ws=ws)), expect0[(j + 1) % 3]), it


def test_apply_group_graph_replay(H):
    """A captured grouped apply replays to the eager result, with eager calls
    on the same workspace in between."""
    import torch
    dtype, n, b = O.BF16, 256, 1
    mats = []
    for i, (m, r) in enumerate([(400, 16), (256, 32), (256, 32)]):
        W = syn.random_matrix(m, n, dtype, seed=500 + i, kind="t3")
        ref = O.split_csr(W, dtype, O.topk_count(m, n, 5, 100))
        U, V = _factors(m, n, r, dtype, 600 + i)
        mats.append(_matrix(H, "csr", dtype, m, n, ref, U, V))
    xs = [to_dev(syn.random_matrix(b, n, dtype, seed=700 + i, kind="normal", scale=1.0), dtype) for i in range(2)]
    ws = torch.zeros(H.hss_apply_group_workspace_size(mats, b), dtype=torch.uint8, device="cuda")
    ys = [[torch.empty((b, A.m), dtype=torch.bfloat16, device="cuda") for A in mats] for _ in xs]
    expect = [[to_host(y) for y in H.hss_apply_group(mats, x, ws=ws)] for x in xs]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for x, y in zip(xs, ys):
            H.hss_apply_group(mats, x, y, ws)
    for rep in range(4):
        g.replay()
        torch.cuda.synchronize()
        for i in range(len(xs)):
            for j in range(len(mats)):
                assert O.bits_equal(to_host(ys[i][j]), expect[i][j]), (rep, i, j)
        assert O.bits_equal(to_host(H.hss_apply(mats[0], xs[rep % 2], ws=ws)), expect[rep % 2][0])


COL16 = [
    # (m, n, r, b): every decode regime, the matrix-core densify and the large tile
    (300, 640, 128, 1), (130, 1000, 64, 3), (2053, 256, 16, 1), (8195, 64, 12, 2), (96, 4104, 33, 8),
    (257, 512, 8, 24), (300, 640, 128, 300), (5, 13, 2, 3),
]


@pytest.mark.parametrize("dtype", [O.F32, O.BF16])
@pytest.mark.parametrize("case", COL16, ids=[f"{c[0]}x{c[1]}-r{c[2]}-b{c[3]}" for c in COL16])
def test_apply_col16(H, dtype, case):
    """16-bit CSR columns: the same result bit for bit as 32-bit columns, and
    within the oracle bound."""
    m, n, r, b = case
    W = syn.random_matrix(m, n, dtype, seed=900 + m + n, kind="t3")
    ref = O.split_csr(W, dtype, O.topk_count(m, n, 5, 100))
    U, V = _factors(m, n, r, dtype, 901)
    X = syn.random_matrix(b, n, dtype, seed=902 + b, kind="normal", scale=1.0)
    A32 = _matrix(H, "csr", dtype, m, n, ref, U, V)
    A16 = A32.with_col16()
    assert A16.struct.flags == H.HSS_COL16
    assert np.array_equal(to_host(A16.col_idx).view(np.uint16).astype(np.int64), ref["col_idx"].astype(np.int64))
    Xd = to_dev(X, dtype)
    Y16, Y32 = H.hss_apply(A16, Xd), H.hss_apply(A32, Xd)
    assert O.bits_equal(to_host(Y16), to_host(Y32))
    S64 = _dense_S("csr", dtype, m, n, ref)
    Uw, Vw, Xw = O.widen(U, dtype), O.widen(V, dtype), O.widen(X, dtype)
    _check(Y16, dtype, O.apply_factored(S64, Uw, Vw, Xw), O.normaliser(S64, Uw, Vw, Xw))


def test_apply_group_col16(H):
    dtype, n, b = O.BF16, 256, 1
    X = to_dev(syn.random_matrix(b, n, dtype, seed=77, kind="normal", scale=1.0), dtype)
    mats = []
    for i, (m, r) in enumerate([(200, 16), (64, 8)]):
        W = syn.random_matrix(m, n, dtype, seed=78 + i, kind="t3")
        ref = O.split_csr(W, dtype, O.topk_count(m, n, 5, 100))
        U, V = _factors(m, n, r, dtype, 80 + i)
        mats.append(_matrix(H, "csr", dtype, m, n, ref, U, V))
    y32 = H.hss_apply_group(mats, X)
    y16 = H.hss_apply_group([A.with_col16() for A in mats], X)
    for a, c in zip(y32, y16):
        assert O.bits_equal(to_host(a), to_host(c))
