"""Planted mistakes in the oracle must fail its pins.

Each case swaps one oracle function for a plausibly wrong variant (a dropped
term, a reversed tie-break, a transposed operand, a wrong rounding ...) and
checks that at least one of the pins in test_oracle_pins raises.  This shows
the pins can see the mistakes they are meant to catch.  Everything runs on the
CPU; nothing here touches the GPU path.
"""
import numpy as np
import pytest

import oracle
import oracle.hss_oracle as H
import test_oracle_pins as P


def _patch(monkeypatch, name, fn):
    monkeypatch.setattr(H, name, fn)
    monkeypatch.setattr(oracle, name, fn)


def _fails(*tests):
    for t in tests:
        try:
            t()
        except (AssertionError, ValueError, IndexError):
            return True
    return False


def _bits_equal_by_value(a, b):
    a, b = np.asarray(a), np.asarray(b)
    return a.shape == b.shape and bool(np.array_equal(a, b))      # values: +0 == -0, NaN != NaN


def _bits_equal_flat(a, b):
    a, b = np.ascontiguousarray(a).reshape(-1), np.ascontiguousarray(b).reshape(-1)
    if a.size != b.size or a.dtype.itemsize != b.dtype.itemsize:   # shape ignored
        return False
    v = {2: np.uint16, 4: np.uint32, 8: np.uint64}[a.dtype.itemsize]
    return bool(np.array_equal(a.view(v), b.view(v)))


def _bits_equal_low_half(a, b):
    a, b = np.ascontiguousarray(a), np.ascontiguousarray(b)
    if a.shape != b.shape:
        return False
    return bool(np.array_equal(a.view(np.uint8)[..., ::2], b.view(np.uint8)[..., ::2]))   # half the bytes


def _hier_count_halves_equal(k, m, n, r_diag, r_off):
    return int(k) + 2 * (m // 2 + n // 2) * (r_diag + r_off)       # odd sides lose a row/column


def _hier_count_dense_blocks(k, m, n, r_diag, r_off):
    return int(k) + 2 * (m // 2) * (n // 2) // 64 * (r_diag + r_off)


def _hier_count_one_diag(k, m, n, r_diag, r_off):
    return int(k) + (m // 2 + n // 2) * r_diag + (m + n) * r_off


_orig_apply_csr = H.apply_csr


def _apply_csr_no_lowrank(m, n, rp, ci, vals, dt, U, V, X):
    return _orig_apply_csr(m, n, rp, ci, vals, dt, U[:, :0], V[:, :0], X)     # the factor term dropped


def _apply_csr_rows_shifted(m, n, rp, ci, vals, dt, U, V, X):
    return np.roll(_orig_apply_csr(m, n, rp, ci, vals, dt, U, V, X), 1, axis=1)


_orig_nm24_pattern = H.nm24_pattern


def _nm24_pattern_slots_swapped(m, n, nm_meta):
    rp, ci = _orig_nm24_pattern(m, n, nm_meta)
    return rp, ci.reshape(-1, 2)[:, ::-1].reshape(-1).copy()     # the pair's columns in the wrong order


_orig_backward = H.backward
_orig_csr_transpose = H.csr_transpose


def _backward_dU_uses_U(m, n, rp, ci, S, U, V, X, G):
    g = _orig_backward(m, n, rp, ci, S, U, V, X, G)
    g["dU"] = (G.T @ X) @ np.resize(U, V.shape)                 # U where V belongs
    return g


def _backward_dX_no_lowrank(m, n, rp, ci, S, U, V, X, G):
    g = _orig_backward(m, n, rp, ci, S, U, V, X, G)
    g["dX"] = G @ S
    return g


def _backward_sign_flipped(m, n, rp, ci, S, U, V, X, G):
    g = _orig_backward(m, n, rp, ci, S, U, V, X, G)
    g["dV"] = -g["dV"]
    return g


def _backward_dS_transposed_index(m, n, rp, ci, S, U, V, X, G):
    g = _orig_backward(m, n, rp, ci, S, U, V, X, G)
    dA = G.T @ X
    rows = H.csr_row_of_entry(m, rp)
    g["dS"] = dA[np.asarray(ci) % m, rows % n]                  # row and column swapped
    return g


def _csr_transpose_row_major_order(m, n, rp, ci):
    rpt, cit, perm = _orig_csr_transpose(m, n, rp, ci)
    return rpt, cit, np.arange(len(perm))                          # storage order kept


def _csr_permute_cols_by_perm(n, row_ptr, col_idx, perm):
    perm = np.asarray(perm, dtype=np.int64)
    rp, ci = np.asarray(row_ptr, dtype=np.int64), np.asarray(col_idx, dtype=np.int64)
    out_rp, out_ci, src = [0], [], []
    for i in range(n):
        row = sorted((int(perm[ci[p]]), p) for p in range(rp[perm[i]], rp[perm[i] + 1]))  # perm, not its inverse
        out_ci.extend(c for c, _ in row)
        src.extend(p for _, p in row)
        out_rp.append(len(out_ci))
    return np.array(out_rp, dtype=np.int32), np.array(out_ci, dtype=np.int32), np.array(src, dtype=np.int64)


def _csr_permute_rows_by_inverse(n, row_ptr, col_idx, perm):
    inv = np.argsort(np.asarray(perm))
    rp, ci = np.asarray(row_ptr, dtype=np.int64), np.asarray(col_idx, dtype=np.int64)
    out_rp, out_ci, src = [0], [], []
    for i in range(n):
        row = sorted((int(inv[ci[p]]), p) for p in range(rp[inv[i]], rp[inv[i] + 1]))  # row inv[i], not perm[i]
        out_ci.extend(c for c, _ in row)
        src.extend(p for _, p in row)
        out_rp.append(len(out_ci))
    return np.array(out_rp, dtype=np.int32), np.array(out_ci, dtype=np.int32), np.array(src, dtype=np.int64)


_orig_csr_permute = H.csr_permute


def _csr_permute_unsorted(n, row_ptr, col_idx, perm):
    rp, ci, src = _orig_csr_permute(n, row_ptr, col_idx, perm)
    for i in range(n):                                     # each row in S's storage order instead
        seg = slice(rp[i], rp[i + 1])
        o = np.argsort(src[seg], kind="stable")
        ci[seg], src[seg] = ci[seg][o], src[seg][o]
    return rp, ci, src


def _apply_no_lowrank(S, U, V, X):
    return X @ S.T


def _apply_swapped_factors(S, U, V, X):
    return X @ S.T + (X @ U) @ V.T          # U and V exchanged


def _apply_transposed_sparse(S, U, V, X):
    return X @ S + (X @ V) @ U.T            # S not transposed


def _topk_ties_high(W, dtype, k):
    m, n = W.shape
    a = H.magnitudes(W, dtype).reshape(-1)
    order = np.argsort(-a[::-1], kind="stable")
    order = (m * n - 1) - order
    mask = np.zeros(m * n, dtype=bool)
    mask[order[:k]] = True
    return mask.reshape(m, n)


def _topk_signed(W, dtype, k):
    m, n = W.shape
    a = H.widen(W, dtype).reshape(-1)                  # sign kept: not a magnitude
    order = np.argsort(-a, kind="stable")
    mask = np.zeros(m * n, dtype=bool)
    mask[order[:k]] = True
    return mask.reshape(m, n)


def _count_rounded(m, n, num, den):
    return int(round(m * n * num / den))


def _nm24_ties_high(W, dtype):
    m, n = W.shape
    a = H.magnitudes(W, dtype).reshape(m, n // 4, 4)[..., ::-1]
    order = 3 - np.argsort(-a, axis=-1, kind="stable")
    keep = np.zeros((m, n // 4, 4), dtype=bool)
    np.put_along_axis(keep, order[..., :2], True, axis=-1)
    return keep.reshape(m, n)


_orig_split_24 = H.split_24


def _split24_nibble_swapped(W, dtype):
    out = _orig_split_24(W, dtype)
    meta = out["nm_meta"].astype(np.uint64)
    fixed = np.zeros_like(meta)
    for s in range(8):
        nib = (meta >> np.uint64(4 * s)) & np.uint64(0xF)
        swapped = ((nib & np.uint64(3)) << np.uint64(2)) | (nib >> np.uint64(2))
        fixed |= swapped << np.uint64(4 * s)
    out["nm_meta"] = fixed.astype(np.uint32)
    return out


def _svd_sigma_dropped(R64, r):
    Uf, s, Vt = np.linalg.svd(R64, full_matrices=False)
    return Uf[:, :r].copy(), Vt[:r].T.copy(), s


def _svd_v_not_transposed(R64, r):
    Uf, s, Vt = np.linalg.svd(R64, full_matrices=False)
    V = Vt[:r].copy()
    if V.shape != (R64.shape[1], r):
        V = np.resize(V, (R64.shape[1], r))
    return Uf[:, :r] * s[:r], V, s


def _normaliser_no_abs_x(S, U, V, X):
    return X @ np.abs(S + U @ V.T).T


_orig_csr_from_mask = H.csr_from_mask


def _csr_cols_descending(W, mask):
    rp, ci, v = _orig_csr_from_mask(W, mask)
    for i in range(len(rp) - 1):
        ci[rp[i]:rp[i + 1]] = ci[rp[i]:rp[i + 1]][::-1]
    return rp, ci, v


def _residual_keeps_values(W, mask):
    return np.array(W, copy=True)


def _pack_nibbles_swapped(codes):
    codes = np.asarray(codes, dtype=np.uint8)
    return (codes[..., 1::2] | (codes[..., 0::2] << 4)).astype(np.uint8)


_orig_kmeans = H.kmeans_1d


def _kmeans_ties_high(v64, K, max_iter=200):
    v = np.asarray(v64, dtype=np.float64).reshape(-1)
    u = np.unique(v)
    c = u[(2 * np.arange(K) + 1) * u.size // (2 * K)].astype(np.float64)
    codes = None
    for _ in range(max_iter):
        d = np.abs(v[:, None] - c[None, :])[:, ::-1]
        new = (K - 1) - np.argmin(d, axis=1)             # last minimum: upper index
        if codes is not None and np.array_equal(new, codes):
            break
        codes = new
        for k in range(K):
            if np.any(codes == k):
                c[k] = v[codes == k].mean()
    return c, codes


def _kmeans_one_step(v64, K, max_iter=200):
    return _orig_kmeans(v64, K, max_iter=1)


def _quantize_no_reassign(D, dtype, bits=4):
    m, n = D.shape
    K = 1 << bits
    D64 = H.widen(D, dtype)
    lut = np.zeros((m, K), dtype=np.float32 if dtype == H.F32 else np.uint16)
    codes = np.zeros((m, n), dtype=np.uint8)
    for i in range(m):
        c, cd = _orig_kmeans(D64[i], K)
        lut[i] = H.narrow(c, dtype)
        codes[i] = cd                                    # codes of the unrounded levels
    return lut, codes


def _dense_from_codes_row0_lut(codes, lut, dtype):
    L = H.widen(lut, dtype)
    return L[0][np.asarray(codes, dtype=np.int64)]       # one row's levels for every row


_orig_rcm = H.rcm_order


def _rcm_not_reversed(n, row_ptr, col_idx):
    return _orig_rcm(n, row_ptr, col_idx)[::-1].copy()


def _rcm_ties_high(n, row_ptr, col_idx):
    nbr = H.rcm_graph(n, row_ptr, col_idx)
    deg = [len(x) for x in nbr]
    seen, order = [False] * n, []
    while len(order) < n:
        start = min((v for v in range(n) if not seen[v]), key=lambda v: (deg[v], -v))
        seen[start] = True
        queue, head = [start], 0
        while head < len(queue):
            u = queue[head]
            head += 1
            for v in sorted((v for v in nbr[u] if not seen[v]), key=lambda v: (deg[v], -v)):
                seen[v] = True
                queue.append(v)
        order.extend(queue)
    return np.array(order[::-1], dtype=np.int32)


def _rho_off_diagonal(W, dtype, perm=None):
    a = H.magnitudes(W, dtype)
    if perm is not None:
        p = np.asarray(perm, dtype=np.int64)
        a = a[p][:, p]
    m, n = a.shape
    t = a.sum()
    return 0.0 if t == 0 else float((a[:m // 2, n // 2:].sum() + a[m // 2:, :n // 2].sum()) / t)


def _hier_factors_split_shifted(R64p, r_diag, r_off):
    R64p = np.asarray(R64p, dtype=np.float64)
    m, n = R64p.shape
    rows = [(0, m // 2 + 1), (m // 2 + 1, m)]
    cols = [(0, n // 2), (n // 2, n)]
    out = {}
    for bi in range(2):
        for bj in range(2):
            blk = R64p[rows[bi][0]:rows[bi][1], cols[bj][0]:cols[bj][1]]
            r = min(r_diag if bi == bj else r_off, min(blk.shape))
            U, V, _ = H.truncated_svd(blk, r)
            out[(bi, bj)] = (U, V)
    return out


def _hier_apply_perm_inverted(S64, blocks, perm, X64):
    m, n = S64.shape
    p = np.arange(n) if perm is None else np.asarray(perm, dtype=np.int64)
    Xp = X64[:, p]
    Yp = np.zeros((X64.shape[0], m))
    for (bi, bj), (U, V) in blocks.items():
        r0, r1 = (0, m // 2) if bi == 0 else (m // 2, m)
        c0, c1 = (0, n // 2) if bj == 0 else (n // 2, n)
        Yp[:, r0:r1] += (Xp[:, c0:c1] @ V) @ U.T
    return X64 @ S64.T + Yp[:, p]                         # y = y'[perm] instead of y[perm] = y'


CASES = [
    ("apply_factored", _apply_no_lowrank,
     [P.test_apply_hand_example, lambda: [P.test_apply_factored_equals_dense(s) for s in range(5)]]),
    ("apply_factored", _apply_swapped_factors,
     [P.test_apply_hand_example, lambda: P.test_apply_factored_equals_dense(0)]),
    ("apply_factored", _apply_transposed_sparse,
     [P.test_apply_hand_example, lambda: P.test_apply_factored_equals_dense(0)]),
    ("topk_mask", _topk_ties_high,
     [lambda: P.test_topk_matches_brute_force("equal", H.BF16, (3, 4)), P.test_topk_tie_split_across_rows]),
    ("topk_mask", _topk_signed,
     [lambda: P.test_topk_matches_brute_force("t3", H.F32, (6, 6))]),
    ("topk_count", _count_rounded, [P.test_worked_example_counts]),
    ("nm24_mask", _nm24_ties_high,
     [lambda: P.test_nm24_matches_brute_force("ties", H.BF16), P.test_nm24_hand_row]),
    ("split_24", _split24_nibble_swapped, [P.test_nm24_hand_row]),
    ("truncated_svd", _svd_sigma_dropped,
     [P.test_svd_eckart_young_and_orthonormality, P.test_svd_recovers_known_spectrum]),
    ("truncated_svd", _svd_v_not_transposed,
     [P.test_svd_eckart_young_and_orthonormality, P.test_svd_recovers_known_spectrum]),
    ("normaliser", _normaliser_no_abs_x, [P.test_normaliser_loop_definition]),
    ("csr_from_mask", _csr_cols_descending,
     [lambda: P.test_csr_matches_scipy(H.F32), lambda: P.test_csr_roundtrip_and_residual("t3")]),
    ("residual", _residual_keeps_values, [lambda: P.test_csr_roundtrip_and_residual("t3")]),
    ("pack_nibbles", _pack_nibbles_swapped, [P.test_pack_nibbles_hand_and_roundtrip]),
    ("kmeans_1d", _kmeans_ties_high, [P.test_kmeans_hand_tie_rule]),
    ("kmeans_1d", _kmeans_one_step,
     [lambda: [P.test_kmeans_fixed_point_and_not_worse_than_start(s) for s in range(3)]]),
    ("quantize_rows", _quantize_no_reassign,
     [lambda: P.test_quantize_rows_codes_are_nearest_stored_level(H.BF16)]),
    ("dense_from_codes", _dense_from_codes_row0_lut,
     [P.test_dense_sparse_apply_histogram_form, P.test_quantize_rows_few_distinct_values_is_exact]),
    ("rcm_order", _rcm_not_reversed, [P.test_rcm_hand_example]),
    ("rcm_order", _rcm_ties_high, [P.test_rcm_hand_example]),
    ("concentration_ratio", _rho_off_diagonal, [P.test_concentration_ratio_closed_forms]),
    ("hier_factors", _hier_factors_split_shifted, [P.test_hier_full_rank_reproduces_residual_and_eckart_young]),
    ("hier_apply", _hier_apply_perm_inverted, [lambda: P.test_hier_apply_equals_dense(True)]),
    ("backward", _backward_dU_uses_U, [lambda: P.test_backward_matches_exact_finite_differences(0)]),
    ("backward", _backward_dX_no_lowrank, [lambda: P.test_backward_matches_exact_finite_differences(0)]),
    ("backward", _backward_sign_flipped, [lambda: P.test_backward_matches_exact_finite_differences(0)]),
    ("backward", _backward_dS_transposed_index, [P.test_backward_one_hot_upstream_and_full_support_brute_force]),
    ("csr_transpose", _csr_transpose_row_major_order, [P.test_csr_transpose_is_the_transposed_matrix]),
    ("nm24_pattern", _nm24_pattern_slots_swapped, [P.test_nm24_pattern_is_the_mask_in_storage_order]),
    ("csr_permute", _csr_permute_cols_by_perm,
     [P.test_csr_permute_hand_example, lambda: P.test_csr_permute_is_the_permuted_matrix(17, 0.2, 2)]),
    ("csr_permute", _csr_permute_rows_by_inverse,
     [P.test_csr_permute_hand_example, lambda: P.test_csr_permute_is_the_permuted_matrix(17, 0.2, 2)]),
    ("csr_permute", _csr_permute_unsorted,
     [P.test_csr_permute_hand_example, lambda: P.test_csr_permute_is_the_permuted_matrix(17, 0.2, 2)]),
    ("apply_csr", _apply_csr_no_lowrank, [lambda: P.test_apply_csr_equals_the_hand_loop(11, 3)]),
    ("apply_csr", _apply_csr_rows_shifted, [lambda: P.test_apply_csr_equals_the_hand_loop(12, 0)]),
    ("bits_equal", _bits_equal_by_value, [P.test_bits_equal_compares_bit_patterns]),
    ("bits_equal", _bits_equal_flat, [P.test_bits_equal_compares_bit_patterns]),
    ("bits_equal", _bits_equal_low_half, [P.test_bits_equal_compares_bit_patterns]),
    ("hier_param_count", _hier_count_halves_equal, [P.test_hier_param_count_hand_counts]),
    ("hier_param_count", _hier_count_dense_blocks, [P.test_hier_param_count_hand_counts]),
    ("hier_param_count", _hier_count_one_diag,
     [lambda: P.test_hier_param_count_counts_the_stored_factors(9, 9, 3, 1)]),
]


@pytest.mark.parametrize("name,fn,pins", CASES, ids=[f"{c[0]}:{c[1].__name__}" for c in CASES])
def test_planted_mistake_is_caught(monkeypatch, name, fn, pins):
    _patch(monkeypatch, name, fn)
    assert _fails(*pins), f"no pin caught the planted mistake {fn.__name__} in {name}"
