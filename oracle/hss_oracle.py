"""CPU oracle for the sparse + low-rank (HSS) linear layer  Y = X (S + U V^T)^T.

TEST INFRASTRUCTURE ONLY.  This module is the slow, obviously-correct fp64
statement of what the GPU library computes.  Only the tests, the package's
smoke check and the benchmark's CPU-baseline leg may import it; the product
path never does.  It shares no code with the HIP library and imports nothing
from this repository.

Sources (web pages; section names as printed on each page)
-----------------------------------------------------------
[HSS]     "LLMの階層的スパース+低ランク圧縮" (hierarchical sparse + low-rank
          compression of LLMs), d7fyzohlfz9vz.cloudfront.net/posts/
          hierarchical-sparse-plus-low-rank-compression-of-llm
          - section "2段階階層的スパース+低ランク圧縮" (two-stage HSS):
            the decomposition W ~= S + U V^T with U (m x r), V (n x r);
            stage 1 keeps the top fraction of weights by absolute magnitude,
            stage 2 factors the remaining dense residual; the 1024 x 1024
            worked example (具体例); rank starts at 10 % of the dimension
            (actionable-implications paragraph).
          - section "2段階階層的スパース+低ランク圧縮:ハイブリッドの利点" (vision
            rewrite): top 5-10 % by magnitude, the residual is rebuilt with
            minimal error; rank = 102 for a 1024-wide layer.
          - section "実装と運用パターン" (implementation patterns): S stored as
            indices + values (COO/CSR), U and V dense; the forward pass splits
            into one sparse product plus two small dense products.
          - section "順列と階層的整列" (permutation and hierarchical alignment; its
            vision rewrite "置換と階層的整列"): the concentration ratio rho =
            (sum of |W| over the diagonal blocks) / (sum of |W|); a Reverse
            Cuthill-McKee order of rows and columns pulls large |w| towards the
            diagonal; the factorisation works on a 2 x 2 block partition, the
            off-diagonal blocks at a low rank (8), the diagonal ones higher (32).
[HASSLE]  aibr.jp/archives/82335 (explainer of HASSLE-free), section
          "3.中核となる技術的要素": N:M sparsity as the GPU-friendly structure.
[SQZ]     aibr.jp/archives/208940 (explainer of SqueezeLLM), section
          "3.中核となる技術的要素": the dense-and-sparse decomposition W = D + S
          (the rare outliers kept exactly in a CSR matrix S, the dense rest D
          quantised with non-uniform levels); section "4.有効性の検証方法と成果":
          the sparse part is about 0.5 % of the weights.

Readings where the pages are silent or ambiguous:
* k = floor(m*n*num/den) in exact integer arithmetic (the worked example
  prints 52,428 for 5 % of 1,048,576, i.e. floor).
* Ties at the threshold go to the lower row-major linear index; exactly k
  entries are kept.
* |+0| = |-0| = 0; NaN/Inf weights are rejected.
* 2:4 = keep the 2 largest |w| of each group of 4 consecutive columns (along
  the reduction dimension), ties to the lower column.
* Stage 2 is one truncated SVD of the whole residual at rank r, with the
  singular values folded into U (U = U_r diag(s_r), V = V_r).
* The residual equals W with the kept positions set to +0 (no subtraction).
* Dense-and-sparse: S = the top 0.5 % by |w| (k = floor(m*n*5/1000)), D = the
  residual; each row of D is quantised to 2^bits levels by unweighted 1-D
  k-means (the pages' sensitivity weights need gradients from data, which
  this path has none of), started at quantiles of the distinct values, ties
  to the lower level; levels are stored in the weight's type and every code
  is the nearest stored level.  4-bit codes are packed two per byte, the even
  column in the low nibble.
* Hierarchical variant (one level, as the 512 x 512 example describes): the
  2 x 2 blocks split rows at m1 = m // 2 and columns at n1 = n // 2; rho
  counts the two diagonal blocks.  RCM works on the symmetric graph of the
  stage-1 support (edge i - j when S has (i, j) or (j, i), i != j) of a
  square matrix: components in order of their lowest-degree (then lowest
  index) unvisited node, breadth-first, each node's unvisited neighbours
  queued by (degree, index) ascending; the visit order reversed.  perm[i] is
  the original index at position i; the permuted matrix is W'[i, j] =
  W[perm[i], perm[j]].  S stays in the original order (stage 1 before the
  permutation); each block of the permuted residual gets its own truncated
  SVD.  A layer reordered by perm can also be held entirely in the permuted
  order (as when the permutation is folded into the neighbouring layers):
  S' = P S P^T (csr_permute), x' = x[perm], y[perm] = y'; its block term is
  then the plain block matrix, with no permutation inside.

* Backward: the pages give dS, dU and dV; the input gradient dX = G A is
  added, since a layer's backward pass needs it.  dS is restricted to S's
  stored positions (its pattern is fixed).  S^T's CSR orders each row's
  entries by original row.

Storage conventions (the same ones the C library documents):
  fp32 values are numpy.float32; bf16 values are their bit patterns in
  numpy.uint16.  Matrices are row-major.  W is m x n (out x in), X is b x n,
  Y is b x m.
"""
from __future__ import annotations

import numpy as np

F32 = "f32"
BF16 = "bf16"


# ---------------------------------------------------------------------------
# Storage-type helpers (exact widening; RNE narrowing)
# ---------------------------------------------------------------------------

def widen(a, dtype):
    """Exact fp64 values of stored fp32 / bf16 data."""
    if dtype == F32:
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == BF16:
        bits = np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def narrow(a64, dtype):
    """fp64 -> storage type, round to nearest even at each step (fp64->fp32->bf16)."""
    a32 = np.asarray(a64, dtype=np.float64).astype(np.float32)
    if dtype == F32:
        return a32
    if dtype == BF16:
        u = a32.view(np.uint32).astype(np.uint64)
        # bf16 = upper half of fp32; add half an ulp minus one, plus the lsb of
        # the kept part, then truncate: ties go to the even pattern.
        return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    raise ValueError(dtype)


def bits_equal(a, b):
    """Bitwise equality of two stored arrays of the same storage type: the same
    shape, the same element width and every bit pattern equal.  It compares
    patterns, not values: +0 and -0 differ, and a NaN equals only the same NaN
    pattern."""
    a = np.ascontiguousarray(a)
    b = np.ascontiguousarray(b)
    if a.shape != b.shape or a.dtype.itemsize != b.dtype.itemsize:
        return False
    view = {2: np.uint16, 4: np.uint32, 8: np.uint64}[a.dtype.itemsize]
    return bool(np.array_equal(a.view(view), b.view(view)))


# ---------------------------------------------------------------------------
# Counts  ([HSS] two-stage section, worked example; vision rewrite, rank rule)
# ---------------------------------------------------------------------------

def topk_count(m, n, num, den):
    """Number of weights kept in S for a kept fraction num/den: floor(m*n*num/den)."""
    m, n, num, den = int(m), int(n), int(num), int(den)
    if m < 0 or n < 0 or num < 0 or den <= 0:
        raise ValueError("bad count arguments")
    return (m * n * num) // den


def rank_rule(m, n, num=10, den=100):
    """Starting rank: num/den of the smaller matrix dimension, floored (1024 -> 102)."""
    return (min(int(m), int(n)) * int(num)) // int(den)


def param_count(k, m, n, r):
    """Stored parameters of S + U V^T: k sparse values plus (m + n) r factor entries."""
    return int(k) + (int(m) + int(n)) * int(r)


def compression_ratio(m, n, k, r):
    """Dense parameters over stored parameters (1024^2, 5 %, rank 64 -> 5.714)."""
    return (int(m) * int(n)) / param_count(k, m, n, r)


# ---------------------------------------------------------------------------
# Stage 1: magnitude top-k and its storage
# ---------------------------------------------------------------------------

def magnitudes(W, dtype):
    """|w| in fp64 (exact).  Non-finite weights have no magnitude order: rejected."""
    a = np.abs(widen(W, dtype))
    if not np.all(np.isfinite(a)):
        raise ValueError("non-finite weight")
    return a


def topk_mask(W, dtype, k):
    """Boolean m x n mask of the k weights of largest |w|.

    Order: |w| descending, then row-major linear index ascending (a stable
    sort of -|w|), and the first k positions of that order are kept."""
    m, n = W.shape
    k = int(k)
    if not 0 <= k <= m * n:
        raise ValueError("k out of range")
    a = magnitudes(W, dtype).reshape(-1)
    order = np.argsort(-a, kind="stable")
    mask = np.zeros(m * n, dtype=bool)
    mask[order[:k]] = True
    return mask.reshape(m, n)


def csr_from_mask(W, mask):
    """CSR of the masked entries: row_ptr int32[m+1], col_idx int32[nnz]
    (ascending within each row), values[nnz] = the stored W bits."""
    m, n = W.shape
    counts = mask.sum(axis=1)
    row_ptr = np.zeros(m + 1, dtype=np.int64)
    row_ptr[1:] = np.cumsum(counts)
    rows, cols = np.nonzero(mask)          # row-major order: rows asc, cols asc
    values = np.ascontiguousarray(W[rows, cols])
    return row_ptr.astype(np.int32), cols.astype(np.int32), values


def residual(W, mask):
    """W with the kept positions replaced by +0 (bit pattern 0); other bits unchanged."""
    R = np.array(W, copy=True)
    R[mask] = 0
    return R


def split_csr(W, dtype, k):
    """Stage 1 in CSR form.  Returns dict(row_ptr, col_idx, values, residual, mask)."""
    mask = topk_mask(W, dtype, k)
    row_ptr, col_idx, values = csr_from_mask(W, mask)
    return dict(row_ptr=row_ptr, col_idx=col_idx, values=values,
                residual=residual(W, mask), mask=mask)


def nm24_mask(W, dtype):
    """2:4 mask: in each group of 4 consecutive columns keep the 2 largest |w|,
    ties to the lower column ([HASSLE] N:M structure; groups along the input
    (reduction) dimension, starting at column 0)."""
    m, n = W.shape
    if n % 4 != 0:
        raise ValueError("2:4 needs n % 4 == 0")
    a = magnitudes(W, dtype).reshape(m, n // 4, 4)
    order = np.argsort(-a, axis=-1, kind="stable")      # (|w| desc, column asc)
    keep = np.zeros_like(a, dtype=bool)
    np.put_along_axis(keep, order[..., :2], True, axis=-1)
    return keep.reshape(m, n)


def split_24(W, dtype):
    """Stage 1 in 2:4 form.

    nm_values[i, 2g+s] = W bits of the s-th kept entry (ascending column) of
    group g of row i; nm_meta[i, g // 8] holds, at bits 4*(g % 8) .. +3, the
    nibble i0 | (i1 << 2) with i0 < i1 the kept positions inside the group.
    Returns dict(nm_values, nm_meta, residual, mask)."""
    m, n = W.shape
    mask = nm24_mask(W, dtype)
    groups = n // 4
    words = (n + 31) // 32
    kept_pos = np.nonzero(mask.reshape(m, groups, 4))[2].reshape(m, groups, 2)  # ascending
    nm_values = np.ascontiguousarray(W[mask].reshape(m, groups * 2))
    nib = (kept_pos[..., 0] | (kept_pos[..., 1] << 2)).astype(np.uint64)
    nm_meta = np.zeros((m, words), dtype=np.uint64)
    for g in range(groups):
        nm_meta[:, g // 8] |= nib[:, g] << np.uint64(4 * (g % 8))
    return dict(nm_values=nm_values, nm_meta=nm_meta.astype(np.uint32),
                residual=residual(W, mask), mask=mask)


def dense_from_csr(m, n, row_ptr, col_idx, values, dtype):
    """fp64 dense S rebuilt from CSR (stored values widened exactly)."""
    S = np.zeros((m, n), dtype=np.float64)
    v = widen(values, dtype)
    for i in range(m):
        lo, hi = int(row_ptr[i]), int(row_ptr[i + 1])
        S[i, col_idx[lo:hi]] = v[lo:hi]
    return S


def dense_from_24(m, n, nm_values, nm_meta, dtype):
    """fp64 dense S rebuilt from 2:4 values + nibble metadata."""
    S = np.zeros((m, n), dtype=np.float64)
    v = widen(nm_values, dtype).reshape(m, n // 2)
    meta = np.asarray(nm_meta, dtype=np.uint32).reshape(m, -1)
    for g in range(n // 4):
        nib = (meta[:, g // 8] >> np.uint32(4 * (g % 8))) & np.uint32(0xF)
        i0 = (nib & 3).astype(np.int64)
        i1 = ((nib >> 2) & 3).astype(np.int64)
        rows = np.arange(m)
        S[rows, 4 * g + i0] = v[:, 2 * g]
        S[rows, 4 * g + i1] = v[:, 2 * g + 1]
    return S


# ---------------------------------------------------------------------------
# Stage 2: truncated SVD of the residual  ([HSS] two-stage section)
# ---------------------------------------------------------------------------

def truncated_svd(R64, r):
    """Rank-r factors of the fp64 residual: U = U_r diag(s_r) (m x r), V = V_r (n x r).

    LAPACK gesdd through numpy.  Each singular pair is sign-normalised so that
    the largest-|.| entry of the V column is positive (first index on ties).
    Returns (U, V, s) with s the full vector of singular values."""
    R64 = np.asarray(R64, dtype=np.float64)
    m, n = R64.shape
    r = int(r)
    if not 0 <= r <= min(m, n):
        raise ValueError("rank out of range")
    Uf, s, Vt = np.linalg.svd(R64, full_matrices=False)
    U = Uf[:, :r] * s[:r][None, :]
    V = Vt[:r].T.copy()
    for l in range(r):
        j = int(np.argmax(np.abs(V[:, l])))
        if V[j, l] < 0:
            V[:, l] = -V[:, l]
            U[:, l] = -U[:, l]
    return U, V, s


# ---------------------------------------------------------------------------
# Apply: Y = X S^T + (X V) U^T   ([HSS] implementation-patterns section)
# ---------------------------------------------------------------------------

def apply_factored(S64, U64, V64, X64):
    """Factored forward in fp64: sparse term plus two small dense products."""
    Y = X64 @ S64.T
    if U64.shape[1] > 0:
        Y = Y + (X64 @ V64) @ U64.T
    return Y


def apply_csr(m, n, row_ptr, col_idx, values, dtype, U64, V64, X64):
    """Factored forward with S kept in CSR, as the pages store it (indices +
    values): the sparse product through scipy.sparse, plus (X V) U^T, fp64."""
    import scipy.sparse
    S = scipy.sparse.csr_matrix((widen(values, dtype), np.asarray(col_idx, dtype=np.int64),
                                 np.asarray(row_ptr, dtype=np.int64)), shape=(m, n))
    Y = (S @ X64.T).T
    if U64.shape[1] > 0:
        Y = Y + (X64 @ V64) @ U64.T
    return np.asarray(Y)


def apply_dense(S64, U64, V64, X64):
    """Dense forward in fp64 with the rebuilt A = S + U V^T."""
    return X64 @ (S64 + U64 @ V64.T).T


def normaliser(S64, U64, V64, X64):
    """N[c, i] = sum_j |A_ij X_cj| with A = S + U V^T in fp64: the scale the
    per-output error bound is stated against."""
    A = S64 + U64 @ V64.T
    return np.abs(X64) @ np.abs(A).T


def max_normalised_error(Y, Y_ref, N):
    """max over outputs of |Y - Y_ref| / N; an output with N == 0 must be 0 exactly
    (else the result is inf)."""
    Y = np.asarray(Y, dtype=np.float64)
    err = np.abs(Y - Y_ref)
    zero = N == 0
    if np.any(err[zero] != 0):
        return float("inf")
    if not np.any(~zero):
        return 0.0
    return float(np.max(err[~zero] / N[~zero]))


# Error tolerances of the apply step (per output, relative to N).
TOL = {F32: 1e-5, BF16: 8e-3}


# ---------------------------------------------------------------------------
# Row-sampled apply for full-size checks (same definitions, a subset of rows)
# ---------------------------------------------------------------------------

def csr_rows_dense(rows, n, row_ptr, col_idx, values, dtype):
    """fp64 dense rows of S (len(rows) x n) from CSR."""
    out = np.zeros((len(rows), n), dtype=np.float64)
    v = widen(values, dtype)
    for t, i in enumerate(rows):
        lo, hi = int(row_ptr[i]), int(row_ptr[i + 1])
        out[t, col_idx[lo:hi]] = v[lo:hi]
    return out


def apply_rows(S_rows64, U_rows64, V64, X64):
    """Y[:, rows] and N[:, rows] from the dense rows of S and the rows of U."""
    A_rows = S_rows64 + U_rows64 @ V64.T
    return X64 @ A_rows.T, np.abs(X64) @ np.abs(A_rows).T


# ---------------------------------------------------------------------------
# Dense-and-sparse variant W = D + S  ([SQZ] section "3.中核となる技術的要素":
# the few outliers stay exact in a sparse CSR matrix, the dense remainder is
# quantised with non-uniform levels)
# ---------------------------------------------------------------------------

def outlier_count(m, n):
    """Outliers kept in S: 0.5 % of the weights, floor(m*n*5/1000)."""
    return topk_count(m, n, 5, 1000)


def kmeans_1d(v64, K, max_iter=200):
    """K-level quantiser of the values v by Lloyd's algorithm.

    Start: with u the sorted distinct values, centroid k is u[floor((k + 1/2)
    * |u| / K)] (the middle of the k-th of K equal bins of distinct values; with
    at most K distinct values every one of them is a starting centroid, so the
    result is exact).  Step: every value goes to its nearest centroid (ties to
    the lower index); every non-empty cluster's centroid moves to the mean of
    its values, an empty one stays.  Stops when no assignment changes.
    Returns (centroids fp64[K], codes int[n])."""
    v = np.asarray(v64, dtype=np.float64).reshape(-1)
    if v.size == 0:
        return np.zeros(K), np.zeros(0, dtype=np.int64)
    u = np.unique(v)
    c = u[(2 * np.arange(K) + 1) * u.size // (2 * K)].astype(np.float64)
    codes = None
    for _ in range(max_iter):
        new = np.argmin(np.abs(v[:, None] - c[None, :]), axis=1)   # first minimum: lower index
        if codes is not None and np.array_equal(new, codes):
            break
        codes = new
        for k in range(K):
            members = v[codes == k]
            if members.size:
                c[k] = members.mean()
    return c, codes


def nearest_level(v64, levels64):
    """Index of the nearest level for each value (ties to the lower index)."""
    v = np.asarray(v64, dtype=np.float64)
    return np.argmin(np.abs(v[..., None] - np.asarray(levels64)[None, :]), axis=-1)


def quantize_rows(D, dtype, bits=4):
    """Per-row non-uniform quantisation of D (m x n, stored type).

    Returns (lut, codes): lut m x 2^bits in the stored type (the row's k-means
    centroids, rounded), codes m x n uint8 = index of the nearest stored level."""
    m, n = D.shape
    K = 1 << int(bits)
    D64 = widen(D, dtype)
    lut = np.zeros((m, K), dtype=np.float32 if dtype == F32 else np.uint16)
    codes = np.zeros((m, n), dtype=np.uint8)
    for i in range(m):
        c, _ = kmeans_1d(D64[i], K)
        lut[i] = narrow(c, dtype)
        codes[i] = nearest_level(D64[i], widen(lut[i], dtype))
    return lut, codes


def pack_nibbles(codes):
    """4-bit codes m x n (n even) -> bytes m x n/2: byte j = code[2j] | code[2j+1] << 4."""
    codes = np.asarray(codes, dtype=np.uint8)
    if codes.shape[-1] % 2 or np.any(codes > 15):
        raise ValueError("4-bit codes need an even row length and values < 16")
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed, n):
    """Inverse of pack_nibbles."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.zeros(packed.shape[:-1] + (n,), dtype=np.uint8)
    out[..., 0::2] = packed & 0xF
    out[..., 1::2] = packed >> 4
    return out


def dense_from_codes(codes, lut, dtype):
    """fp64 dequantised D: D[i, j] = lut[i, codes[i, j]] (stored level, widened)."""
    L = widen(lut, dtype)
    rows = np.arange(L.shape[0])[:, None]
    return L[rows, np.asarray(codes, dtype=np.int64)]


def split_dense_sparse(W, dtype, k=None, bits=4):
    """Dense-and-sparse form of W: the k outliers (default 0.5 %) as CSR, the
    residual quantised per row.  Returns dict(row_ptr, col_idx, values, lut,
    codes, codes_packed, residual, mask)."""
    m, n = W.shape
    s = split_csr(W, dtype, outlier_count(m, n) if k is None else k)
    lut, codes = quantize_rows(s["residual"], dtype, bits)
    s.update(lut=lut, codes=codes, codes_packed=pack_nibbles(codes) if bits == 4 else None)
    return s


# ---------------------------------------------------------------------------
# Hierarchical variant ([HSS] section "順列と階層的整列"): concentration ratio,
# Reverse Cuthill-McKee order, 2 x 2 block low-rank factors
# ---------------------------------------------------------------------------

def concentration_ratio(W, dtype, perm=None):
    """rho = sum |W'| over the two diagonal blocks / sum |W'|, W' = W with rows
    and columns in the order perm (identity when None); blocks split at
    m // 2 and n // 2.  0 for an all-zero matrix."""
    a = magnitudes(W, dtype)
    if perm is not None:
        p = np.asarray(perm, dtype=np.int64)
        a = a[p][:, p]
    m, n = a.shape
    m1, n1 = m // 2, n // 2
    total = a.sum()
    if total == 0:
        return 0.0
    return float((a[:m1, :n1].sum() + a[m1:, n1:].sum()) / total)


def rcm_graph(n, row_ptr, col_idx):
    """Neighbour sets of the symmetric graph of a square CSR pattern (i != j)."""
    nbr = [set() for _ in range(n)]
    for i in range(n):
        for p in range(int(row_ptr[i]), int(row_ptr[i + 1])):
            j = int(col_idx[p])
            if j != i:
                nbr[i].add(j)
                nbr[j].add(i)
    return nbr


def rcm_order(n, row_ptr, col_idx):
    """Reverse Cuthill-McKee order of the pattern (module notes):
    perm[i] = original index placed at position i."""
    nbr = rcm_graph(n, row_ptr, col_idx)
    deg = [len(s) for s in nbr]
    seen = [False] * n
    order = []
    while len(order) < n:
        start = min((v for v in range(n) if not seen[v]), key=lambda v: (deg[v], v))
        seen[start] = True
        queue = [start]
        head = 0
        while head < len(queue):
            u = queue[head]
            head += 1
            for v in sorted((v for v in nbr[u] if not seen[v]), key=lambda v: (deg[v], v)):
                seen[v] = True
                queue.append(v)
        order.extend(queue)
    return np.array(order[::-1], dtype=np.int32)


def bandwidth(n, row_ptr, col_idx, perm=None):
    """max |pos(i) - pos(j)| over the pattern's entries, positions after perm."""
    pos = np.arange(n) if perm is None else np.argsort(np.asarray(perm))
    bw = 0
    for i in range(n):
        for p in range(int(row_ptr[i]), int(row_ptr[i + 1])):
            bw = max(bw, abs(int(pos[i]) - int(pos[int(col_idx[p])])))
    return bw


def hier_factors(R64p, r_diag, r_off):
    """Truncated SVD of each block of the (permuted) residual, blocks split at
    m // 2 and n // 2: rank r_diag on the diagonal blocks, r_off off it (each
    capped at the block's smaller side).  Returns {(bi, bj): (U, V)}, U
    (block rows) x r and V (block columns) x r, U carrying the singular values."""
    R64p = np.asarray(R64p, dtype=np.float64)
    m, n = R64p.shape
    rows = [(0, m // 2), (m // 2, m)]
    cols = [(0, n // 2), (n // 2, n)]
    out = {}
    for bi in range(2):
        for bj in range(2):
            blk = R64p[rows[bi][0]:rows[bi][1], cols[bj][0]:cols[bj][1]]
            r = min(r_diag if bi == bj else r_off, min(blk.shape))
            U, V, _ = truncated_svd(blk, r)
            out[(bi, bj)] = (U, V)
    return out


def hier_param_count(k, m, n, r_diag, r_off):
    """Stored parameters of the one-level 2 x 2 form: k sparse values plus, for
    each block, (its rows + its columns) * its rank -- r_diag on the blocks
    (0, 0) and (1, 1), r_off on (0, 1) and (1, 0); rows split at m // 2,
    columns at n // 2.  Ranks are taken as given (no clamp to a block's side)."""
    m1, n1 = m // 2, n // 2
    m2, n2 = m - m1, n - n1
    return int(k) + (m1 + n1 + m2 + n2) * r_diag + (m1 + n2 + m2 + n1) * r_off


def hier_lowrank_dense(blocks, perm, m, n):
    """The block low-rank term as a dense m x n matrix in the original order:
    block (bi, bj) of the permuted matrix is U V^T, and permuted position
    (i, j) is original (perm[i], perm[j]) (identity when perm is None; then
    m and n may differ)."""
    Lp = np.zeros((m, n))
    for (bi, bj), (U, V) in blocks.items():
        r0, r1 = (0, m // 2) if bi == 0 else (m // 2, m)
        c0, c1 = (0, n // 2) if bj == 0 else (n // 2, n)
        Lp[r0:r1, c0:c1] = U @ V.T
    if perm is None:
        return Lp
    p = np.asarray(perm, dtype=np.int64)
    L = np.zeros((m, n))
    L[np.ix_(p, p)] = Lp
    return L


def csr_permute(n, row_ptr, col_idx, perm):
    """S' = P S P^T of a square n x n CSR pattern, S'[i, j] = S[perm[i],
    perm[j]]: (row_ptr', col_idx', src) with each row's columns ascending;
    entry q of S' is entry src[q] of S (values' = values[src]).  Row i of S'
    is row perm[i] of S with every column c renamed to its position pos[c]
    (pos = the inverse of perm)."""
    perm = np.asarray(perm, dtype=np.int64)
    pos = np.empty(n, dtype=np.int64)
    pos[perm] = np.arange(n)
    rp = np.asarray(row_ptr, dtype=np.int64)
    ci = np.asarray(col_idx, dtype=np.int64)
    out_rp = [0]
    out_ci, src = [], []
    for i in range(n):
        row = sorted((int(pos[ci[p]]), p) for p in range(rp[perm[i]], rp[perm[i] + 1]))
        out_ci.extend(c for c, _ in row)
        src.extend(p for _, p in row)
        out_rp.append(len(out_ci))
    return (np.array(out_rp, dtype=np.int32), np.array(out_ci, dtype=np.int32),
            np.array(src, dtype=np.int64))


def hier_apply(S64, blocks, perm, X64):
    """Y = X S^T + the block low-rank term applied through its factors: x' =
    x[perm], y'_block_rows += (x'_block_cols V) U^T, y[perm] += y'."""
    m, n = S64.shape
    p = np.arange(n) if perm is None else np.asarray(perm, dtype=np.int64)
    Xp = X64[:, p]
    Yp = np.zeros((X64.shape[0], m))
    for (bi, bj), (U, V) in blocks.items():
        r0, r1 = (0, m // 2) if bi == 0 else (m // 2, m)
        c0, c1 = (0, n // 2) if bj == 0 else (n // 2, n)
        Yp[:, r0:r1] += (Xp[:, c0:c1] @ V) @ U.T
    Y = X64 @ S64.T
    q = np.arange(m) if perm is None else np.asarray(perm, dtype=np.int64)
    Y[:, q] += Yp
    return Y



# ---------------------------------------------------------------------------
# Backward pass ([HSS] section "実装と運用パターン", the backward formulas: the
# gradients of S, U and V are computed separately, S's restricted to its
# stored positions).  With Y = X A^T, A = S + U V^T and G = dL/dY (b x m):
#   dA = G^T X (m x n), dS = dA on S's support, dU = dA V, dV = dA^T U,
# and the input gradient dX = G A (the layer's backward needs it too; the
# pages' formulas are written in the in x out orientation, these are the
# same quantities in this module's out x in one).
# ---------------------------------------------------------------------------

def csr_row_of_entry(m, row_ptr):
    """Row index of every stored entry, in storage order."""
    return np.repeat(np.arange(m, dtype=np.int64), np.diff(np.asarray(row_ptr, dtype=np.int64)))


def csr_transpose(m, n, row_ptr, col_idx):
    """S^T's CSR pattern (n rows) and perm with values_t = values[perm]:
    the stored entries ordered by (column, row)."""
    rows = csr_row_of_entry(m, row_ptr)
    cols = np.asarray(col_idx, dtype=np.int64)
    perm = np.lexsort((rows, cols))
    row_ptr_t = np.zeros(n + 1, dtype=np.int64)
    np.add.at(row_ptr_t, cols + 1, 1)
    return np.cumsum(row_ptr_t).astype(np.int32), rows[perm].astype(np.int32), perm.astype(np.int64)


def backward(m, n, row_ptr, col_idx, S64, U64, V64, X64, G64):
    """fp64 gradients of L with dL/dY = G: dX (b x n), dS (values, storage
    order), dU (m x r), dV (n x r)."""
    dA = G64.T @ X64
    rows = csr_row_of_entry(m, row_ptr)
    dS = dA[rows, np.asarray(col_idx, dtype=np.int64)]
    return {"dX": G64 @ (S64 + U64 @ V64.T), "dS": dS, "dU": dA @ V64, "dV": dA.T @ U64}


def backward_normalisers(m, n, row_ptr, col_idx, S64, U64, V64, X64, G64):
    """Per-output scales of the gradients' error bounds (the same sums with
    every term's magnitude): dS_p ~ sum_c |G_ci X_cj|, dU ~ |G|^T |X| |V|,
    dV ~ |X|^T |G| |U|, dX ~ |G| |S + U V^T|."""
    aG, aX = np.abs(G64), np.abs(X64)
    rows = csr_row_of_entry(m, row_ptr)
    NS = (aG.T @ aX)[rows, np.asarray(col_idx, dtype=np.int64)]
    return {"dX": aG @ np.abs(S64 + U64 @ V64.T), "dS": NS, "dU": aG.T @ (aX @ np.abs(V64)),
            "dV": aX.T @ (aG @ np.abs(U64))}


def backward_sampled(rows, cols, ent_rows, ent_cols, U64, V64, X64, G64):
    """The same gradients on a sample, for full-size checks: dU's rows
    `rows` (= G[:, rows]^T X V), dV's rows `cols` (= X[:, cols]^T G U) and dS
    at the positions (ent_rows[e], ent_cols[e]) (= sum_c G[c, i] X[c, j]),
    each with its error-bound scale (the same sums of magnitudes)."""
    aG, aX = np.abs(G64), np.abs(X64)
    XV, GU = X64 @ V64, G64 @ U64
    dS = np.sum(G64[:, ent_rows] * X64[:, ent_cols], axis=0)
    NS = np.sum(aG[:, ent_rows] * aX[:, ent_cols], axis=0)
    return {"dU": G64[:, rows].T @ XV, "dV": X64[:, cols].T @ GU, "dS": dS,
            "NU": aG[:, rows].T @ (aX @ np.abs(V64)), "NV": aX[:, cols].T @ (aG @ np.abs(U64)), "NS": NS}


def nm24_pattern(m, n, nm_meta):
    """The stored positions of a 2:4 matrix as a CSR pattern, in storage order
    (entry 2g + s of row i is the s-th kept column of group g), so that its
    values array is nm_values flattened: row_ptr[i] = i n / 2."""
    meta = np.asarray(nm_meta, dtype=np.uint32).reshape(m, -1)
    cols = np.zeros((m, n // 2), dtype=np.int64)
    for g in range(n // 4):
        nib = (meta[:, g // 8] >> np.uint32(4 * (g % 8))) & np.uint32(0xF)
        cols[:, 2 * g] = 4 * g + (nib & 3)
        cols[:, 2 * g + 1] = 4 * g + ((nib >> 2) & 3)
    row_ptr = (np.arange(m + 1, dtype=np.int64) * (n // 2)).astype(np.int32)
    return row_ptr, cols.reshape(-1).astype(np.int32)
