/*
 * hss.h -- C ABI of the sparse + low-rank (HSS) linear layer for AMD MI355X (gfx950).
 *
 *   W  ~=  S + U V^T          W: m x n (out features x in features)
 *   Y   =  X (S + U V^T)^T     X: b x n,  Y: b x m   (row-major)
 *
 * Sources (web pages; section names as printed on each page):
 *   [HSS]    "LLMの階層的スパース+低ランク圧縮" (hierarchical sparse + low-rank
 *            compression of LLMs), d7fyzohlfz9vz.cloudfront.net/posts/
 *            hierarchical-sparse-plus-low-rank-compression-of-llm
 *            section "2段階階層的スパース+低ランク圧縮": the decomposition
 *            W ~= S + U V^T, U in R^{m x r}, V in R^{n x r}; stage 1 keeps the
 *            weights of largest absolute magnitude as S (stored as indices +
 *            values, e.g. CSR), stage 2 factors the dense residual.
 *            section "実装と運用パターン": the forward product splits into the
 *            sparse product plus two small dense products.
 *   [HASSLE] aibr.jp/archives/82335, section "3.中核となる技術的要素": N:M
 *            (here 2:4) structured sparsity as the GPU-friendly form of S.
 *   [SQZ]    aibr.jp/archives/208940 (SqueezeLLM explainer), section
 *            "3.中核となる技術的要素": the dense-and-sparse decomposition W = D + S,
 *            the rare outliers kept exactly as a sparse (CSR) matrix and the
 *            dense rest quantised with non-uniform levels.
 *
 * Conventions shared by every call
 *   - Every pointer is a caller-owned DEVICE pointer unless stated otherwise.
 *     The library never allocates or frees memory.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = legacy default
 *     stream) and never synchronise, except hss_get_error.
 *   - All argument checks run on the host before any device work: a call that
 *     returns an error has enqueued nothing.
 *   - Storage types: HSS_F32 = IEEE binary32; HSS_BF16 = bfloat16 (upper 16
 *     bits of binary32).  Matrices are dense row-major unless stated.
 *   - Sizes are int32; every array addressed by the library must have fewer
 *     than 2^31 elements.
 *   - Calls are thread-safe given distinct workspaces; two calls that share a
 *     workspace must be ordered (same stream or explicit events).
 */
#ifndef HSS_H
#define HSS_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HSS_VERSION_MAJOR 1
#define HSS_VERSION_MINOR 7

/* Largest batch (columns of X) one hss_apply / hss_apply_group / hss_grad
 * call takes: decode (1) up to a prefill of 2048 tokens. */
#define HSS_MAX_BATCH 2048

typedef enum {
  HSS_OK = 0,
  HSS_ERR_INVALID_ARG = 1, /* bad size, null pointer, aliasing, unknown enum          */
  HSS_ERR_UNSUPPORTED = 2, /* valid request the library does not implement          */
  HSS_ERR_WORKSPACE = 3,   /* workspace pointer null or smaller than *_workspace_size */
  HSS_ERR_NONFINITE = 4,   /* device-side: a NaN/Inf weight was seen by hss_split     */
  HSS_ERR_HIP = 5          /* a HIP runtime call or kernel launch failed              */
} hss_status;

typedef enum { HSS_F32 = 0, HSS_BF16 = 1 } hss_dtype;

typedef enum {
  HSS_FMT_CSR = 0,  /* unstructured top-k, compressed sparse rows          */
  HSS_FMT_2OF4 = 1  /* 2 kept of every 4 consecutive columns (N:M = 2:4)   */
} hss_format;

/* Library version: 100 * major + minor. */
int hss_version(void);

/* Process-wide diagnostic switches, for comparing execution routes and for
 * testing the decode kernel's fallback.  Each starts at the value of the
 * environment variable named below (read once, at the first lookup), else
 * at its default; hss_set_option changes it for every later call.  Changing
 * a switch while another thread is inside a call of this library gives that
 * call either value.
 *   HSS_OPT_BATCH_ROUTE   (HSS_CSR_BATCH_ROUTE = decode | spmm | densify |
 *       smfmac): 0 = by batch size (default), 1 = the fused decode kernel,
 *       2 = the gather SpMM, 3 = densify + matrix cores, 4 = the sparse
 *       matrix cores; forces a bf16 call with b >= 2 onto that route where
 *       the route supports the matrix.  Workspace sizes cover every route.
 *   HSS_OPT_GRAD_DS_ROUTE (HSS_GRAD_DS_ROUTE = sparse | dense): 0 = by batch
 *       size (default), 1 = sampled product, 2 = dense G^T X then gather.
 *       Query hss_grad_workspace_size with the same setting.
 *   HSS_OPT_DECODE_SPIN   (HSS_DECODE_SPIN = count): polls of a stale T word
 *       before a block computes that T row itself (default 4096).
 *   HSS_OPT_DECODE_MERGED (HSS_DECODE_MERGED = 0): 1 (default) = T rows
 *       produced inside the row blocks where they fit, 0 = separate
 *       producer blocks.
 *   HSS_OPT_DECODE_FORCE_LOCAL: 1 = every decode block ignores the T words
 *       and computes every T row itself (same arithmetic, same bits), to
 *       test that fallback; default 0.
 *   HSS_OPT_DECODE_WAVE_PRODUCERS (HSS_DECODE_WAVE_PRODUCERS = 0): 1
 *       (default) = in one-column bf16 decode launches with separate
 *       producer blocks and n <= 4096, each wave of a producer block makes
 *       one T row (same bits); 0 = one T row per producer block.
 *   HSS_OPT_DECODE_RPW (HSS_DECODE_RPW = 1 | 2 | 4): output rows per wave of
 *       the decode kernel's row blocks (launches that merge the T producers
 *       into the row blocks choose their own); 0 (default) = by matrix
 *       height: 1 below 2048 rows, else 4 for one column and, for more
 *       columns, 2 below 8192 rows, else 4.  Bits do not depend on it.
 * hss_set_option returns HSS_ERR_INVALID_ARG for an unknown option or a
 * value out of range (routes 0..4 / 0..2, spin >= 0, flags 0..1, rows per
 * wave 0, 1, 2 or 4);
 * hss_get_option returns -1 for an unknown option. */
typedef enum {
  HSS_OPT_BATCH_ROUTE = 0,
  HSS_OPT_GRAD_DS_ROUTE = 1,
  HSS_OPT_DECODE_SPIN = 2,
  HSS_OPT_DECODE_MERGED = 3,
  HSS_OPT_DECODE_FORCE_LOCAL = 4,
  HSS_OPT_DECODE_WAVE_PRODUCERS = 5,
  HSS_OPT_DECODE_RPW = 6
} hss_option;
hss_status hss_set_option(int32_t opt, int32_t value);
int32_t hss_get_option(int32_t opt);

/* Entry points take enumerations (hss_format, hss_dtype, hss_option,
 * hss_status) as int32_t, so that a value outside the enumeration is a
 * rejected argument rather than undefined behaviour. */

/* Static text for a status code (never NULL; "HSS: unknown status" for a
 * value that is none). */
const char* hss_status_string(int32_t s);

/* Number of weights stage 1 keeps for a kept fraction num/den:
 *   floor(m * n * num / den), exact integer arithmetic ([HSS] worked example:
 *   5 % of 1024 x 1024 keeps 52,428).  Returns -1 if m, n, num < 0, den <= 0
 *   or the product overflows int64. */
int64_t hss_topk_count(int64_t m, int64_t n, int64_t num, int64_t den);

/* ------------------------------------------------------------------------
 * Stage 1: hss_split -- magnitude top-k of W into S, plus the residual.
 * ------------------------------------------------------------------------
 * [HSS] two-stage section: S holds the k weights of largest |w|; the rest form
 * the dense residual that stage 2 factors.
 *
 * Selection rule (exact, deterministic):
 *   key(w) = |w| (the bit pattern with the sign cleared; |+0| = |-0|).
 *   Order entries by key descending, then by row-major linear index i*n+j
 *   ascending, and keep the first k.  Exactly k entries are kept even when
 *   many share the threshold magnitude.
 *
 * fmt = HSS_FMT_CSR:
 *   k         in [0, m*n].
 *   row_ptr   int32[m+1]  out: row_ptr[0] = 0, row_ptr[m] = k.
 *   col_idx   int32[k]    out: column of each kept entry, ascending within a row.
 *   values    dt[k]       out: the kept W values, bit-copied.
 *   nm_values, nm_meta    must be NULL.
 *   col_idx / values may be NULL only when k == 0.
 * fmt = HSS_FMT_2OF4  ([HASSLE] N:M structure, groups along the input dim):
 *   n % 4 == 0 required; k must be m*n/2 or -1.
 *   In every group of 4 consecutive columns (4g .. 4g+3) of every row, keep the
 *   2 entries of largest |w|, ties to the lower column.
 *   nm_values dt[m * n/2]          out: row i, group g: [2g] = kept entry with
 *                                  the lower column, [2g+1] = the higher one.
 *   nm_meta   uint32[m * ceil(n/32)] out: row i, word g/8, bits 4*(g%8) .. +3
 *                                  hold i0 | (i1 << 2), i0 < i1 the kept
 *                                  positions within the group; unused bits 0.
 *   row_ptr, col_idx, values must be NULL.
 * residual  dt[m*n], nullable: out: W with every kept position set to +0 and
 *           every other position bit-copied (no arithmetic).
 * W         dt[m*n] in, row-major.  Must not overlap any output.
 * ws        workspace of at least hss_split_workspace_size() bytes; no
 *           initial contents required.  After the split, hss_get_error(ws)
 *           reports HSS_ERR_NONFINITE if W held a NaN or an infinity (the
 *           outputs are then unspecified).
 * Returns HSS_ERR_INVALID_ARG for: unknown fmt/dt, m or n <= 0, m*n >= 2^31,
 *   W null, k out of range, required output null, a forbidden output non-NULL,
 *   n % 4 != 0 for 2:4, residual aliasing W.  HSS_ERR_WORKSPACE for a null or
 *   short workspace.  HSS_ERR_HIP if a launch fails.
 */
hss_status hss_split_workspace_size(int32_t fmt, int32_t dt, int32_t m, int32_t n,
                                    size_t* bytes);
hss_status hss_split(int32_t fmt, int32_t dt, int32_t m, int32_t n, const void* W, int64_t k,
                     int32_t* row_ptr, int32_t* col_idx, void* values, void* nm_values,
                     uint32_t* nm_meta, void* residual, void* ws, size_t ws_bytes,
                     hipStream_t stream);

/* Reads the device error word a split left in `ws`: synchronises `stream`.
 * Returns HSS_OK, HSS_ERR_NONFINITE, HSS_ERR_INVALID_ARG (ws NULL) or HSS_ERR_HIP. */
hss_status hss_get_error(const void* ws, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Apply: Y = X S^T + (X V) U^T   ([HSS] implementation-patterns section)
 * ------------------------------------------------------------------------
 * The compressed matrix.  All arrays are device memory in `dtype` unless
 * stated.  r = 0 means no low-rank term (U, Vt ignored).
 *   fmt == HSS_FMT_CSR:  row_ptr int32[m+1], col_idx int32[nnz] (each row's
 *     columns in [0, n), strictly ascending -- the order hss_split writes),
 *     values dtype[nnz]; nnz = row_ptr[m].
 *     The nm_* fields are ignored.
 *   fmt == HSS_FMT_2OF4: nm_values dtype[m*n/2], nm_meta uint32[m*ceil(n/32)]
 *     in the layout hss_split writes; CSR fields ignored.
 *   flags & HSS_COL16: col_idx points to uint16[nnz] columns instead of
 *     int32 (n <= 65536), 2 bytes per entry less to read ([HSS] implementation
 *     section: narrower indices for the stored sparse part).  Convert the
 *     int32 columns hss_split writes with hss_csr_cols_to_u16.
 *   U  dtype[m*r]  row-major m x r.  bf16 U 16-byte aligned takes the
 *                  vector path for any r: U is read as the aligned 16-byte
 *                  pieces that cover each row, so the last piece may reach
 *                  up to 14 bytes past U's end (inside the same aligned 16
 *                  bytes, never into another page).
 *   Vt dtype[r*n]  the n x r factor V of the pages stored column-major
 *                  (equivalently V^T row-major, r x n), so that each of the r
 *                  dot products of T = V^T x reads one contiguous stream.
 *                  hss_transpose turns a row-major V into this form once per
 *                  weight.
 *   flags & HSS_DQ4: a quantised dense part D is added to the layer
 *     ([SQZ] dense-and-sparse: W ~= D + S with S the outliers, e.g. the top
 *     0.5 % by |w| from hss_split, and D the residual quantised offline):
 *       dq_codes  uint8[m*n/2]  row i, byte j holds the 4-bit codes of
 *                 columns 2j (low nibble) and 2j+1 (high nibble);
 *       dq_levels dtype[m*16]   row i's 16 levels;
 *       D[i][j] = dq_levels[16 i + code(i, j)].
 *     Requires fmt == HSS_FMT_CSR, n even and r == 0 (a dense part together
 *     with a low-rank term returns HSS_ERR_UNSUPPORTED).
 *   flags & HSS_HIER2: the low-rank term is the one-level 2 x 2 block form
 *     ([HSS] section "順列と階層的整列": a higher rank on the diagonal blocks
 *     than off them) held compactly, with no zeros: rows split at m0 = m/2,
 *     columns at n0 = n/2, block b = (bi, bj) in the order 00, 01, 10, 11 of
 *     rank hier_r[b] is U_b (rows of half bi) times V_b^T (columns of half
 *     bj), and the term is their sum, each on its own block.  The matrix is
 *     in the basis the blocks are defined in: for a layer reordered by a
 *     permutation P (hss_rcm_order), S, X and Y are all in the permuted
 *     order (S' = P S P^T from hss_csr_permute, x' = x[perm], y[perm[i]] =
 *     y'[i]), as when P is folded into the neighbouring layers.
 *       r  = hier_r[0] + hier_r[1] + hier_r[2] + hier_r[3];
 *       ru = hier_r[0] + hier_r[1] = hier_r[2] + hier_r[3] (required);
 *       U  dtype[m*ru]: row i < m0 holds [U_00 row i | U_01 row i], row
 *          i >= m0 holds [U_10 row i - m0 | U_11 row i - m0];
 *       Vt dtype[r * (n - n0)]: row o_b + l (o_b = hier_r[0] + ... +
 *          hier_r[b-1]) holds row l of V_b^T, the n0 (bj = 0) or n - n0
 *          (bj = 1) values of its column half, first; rows are n - n0 long
 *          (with odd n the last value of a first-half row is not read).
 *     hss_hier_pack_compact writes U and Vt from the four blocks.  Requires
 *     fmt == HSS_FMT_CSR, no HSS_DQ4, m >= 2, n >= 2, every hier_r[b] >= 0.
 *     Up to 8 columns per pass the fused decode kernel reads the compact
 *     factors directly; wider batches first expand them into flat m x r /
 *     r x n factors inside the workspace (hss_apply_workspace_size counts
 *     them).  hss_grad does not take HSS_HIER2 (HSS_ERR_UNSUPPORTED).
 */
#define HSS_COL16 1
#define HSS_DQ4 2
#define HSS_HIER2 4

typedef struct hss_matrix {
  int32_t fmt;   /* hss_format */
  int32_t dtype; /* hss_dtype  */
  int32_t m, n, r;
  int32_t flags;    /* 0, or HSS_COL16 (CSR only: col_idx holds uint16 columns) */
  int64_t nnz;      /* CSR: row_ptr[m] (>= 0); 2:4: ignored */
  const int32_t* row_ptr;
  const int32_t* col_idx;
  const void* values;
  const void* nm_values;
  const uint32_t* nm_meta;
  const void* U;
  const void* Vt;
  const uint8_t* dq_codes; /* HSS_DQ4 only (else ignored) */
  const void* dq_levels;   /* HSS_DQ4 only (else ignored) */
  int32_t hier_r[4];       /* HSS_HIER2 only (else ignored): block ranks, order 00, 01, 10, 11 */
} hss_matrix;

/* out[i] = (uint16) col_idx[i] for i < nnz, on `stream`: the 16-bit column
 * array of an HSS_COL16 matrix.  Requires 0 < n <= 65536 (every column fits);
 * col_idx and out must not overlap.  Returns HSS_ERR_INVALID_ARG for bad
 * arguments (nnz < 0, n out of range, null arrays with nnz > 0), HSS_ERR_HIP if
 * the launch fails. */
hss_status hss_csr_cols_to_u16(const int32_t* col_idx, int64_t nnz, int32_t n, uint16_t* out,
                               hipStream_t stream);

/* Workspace bytes hss_apply needs for this matrix and batch size. */
hss_status hss_apply_workspace_size(const hss_matrix* A, int32_t b, size_t* bytes);

/* Y (b x m, row-major) = X (b x n, row-major) times (S + U V^T)^T, plus the
 * quantised dense part D for HSS_DQ4 matrices: X (S + D)^T.
 *   HSS_F32 : X, Y fp32; accumulation fp32.
 *   HSS_BF16: X bf16; products accumulated in fp32; Y bf16 = round-to-nearest-
 *             even of the fp32 result.
 * ws: at least hss_apply_workspace_size() bytes, initialised ONCE by
 *     hss_apply_workspace_init before its first apply.  The fused decode
 *     kernel keeps state in it from call to call: a 32-bit call epoch, 64
 *     arrival counters (all in the first 16 KiB) and the tagged words through
 *     which its blocks hand T = V^T x to each other (a word is used only when
 *     its tag is the current epoch + 1, so a word left by an earlier call is
 *     never taken for this one's).  The caller must not write to the
 *     workspace after the init.  Any number of calls, with any matrices and
 *     batch sizes, may share one workspace if they are ORDERED (one stream,
 *     or events between streams); two calls that overlap in time must use
 *     different workspaces -- overlapping calls on one workspace can make
 *     both return wrong values with no error.  The epoch wraps after 2^32 - 1
 *     calls and skips the tag that a zero-filled word carries.
 * Execution: bf16 2:4 with 3 <= b <= 64 (n % 128 == 0; nm_values, nm_meta
 * and X 16-byte aligned) runs on the sparse matrix cores: S's stored values
 * and 2-bit indices are the operands of v_smfmac as they are, with fp32
 * accumulation, and T = X V is rounded to bf16 once before U T is added.  bf16 2:4 beyond 64
 * columns, and bf16 CSR with b > 128, run on the matrix cores (T^T = X V and
 * Y = [X | T^T] [S | U]^T as MFMA GEMMs with fp32 accumulation; T is rounded
 * to bf16 once, between the two; a CSR S is first expanded into a dense bf16
 * copy inside the workspace, so the workspace then holds m*n*2 more bytes).
 * bf16 CSR with 3 <= b <= 128 runs the gather SpMM (T = X V rounded to bf16
 * once, X^T staged in the workspace, then every stored entry gathers its X^T
 * row; fp32 accumulation).  Otherwise one fused kernel per 8 columns (T =
 * X V accumulated in fp32; for bf16 matrices whose U is 16-byte aligned it is
 * rounded to bf16 once before U T is added, as on every other route; fp32
 * matrices keep it in fp32).  On
 * the matrix-core routes (the sparse one included) zeros in an operand
 * multiply X too, so a NaN or infinity in X can reach any output of its
 * batch row.  HSS_OPT_BATCH_ROUTE (hss_set_option) forces a bf16 call with
 * b >= 2 onto one route, for comparing them.
 * HSS_DQ4 matrices always run the fused dense-and-sparse kernel (up to 8
 * columns per pass; no workspace: hss_apply_workspace_size returns 0 and ws
 * may be NULL).
 * Returns HSS_ERR_INVALID_ARG for: A or X or Y null, unknown fmt/dtype,
 *   unknown flags (or HSS_COL16 with a 2:4 matrix or n > 65536; HSS_DQ4 with
 *   a 2:4 matrix, odd n or null dq arrays),
 *   m, n <= 0, r < 0, b < 1 or b > HSS_MAX_BATCH, b*m, b*n, m*n,
 *   r*(m+n) >= 2^31,
 *   nnz < 0, required arrays null, n % 4 != 0 for 2:4, X overlapping Y.
 *   HSS_ERR_WORKSPACE for a null or short workspace.  HSS_ERR_HIP if a launch
 *   fails.
 */
hss_status hss_apply(const hss_matrix* A, int32_t b, const void* X, void* Y, void* ws,
                     size_t ws_bytes, hipStream_t stream);

/* hss_apply without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  Same arguments, arithmetic, routes and errors as
 * hss_apply, with the workspace replaced by a scratch array that the library
 * holds in each GPU's memory: hss_noalloc_scratch_bytes() bytes (16 MiB),
 * kept until the process ends, and cleared by the first call on each device
 * (on that call's stream).  The call allocates and frees nothing.
 * HSS_ERR_WORKSPACE when the route this call takes needs more workspace
 * than the scratch holds (e.g. a large CSR layer densified for the matrix
 * cores at prefill batches): use hss_apply with a workspace of
 * hss_apply_workspace_size() bytes for those.  Every call on one GPU shares
 * that GPU's scratch, which keeps the last call's state: calls that overlap
 * in time on one GPU (other streams or threads) race and can return wrong
 * values with no error, so order them (one stream, or events).
 * HSS_ERR_HIP if the scratch's device address cannot be looked up or a
 * launch fails. */
hss_status hss_apply_noalloc(const hss_matrix* A, int32_t b, const void* X, void* Y, hipStream_t stream);
size_t hss_noalloc_scratch_bytes(void);

/* Puts an apply workspace (ws_bytes bytes, device) in its initial state, on
 * `stream`: every byte zero, written by a kernel (no memset node, so the call
 * may also be captured into a HIP graph).  Call it once per workspace before
 * its first hss_apply / hss_apply_group, and again only when no call using
 * the workspace can still be running.  ws_bytes == 0 does nothing.
 * HSS_ERR_INVALID_ARG for a null ws with ws_bytes > 0; HSS_ERR_HIP if the
 * launch fails. */
hss_status hss_apply_workspace_init(void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Grouped apply: G matrices that read the same X, e.g. the q, k and v
 * projections of one attention block, or gate and up of one MLP block
 * ([HSS] implementation-patterns section: the compressed layers run layer by
 * layer; these share their input).
 * ------------------------------------------------------------------------
 * Y[g] (b x A[g]->m) = X (b x n) times (S_g + U_g V_g^T)^T for g < G, to
 * hss_apply's bound.  The bits can differ from a single hss_apply of the
 * same matrix where the two calls take different launch plans (a lone
 * matrix may produce its T rows inside its row blocks, which sums them in a
 * different order); every call is deterministic.  In the decode regime
 * (everything hss_apply runs in its fused kernel) all G matrices go through
 * ONE launch per pass of up to 8 columns instead of G; on the matrix cores
 * the matrices are applied one after another.
 *   1 <= G <= HSS_MAX_GROUP; every A[g] valid for hss_apply with batch b, all
 *   with the same n, dtype and fmt (m, r and the arrays may differ).
 *   Y[g] device outputs, pairwise disjoint and disjoint from X.
 *   ws: at least hss_apply_group_workspace_size() bytes, initialised once
 *   by hss_apply_workspace_init; the same state rules as hss_apply (it may
 *   also serve hss_apply calls).
 * Returns HSS_ERR_INVALID_ARG for: A, X or Y null, G out of range, any matrix
 *   invalid, mismatched n/dtype/fmt, overlapping outputs; HSS_ERR_WORKSPACE for
 *   a null or short workspace; HSS_ERR_HIP if a launch fails.
 */
#define HSS_MAX_GROUP 4
hss_status hss_apply_group_workspace_size(const hss_matrix* const* A, int32_t G, int32_t b, size_t* bytes);
hss_status hss_apply_group(const hss_matrix* const* A, int32_t G, int32_t b, const void* X, void* const* Y,
                           void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Hierarchical variant ([HSS] section "順列と階層的整列", vision rewrite
 * "置換と階層的整列"): reorder rows and columns so that the large weights sit
 * near the diagonal, measure how much magnitude the diagonal blocks hold,
 * and factor the residual block by block (a higher rank on the two diagonal
 * blocks than off them).  One level of 2 x 2 blocks: rows split at m / 2,
 * columns at n / 2.
 * ------------------------------------------------------------------------
 *
 * hss_rcm_order: Reverse Cuthill-McKee order of a square n x n sparsity
 *   pattern given as CSR in HOST memory (e.g. the support of S from
 *   hss_split), computed on the host, synchronously.  Graph: i - j when the
 *   pattern has (i, j) or (j, i), i != j.  Each component is walked
 *   breadth-first from its unvisited node of lowest degree (then lowest
 *   index), a node's unvisited neighbours are queued by (degree, index)
 *   ascending, and the whole visit order is reversed.
 *   perm (HOST int32[n], out): perm[i] = the original index at position i;
 *   the permuted matrix is W'[i][j] = W[perm[i]][perm[j]].
 *   HSS_ERR_INVALID_ARG: n < 1, null arrays, row_ptr[0] != 0, decreasing
 *   row_ptr, a column outside [0, n).
 */
hss_status hss_rcm_order(int32_t n, const int32_t* row_ptr, const int32_t* col_idx, int32_t* perm);

/* hss_concentration: rho of W (m x n, dtype, device) in the order perm
 *   (device int32[n], a permutation of [0, n); m == n; NULL = identity):
 *     out[0] = rho = out[1] / out[2] (0 if out[2] == 0),
 *     out[1] = sum of |W'[i][j]| over the diagonal blocks (i < m/2 and
 *              j < n/2, or i >= m/2 and j >= n/2),
 *     out[2] = sum of |W|,
 *   out = 3 device doubles, W' = W with rows and columns in the order perm.
 *   Sums in fp64 in a fixed order (the same bits every call).
 *   ws: at least hss_concentration_workspace_size() bytes (no state kept).
 *   HSS_ERR_INVALID_ARG: bad dtype or size, null W or out, perm with m != n;
 *   HSS_ERR_WORKSPACE; HSS_ERR_HIP. */
hss_status hss_concentration_workspace_size(int32_t m, int32_t n, size_t* bytes);
hss_status hss_concentration(int32_t dt, int32_t m, int32_t n, const void* W, const int32_t* perm, double* out,
                             void* ws, size_t ws_bytes, hipStream_t stream);

/* hss_hier_pack: flat factors of the 2 x 2 block low-rank term, for the
 *   ordinary apply.  Block b = (bi, bj), in the order 00, 01, 10, 11, is
 *   U[b] (device, (rows of half bi) x r[b], row-major) times Vt[b] (device,
 *   r[b] x (columns of half bj), row-major) on the matrix permuted by perm
 *   (device int32[n], a permutation; m == n; NULL = identity).  Writes
 *     U_cat  (device, m x R, row-major) and Vt_cat (device, R x n), R = sum r[b],
 *   such that U_cat Vt_cat is the block term in the ORIGINAL order:
 *     U_cat[perm[i]][o_b + l] = U[b][i'][l] for the two blocks of i's row
 *     half (i' = i, or i - m/2), Vt_cat[o_b + l][perm[j]] = Vt[b][l][j'] for
 *     the columns j of block b's column half, zero elsewhere (o_b = r[0] +
 *     ... + r[b-1]).  A matrix with U = U_cat, Vt = Vt_cat and r = R then
 *     applies S + (block term) with hss_apply; the zeros double the factor
 *     bytes the blocks themselves hold.
 *   r, U, Vt: HOST arrays of 4 (the U and Vt entries are device pointers).
 *   A permutation entry outside [0, n) is skipped.
 *   HSS_ERR_INVALID_ARG: bad dtype, m or n < 2, r[b] < 0 or larger than its
 *   block's smaller side, null arrays, perm with m != n, m*R or R*n >= 2^31;
 *   HSS_ERR_HIP. */
hss_status hss_hier_pack(int32_t dt, int32_t m, int32_t n, const int32_t* r, const void* const* U,
                         const void* const* Vt, const int32_t* perm, void* U_cat, void* Vt_cat, hipStream_t stream);

/* hss_hier_pack_compact: the compact factors of an HSS_HIER2 matrix from its
 *   four blocks (layouts as documented at HSS_HIER2; bits copied, device
 *   arrays).  Block b = (bi, bj), in the order 00, 01, 10, 11: U[b] (rows
 *   of half bi) x r[b] and Vt[b] r[b] x (columns of half bj), row-major, in
 *   the blocks' own (permuted) order.  Writes U_c (m x ru, ru = r[0] + r[1]
 *   = r[2] + r[3]) and Vt_c (R x (n - n/2), R = sum r[b]); the unread last
 *   value of a first-half Vt_c row (odd n) is set to zero.
 *   r, U, Vt: HOST arrays of 4 (the U and Vt entries are device pointers;
 *   NULL for a rank-0 block).
 *   HSS_ERR_INVALID_ARG: bad dtype, m or n < 2, r[b] < 0 or larger than its
 *   block's smaller side, r[0] + r[1] != r[2] + r[3], null arrays,
 *   m*ru or R*n >= 2^31; HSS_ERR_HIP. */
hss_status hss_hier_pack_compact(int32_t dt, int32_t m, int32_t n, const int32_t* r, const void* const* U,
                                 const void* const* Vt, void* U_c, void* Vt_c, hipStream_t stream);

/* hss_csr_permute: the CSR pattern of S' = P S P^T, S'[i][j] =
 *   S[perm[i]][perm[j]], for a square n x n S (the sparse part of a layer
 *   reordered by perm, e.g. hss_rcm_order's), in HOST memory, computed on
 *   the host, synchronously (once per pattern): row_ptr_p (int32[n+1]) and
 *   col_idx_p (int32[nnz]) with each row's columns ascending; from
 *   (int32[nnz]): entry q of S' is entry from[q] of S (hss_gather_values
 *   moves the values).
 *   HSS_ERR_INVALID_ARG: n < 1, null arrays, row_ptr[0] != 0, decreasing
 *   row_ptr, a column outside [0, n), perm not a permutation of [0, n),
 *   repeated columns within a row. */
hss_status hss_csr_permute(int32_t n, const int32_t* row_ptr, const int32_t* col_idx, const int32_t* perm,
                           int32_t* row_ptr_p, int32_t* col_idx_p, int32_t* from);

/* ------------------------------------------------------------------------
 * Backward pass ([HSS] section "実装と運用パターン", the backward formulas):
 * the gradients of S, U and V are computed separately, S's restricted to
 * its stored positions.  With Y = X A^T, A = S + U V^T and G = dL/dY
 * (b x m): dA = G^T X, dS = dA on S's support, dU = dA V, dV = dA^T U.
 * The input gradient dX = G A is the forward apply of the transposed layer
 * A^T = S^T + V U^T, built with hss_csr_transpose, hss_gather_values and
 * hss_transpose and applied with hss_apply.
 * ------------------------------------------------------------------------
 *
 * hss_grad: parameter gradients of a bf16 layer, CSR or 2:4 (device arrays):
 *   X (b x n) and G (b x m) bf16, row-major;
 *   dS  (fp32, out; NULL = skip): dS[p] = sum_c G[c][i] X[c][j] for the
 *        stored entry p (row i, column j), in S's storage order: nnz values
 *        for CSR; m * n / 2 for 2:4, laid out as nm_values (entry 2g + s of
 *        row i is the s-th kept column of group g);
 *   dU  (fp32, m x r row-major, out; NULL = skip) = G^T (X V);
 *   dVt (fp32, r x n row-major, out; NULL = skip) = (G U)^T X, the gradient
 *        of the stored V^T.
 *   X V and G U are rounded to bf16 once (matrix-core GEMMs with fp32
 *   accumulation); every sum over the batch accumulates in fp32.  The same
 *   inputs give the same bits on every call.  dS is a sampled product on
 *   the vector units below 512 columns; from 512 on, the dense G^T X on the
 *   matrix cores (its m*n fp32 values in the workspace) then a gather
 *   (HSS_OPT_GRAD_DS_ROUTE forces one; query the workspace size with the
 *   same setting).
 *   ws: at least hss_grad_workspace_size() bytes (no state kept).
 *   HSS_ERR_UNSUPPORTED: an fp32 or dense-and-sparse layer, or
 *   n * round8(b) * 2 or m * round8(b) * 2 >= 2^31.  HSS_ERR_INVALID_ARG: as
 *   hss_apply, plus null X or G, or an output overlapping X, G or another
 *   output.  HSS_ERR_WORKSPACE; HSS_ERR_HIP. */
hss_status hss_grad_workspace_size(const hss_matrix* A, int32_t b, size_t* bytes);
hss_status hss_grad(const hss_matrix* A, int32_t b, const void* X, const void* G, float* dS, float* dU, float* dVt,
                    void* ws, size_t ws_bytes, hipStream_t stream);

/* hss_nm24_to_csr: the stored positions of a 2:4 matrix (m x n, nm_meta as
 *   in hss_matrix) as a CSR pattern on the device: row_ptr (int32[m+1]) =
 *   i n / 2, col_idx (int32[m n / 2]) in storage order, so that nm_values is
 *   its values array (a valid CSR: columns ascend within each row).  The
 *   transposed layer of a 2:4 layer starts from it.
 *   HSS_ERR_INVALID_ARG: m < 1, n < 4 or n % 4 != 0, m * n >= 2^31, null or
 *   overlapping arrays.  HSS_ERR_HIP. */
hss_status hss_nm24_to_csr(int32_t m, int32_t n, const uint32_t* nm_meta, int32_t* row_ptr, int32_t* col_idx,
                           hipStream_t stream);

/* hss_csr_transpose: the CSR pattern of S^T (n x m) from S's (m x n), in
 *   HOST memory, computed on the host, synchronously (once per pattern):
 *   row_ptr_t (int32[n+1]) and col_idx_t (int32[nnz]) with each row's
 *   entries ordered by original row; perm (int32[nnz]): entry q of S^T is
 *   entry perm[q] of S.
 *   HSS_ERR_INVALID_ARG: m or n < 1, null arrays, row_ptr[0] != 0,
 *   decreasing row_ptr, a column outside [0, n). */
hss_status hss_csr_transpose(int32_t m, int32_t n, const int32_t* row_ptr, const int32_t* col_idx, int32_t* row_ptr_t,
                             int32_t* col_idx_t, int32_t* perm);

/* hss_gather_values: values_t[q] = values[perm[q]] for q < nnz (device
 *   arrays, bits copied): S^T's values after each change of S's.
 *   perm must hold indices in [0, nnz).
 *   HSS_ERR_INVALID_ARG: bad dtype, nnz < 0 or >= 2^31, null arrays with
 *   nnz > 0, values overlapping values_t.  HSS_ERR_HIP. */
hss_status hss_gather_values(int32_t dt, int64_t nnz, const void* values, const int32_t* perm, void* values_t,
                             hipStream_t stream);

/* hss_transpose: dst (cols x rows, row-major) = src (rows x cols,
 *   row-major)^T, device arrays, bits copied (U^T and V for the transposed
 *   layer: its U is V = (stored V^T)^T, its V^T is U^T).
 *   HSS_ERR_INVALID_ARG: bad dtype, rows or cols < 1, rows * cols >= 2^31,
 *   rows > 2,097,120, null or overlapping arrays.  HSS_ERR_HIP. */
hss_status hss_transpose(int32_t dt, int32_t rows, int32_t cols, const void* src, void* dst, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* HSS_H */
