// Host entry points of libhss: argument checks, workspace sizing, dispatch.
// Every check runs before any HIP call, so an error return has enqueued nothing.
#include <limits.h>

#include <algorithm>
#include <atomic>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "hss_internal.h"

namespace hss {  // grad.hip
size_t grad_ws_bytes(const hss_matrix* A, int b);
hss_status launch_grad(const hss_matrix* A, int b, const void* X, const void* G, float* dS, float* dU, float* dVt,
                       void* ws, hipStream_t s);
hss_status csr_transpose_host(int m, int n, const int32_t* row_ptr, const int32_t* col_idx, int32_t* row_ptr_t,
                              int32_t* col_idx_t, int32_t* perm);
hss_status launch_gather_values(int dt, int64_t nnz, const void* values, const int32_t* perm, void* values_t,
                                hipStream_t s);
hss_status launch_transpose(int dt, int rows, int cols, const void* src, void* dst, hipStream_t s);
hss_status launch_nm_to_csr(int m, int n, const uint32_t* meta, int32_t* row_ptr, int32_t* col, hipStream_t s);
}  // namespace hss

// ---------------------------------------------------------------------------
// Diagnostic switches.  The first value of each comes from the environment
// (read once, when the first switch is looked up); hss_set_option changes it
// for the rest of the process.
// ---------------------------------------------------------------------------
namespace hss {

namespace {
constexpr int kNumOptions = 7;

int env_route(const char* name, const char* const* words, int nwords) {
  const char* e = std::getenv(name);
  if (!e) return 0;
  for (int i = 0; i < nwords; ++i)
    if (!std::strcmp(e, words[i])) return i + 1;
  return 0;
}

struct Options {
  std::atomic<int> v[kNumOptions];
  Options() {
    static const char* const batch[] = {"decode", "spmm", "densify", "smfmac"};
    static const char* const ds[] = {"sparse", "dense"};
    v[HSS_OPT_BATCH_ROUTE] = env_route("HSS_CSR_BATCH_ROUTE", batch, 4);
    v[HSS_OPT_GRAD_DS_ROUTE] = env_route("HSS_GRAD_DS_ROUTE", ds, 2);
    const char* spin = std::getenv("HSS_DECODE_SPIN");
    v[HSS_OPT_DECODE_SPIN] = spin ? std::max(0, atoi(spin)) : 4096;
    const char* merged = std::getenv("HSS_DECODE_MERGED");
    v[HSS_OPT_DECODE_MERGED] = (merged && merged[0] == '0') ? 0 : 1;
    v[HSS_OPT_DECODE_FORCE_LOCAL] = 0;
    const char* wp = std::getenv("HSS_DECODE_WAVE_PRODUCERS");
    v[HSS_OPT_DECODE_WAVE_PRODUCERS] = (wp && wp[0] == '0') ? 0 : 1;
    const char* rpw = std::getenv("HSS_DECODE_RPW");
    const int rv = rpw ? atoi(rpw) : 0;
    v[HSS_OPT_DECODE_RPW] = (rv == 1 || rv == 2 || rv == 4) ? rv : 0;
  }
};

Options& options() {
  static Options o;  // initialised once, thread-safe
  return o;
}
}  // namespace

int option(int opt) { return options().v[opt].load(std::memory_order_relaxed); }

}  // namespace hss

namespace {

constexpr int64_t kLimit = (int64_t)1 << 31;  // arrays must have fewer elements

bool valid_dtype(int dt) { return dt == HSS_F32 || dt == HSS_BF16; }
bool valid_fmt(int f) { return f == HSS_FMT_CSR || f == HSS_FMT_2OF4; }
size_t dsize(int dt) { return dt == HSS_F32 ? 4 : 2; }

bool overlap(const void* a, size_t abytes, const void* b, size_t bbytes) {
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + bbytes && b0 < a0 + abytes;
}

}  // namespace

extern "C" {

int hss_version(void) { return 100 * HSS_VERSION_MAJOR + HSS_VERSION_MINOR; }

hss_status hss_set_option(int32_t opt, int32_t value) {
  static const int32_t hi[] = {4, 2, INT32_MAX, 1, 1, 1, 4};
  if ((int)opt < 0 || (int)opt >= hss::kNumOptions || value < 0 || value > hi[opt]) return HSS_ERR_INVALID_ARG;
  if (opt == HSS_OPT_DECODE_RPW && value == 3) return HSS_ERR_INVALID_ARG;
  hss::options().v[opt].store(value, std::memory_order_relaxed);
  return HSS_OK;
}

int32_t hss_get_option(int32_t opt) {
  if ((int)opt < 0 || (int)opt >= hss::kNumOptions) return -1;
  return hss::option(opt);
}

hss_status hss_apply_workspace_init(void* ws, size_t ws_bytes, hipStream_t stream) {
  if (ws_bytes == 0) return HSS_OK;
  if (!ws) return HSS_ERR_INVALID_ARG;
  return hss::launch_zero_fill(ws, ws_bytes, stream);
}

const char* hss_status_string(int32_t s) {
  switch (s) {
    case HSS_OK: return "HSS_OK";
    case HSS_ERR_INVALID_ARG: return "HSS_ERR_INVALID_ARG: invalid argument";
    case HSS_ERR_UNSUPPORTED: return "HSS_ERR_UNSUPPORTED: not implemented for these arguments";
    case HSS_ERR_WORKSPACE: return "HSS_ERR_WORKSPACE: workspace missing or too small";
    case HSS_ERR_NONFINITE: return "HSS_ERR_NONFINITE: non-finite weight seen by hss_split";
    case HSS_ERR_HIP: return "HSS_ERR_HIP: HIP runtime error";
  }
  return "HSS: unknown status";
}

int64_t hss_topk_count(int64_t m, int64_t n, int64_t num, int64_t den) {
  if (m < 0 || n < 0 || num < 0 || den <= 0) return -1;
  __int128 p = (__int128)m * n * num;
  __int128 q = p / den;
  if (q > (__int128)INT64_MAX) return -1;
  return (int64_t)q;
}

hss_status hss_split_workspace_size(int32_t fmt, int32_t dt, int32_t m, int32_t n,
                                    size_t* bytes) {
  if (!bytes || !valid_fmt(fmt) || !valid_dtype(dt) || m <= 0 || n <= 0 ||
      (int64_t)m * n >= kLimit)
    return HSS_ERR_INVALID_ARG;
  *bytes = hss::split_ws_bytes(fmt, m);
  return HSS_OK;
}

hss_status hss_split(int32_t fmt, int32_t dt, int32_t m, int32_t n, const void* W, int64_t k,
                     int32_t* row_ptr, int32_t* col_idx, void* values, void* nm_values,
                     uint32_t* nm_meta, void* residual, void* ws, size_t ws_bytes,
                     hipStream_t stream) {
  if (!valid_fmt(fmt) || !valid_dtype(dt) || m <= 0 || n <= 0) return HSS_ERR_INVALID_ARG;
  const int64_t mn = (int64_t)m * n;
  if (mn >= kLimit || W == nullptr) return HSS_ERR_INVALID_ARG;
  const size_t wbytes = (size_t)mn * dsize(dt);
  if (residual && overlap(W, wbytes, residual, wbytes)) return HSS_ERR_INVALID_ARG;
  if (fmt == HSS_FMT_CSR) {
    if (k < 0 || k > mn) return HSS_ERR_INVALID_ARG;
    if (!row_ptr || (k > 0 && (!col_idx || !values))) return HSS_ERR_INVALID_ARG;
    if (nm_values || nm_meta) return HSS_ERR_INVALID_ARG;
  } else {
    if (n % 4 != 0) return HSS_ERR_INVALID_ARG;
    if (k != -1 && k != mn / 2) return HSS_ERR_INVALID_ARG;
    if (!nm_values || !nm_meta) return HSS_ERR_INVALID_ARG;
    if (row_ptr || col_idx || values) return HSS_ERR_INVALID_ARG;
  }
  const size_t need = hss::split_ws_bytes(fmt, m);
  if (!ws || ws_bytes < need) return HSS_ERR_WORKSPACE;
  if (fmt == HSS_FMT_CSR)
    return hss::launch_split_csr(dt, m, n, W, k, row_ptr, col_idx, values, residual, ws, stream);
  return hss::launch_split_24(dt, m, n, W, nm_values, nm_meta, residual, ws, stream);
}

hss_status hss_get_error(const void* ws, hipStream_t stream) {
  if (!ws) return HSS_ERR_INVALID_ARG;
  if (hipStreamSynchronize(stream) != hipSuccess) return HSS_ERR_HIP;
  uint32_t err = 0;
  if (hipMemcpy(&err, ws, sizeof(err), hipMemcpyDeviceToHost) != hipSuccess) return HSS_ERR_HIP;
  return err ? HSS_ERR_NONFINITE : HSS_OK;
}

static hss_status check_matrix(const hss_matrix* A, int32_t b) {
  if (!A || !valid_fmt(A->fmt) || !valid_dtype(A->dtype) || (A->flags & ~(HSS_COL16 | HSS_DQ4 | HSS_HIER2)) != 0)
    return HSS_ERR_INVALID_ARG;
  if ((A->flags & HSS_COL16) && (A->fmt != HSS_FMT_CSR || A->n > 65536)) return HSS_ERR_INVALID_ARG;
  const int64_t m = A->m, n = A->n, r = A->r;
  if (m <= 0 || n <= 0 || r < 0 || b < 1 || b > HSS_MAX_BATCH) return HSS_ERR_INVALID_ARG;
  if (A->flags & HSS_DQ4) {
    if (A->fmt != HSS_FMT_CSR || n % 2 != 0 || !A->dq_codes || !A->dq_levels) return HSS_ERR_INVALID_ARG;
    if (r > 0) return HSS_ERR_UNSUPPORTED;
  }
  if (A->flags & HSS_HIER2) {
    if (A->fmt != HSS_FMT_CSR || (A->flags & HSS_DQ4) || m < 2 || n < 2) return HSS_ERR_INVALID_ARG;
    int64_t sum = 0;
    for (int k = 0; k < 4; ++k) {
      if (A->hier_r[k] < 0) return HSS_ERR_INVALID_ARG;
      sum += A->hier_r[k];
    }
    if (sum != r || (int64_t)A->hier_r[0] + A->hier_r[1] != (int64_t)A->hier_r[2] + A->hier_r[3])
      return HSS_ERR_INVALID_ARG;
  }
  if (m * n >= kLimit || (int64_t)b * m >= kLimit || (int64_t)b * n >= kLimit ||
      r * (m + n) >= kLimit)
    return HSS_ERR_INVALID_ARG;
  if (r > 0 && (!A->U || !A->Vt)) return HSS_ERR_INVALID_ARG;
  if (A->fmt == HSS_FMT_CSR) {
    if (A->nnz < 0 || A->nnz > m * n || !A->row_ptr) return HSS_ERR_INVALID_ARG;
    if (A->nnz > 0 && (!A->col_idx || !A->values)) return HSS_ERR_INVALID_ARG;
  } else {
    if (n % 4 != 0 || !A->nm_values || !A->nm_meta) return HSS_ERR_INVALID_ARG;
  }
  return HSS_OK;
}

hss_status hss_csr_cols_to_u16(const int32_t* col_idx, int64_t nnz, int32_t n, uint16_t* out,
                               hipStream_t stream) {
  if (nnz < 0 || n <= 0 || n > 65536) return HSS_ERR_INVALID_ARG;
  if (nnz == 0) return HSS_OK;
  if (!col_idx || !out || overlap(col_idx, (size_t)nnz * 4, out, (size_t)nnz * 2)) return HSS_ERR_INVALID_ARG;
  return hss::launch_cols_to_u16(col_idx, nnz, out, stream);
}

hss_status hss_apply_workspace_size(const hss_matrix* A, int32_t b, size_t* bytes) {
  if (!bytes) return HSS_ERR_INVALID_ARG;
  hss_status st = check_matrix(A, b);
  if (st != HSS_OK) return st;
  *bytes = hss::apply_ws_bytes(A, b);
  return HSS_OK;
}

}  // extern "C"

// The argument checks of hss_apply (also those of hss_apply_noalloc).
hss_status hss::check_apply_args(const hss_matrix* A, int32_t b, const void* X, void* Y) {
  hss_status st = check_matrix(A, b);
  if (st != HSS_OK) return st;
  if (!X || !Y) return HSS_ERR_INVALID_ARG;
  const size_t es = dsize(A->dtype);
  if (overlap(X, (size_t)b * A->n * es, Y, (size_t)b * A->m * es)) return HSS_ERR_INVALID_ARG;
  return HSS_OK;
}

extern "C" {

hss_status hss_apply(const hss_matrix* A, int32_t b, const void* X, void* Y, void* ws,
                     size_t ws_bytes, hipStream_t stream) {
  const hss_status st = hss::check_apply_args(A, b, X, Y);
  if (st != HSS_OK) return st;
  const size_t need = hss::apply_ws_bytes(A, b);
  if ((need > 0 && !ws) || ws_bytes < need) return HSS_ERR_WORKSPACE;
  return hss::launch_apply(A, b, X, Y, ws, stream);
}

static hss_status check_group(const hss_matrix* const* A, int32_t G, int32_t b) {
  if (!A || G < 1 || G > HSS_MAX_GROUP) return HSS_ERR_INVALID_ARG;
  for (int g = 0; g < G; ++g) {
    const hss_status st = check_matrix(A[g], b);
    if (st != HSS_OK) return st;
    if (A[g]->n != A[0]->n || A[g]->dtype != A[0]->dtype || A[g]->fmt != A[0]->fmt ||
        A[g]->flags != A[0]->flags)
      return HSS_ERR_INVALID_ARG;
  }
  return HSS_OK;
}

hss_status hss_apply_group_workspace_size(const hss_matrix* const* A, int32_t G, int32_t b, size_t* bytes) {
  if (!bytes) return HSS_ERR_INVALID_ARG;
  const hss_status st = check_group(A, G, b);
  if (st != HSS_OK) return st;
  *bytes = hss::apply_group_ws_bytes(A, G, b);
  return HSS_OK;
}

hss_status hss_apply_group(const hss_matrix* const* A, int32_t G, int32_t b, const void* X, void* const* Y,
                           void* ws, size_t ws_bytes, hipStream_t stream) {
  hss_status st = check_group(A, G, b);
  if (st != HSS_OK) return st;
  if (!X || !Y) return HSS_ERR_INVALID_ARG;
  const size_t es = dsize(A[0]->dtype);
  const size_t xbytes = (size_t)b * A[0]->n * es;
  for (int g = 0; g < G; ++g) {
    if (!Y[g]) return HSS_ERR_INVALID_ARG;
    const size_t yb = (size_t)b * A[g]->m * es;
    if (overlap(X, xbytes, Y[g], yb)) return HSS_ERR_INVALID_ARG;
    for (int h = 0; h < g; ++h)
      if (overlap(Y[h], (size_t)b * A[h]->m * es, Y[g], yb)) return HSS_ERR_INVALID_ARG;
  }
  if (!ws || ws_bytes < hss::apply_group_ws_bytes(A, G, b)) return HSS_ERR_WORKSPACE;
  return hss::launch_apply_group(A, G, b, X, Y, ws, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Hierarchical variant
// ---------------------------------------------------------------------------
hss_status hss_rcm_order(int32_t n, const int32_t* row_ptr, const int32_t* col_idx, int32_t* perm) {
  if (n < 1 || !row_ptr || !perm || row_ptr[0] != 0) return HSS_ERR_INVALID_ARG;
  for (int32_t i = 0; i < n; ++i)
    if (row_ptr[i + 1] < row_ptr[i]) return HSS_ERR_INVALID_ARG;
  const int64_t nnz = row_ptr[n];
  if (nnz > 0 && !col_idx) return HSS_ERR_INVALID_ARG;
  for (int64_t p = 0; p < nnz; ++p)
    if (col_idx[p] < 0 || col_idx[p] >= n) return HSS_ERR_INVALID_ARG;
  return hss::rcm_order_host(n, row_ptr, col_idx, perm);
}

hss_status hss_concentration_workspace_size(int32_t m, int32_t n, size_t* bytes) {
  if (!bytes || m < 1 || n < 1 || (int64_t)m * n >= kLimit) return HSS_ERR_INVALID_ARG;
  *bytes = hss::concentration_ws_bytes(n);
  return HSS_OK;
}

hss_status hss_concentration(int32_t dt, int32_t m, int32_t n, const void* W, const int32_t* perm, double* out,
                             void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!valid_dtype(dt) || m < 1 || n < 1 || (int64_t)m * n >= kLimit || !W || !out) return HSS_ERR_INVALID_ARG;
  if (perm && m != n) return HSS_ERR_INVALID_ARG;
  if (!ws || ws_bytes < hss::concentration_ws_bytes(n)) return HSS_ERR_WORKSPACE;
  return hss::launch_concentration(dt, m, n, W, perm, out, ws, stream);
}

hss_status hss_hier_pack(int32_t dt, int32_t m, int32_t n, const int32_t* r, const void* const* U,
                         const void* const* Vt, const int32_t* perm, void* U_cat, void* Vt_cat, hipStream_t stream) {
  if (!valid_dtype(dt) || m < 2 || n < 2 || !r || !U || !Vt) return HSS_ERR_INVALID_ARG;
  if (perm && m != n) return HSS_ERR_INVALID_ARG;
  const int32_t rows[2] = {m / 2, m - m / 2}, cols[2] = {n / 2, n - n / 2};
  int64_t R = 0;
  for (int b = 0; b < 4; ++b) {
    const int32_t lim = std::min(rows[b >> 1], cols[b & 1]);
    if (r[b] < 0 || r[b] > lim) return HSS_ERR_INVALID_ARG;
    if (r[b] > 0 && (!U[b] || !Vt[b])) return HSS_ERR_INVALID_ARG;
    R += r[b];
  }
  if (R > 0 && (!U_cat || !Vt_cat)) return HSS_ERR_INVALID_ARG;
  if ((int64_t)m * R >= kLimit || R * (int64_t)n >= kLimit) return HSS_ERR_INVALID_ARG;
  return hss::launch_hier_pack(dt, m, n, r, U, Vt, perm, U_cat, Vt_cat, stream);
}

hss_status hss_hier_pack_compact(int32_t dt, int32_t m, int32_t n, const int32_t* r, const void* const* U,
                                 const void* const* Vt, void* U_c, void* Vt_c, hipStream_t stream) {
  if (!valid_dtype(dt) || m < 2 || n < 2 || !r || !U || !Vt) return HSS_ERR_INVALID_ARG;
  const int32_t rows[2] = {m / 2, m - m / 2}, cols[2] = {n / 2, n - n / 2};
  int64_t R = 0;
  for (int b = 0; b < 4; ++b) {
    const int32_t lim = std::min(rows[b >> 1], cols[b & 1]);
    if (r[b] < 0 || r[b] > lim) return HSS_ERR_INVALID_ARG;
    if (r[b] > 0 && (!U[b] || !Vt[b])) return HSS_ERR_INVALID_ARG;
    R += r[b];
  }
  const int64_t ru = (int64_t)r[0] + r[1];
  if (ru != (int64_t)r[2] + r[3]) return HSS_ERR_INVALID_ARG;
  if (R > 0 && (!U_c || !Vt_c)) return HSS_ERR_INVALID_ARG;
  if ((int64_t)m * ru >= kLimit || R * (int64_t)n >= kLimit) return HSS_ERR_INVALID_ARG;
  if (R == 0) return HSS_OK;
  const size_t es = dsize(dt);
  if (overlap(U_c, (size_t)m * ru * es, Vt_c, (size_t)R * cols[1] * es)) return HSS_ERR_INVALID_ARG;
  return hss::launch_hier_pack_compact(dt, m, n, r, U, Vt, U_c, Vt_c, stream);
}

hss_status hss_csr_permute(int32_t n, const int32_t* row_ptr, const int32_t* col_idx, const int32_t* perm,
                           int32_t* row_ptr_p, int32_t* col_idx_p, int32_t* from) {
  if (n < 1 || !row_ptr || !perm || !row_ptr_p || row_ptr[0] != 0) return HSS_ERR_INVALID_ARG;
  for (int32_t i = 0; i < n; ++i)
    if (row_ptr[i + 1] < row_ptr[i]) return HSS_ERR_INVALID_ARG;
  const int64_t nnz = row_ptr[n];
  if (nnz > 0 && (!col_idx || !col_idx_p || !from)) return HSS_ERR_INVALID_ARG;
  std::vector<int32_t> pos(n, -1);  // pos[perm[i]] = i
  for (int32_t i = 0; i < n; ++i) {
    if (perm[i] < 0 || perm[i] >= n || pos[perm[i]] >= 0) return HSS_ERR_INVALID_ARG;
    pos[perm[i]] = i;
  }
  for (int32_t i = 0; i < n; ++i)
    for (int64_t p = row_ptr[i]; p < row_ptr[i + 1]; ++p)
      if (col_idx[p] < 0 || col_idx[p] >= n || (p > row_ptr[i] && col_idx[p] == col_idx[p - 1]))
        return HSS_ERR_INVALID_ARG;
  return hss::csr_permute_host(n, row_ptr, col_idx, perm, pos.data(), row_ptr_p, col_idx_p, from);
}

// ---------------------------------------------------------------------------
// Backward pass
// ---------------------------------------------------------------------------
static hss_status check_grad(const hss_matrix* A, int32_t b) {
  hss_status st = check_matrix(A, b);
  if (st != HSS_OK) return st;
  if (A->dtype != HSS_BF16 || (A->flags & (HSS_DQ4 | HSS_HIER2))) return HSS_ERR_UNSUPPORTED;
  const int64_t ldt = ((int64_t)b + 7) / 8 * 8;
  if ((int64_t)A->n * ldt * 2 >= kLimit || (int64_t)A->m * ldt * 2 >= kLimit) return HSS_ERR_UNSUPPORTED;
  return HSS_OK;
}

hss_status hss_grad_workspace_size(const hss_matrix* A, int32_t b, size_t* bytes) {
  if (!bytes) return HSS_ERR_INVALID_ARG;
  const hss_status st = check_grad(A, b);
  if (st != HSS_OK) return st;
  *bytes = hss::grad_ws_bytes(A, b);
  return HSS_OK;
}

hss_status hss_grad(const hss_matrix* A, int32_t b, const void* X, const void* G, float* dS, float* dU, float* dVt,
                    void* ws, size_t ws_bytes, hipStream_t stream) {
  const hss_status st = check_grad(A, b);
  if (st != HSS_OK) return st;
  if (!X || !G) return HSS_ERR_INVALID_ARG;
  const int64_t m = A->m, n = A->n, r = A->r;
  const size_t xb = (size_t)b * n * 2, gb = (size_t)b * m * 2;
  const int64_t stored = A->fmt == HSS_FMT_2OF4 ? m * (n / 2) : A->nnz;
  const size_t sb = (size_t)stored * 4, ub = (size_t)m * r * 4, vb = (size_t)r * n * 4;
  const void* outs[3] = {dS, dU, dVt};
  const size_t ob[3] = {sb, ub, vb};
  for (int k = 0; k < 3; ++k) {
    if (!outs[k] || ob[k] == 0) continue;
    if (overlap(outs[k], ob[k], X, xb) || overlap(outs[k], ob[k], G, gb)) return HSS_ERR_INVALID_ARG;
    for (int q = k + 1; q < 3; ++q)
      if (outs[q] && ob[q] && overlap(outs[k], ob[k], outs[q], ob[q])) return HSS_ERR_INVALID_ARG;
  }
  const size_t need = hss::grad_ws_bytes(A, b);
  if (!ws || ws_bytes < need) return HSS_ERR_WORKSPACE;
  return hss::launch_grad(A, b, X, G, dS, dU, dVt, ws, stream);
}

hss_status hss_csr_transpose(int32_t m, int32_t n, const int32_t* row_ptr, const int32_t* col_idx, int32_t* row_ptr_t,
                             int32_t* col_idx_t, int32_t* perm) {
  if (m < 1 || n < 1 || !row_ptr || !row_ptr_t || row_ptr[0] != 0) return HSS_ERR_INVALID_ARG;
  for (int32_t i = 0; i < m; ++i)
    if (row_ptr[i + 1] < row_ptr[i]) return HSS_ERR_INVALID_ARG;
  const int64_t nnz = row_ptr[m];
  if (nnz > 0 && (!col_idx || !col_idx_t || !perm)) return HSS_ERR_INVALID_ARG;
  for (int64_t p = 0; p < nnz; ++p)
    if (col_idx[p] < 0 || col_idx[p] >= n) return HSS_ERR_INVALID_ARG;
  return hss::csr_transpose_host(m, n, row_ptr, col_idx, row_ptr_t, col_idx_t, perm);
}

hss_status hss_gather_values(int32_t dt, int64_t nnz, const void* values, const int32_t* perm, void* values_t,
                             hipStream_t stream) {
  if (!valid_dtype(dt) || nnz < 0 || nnz >= kLimit) return HSS_ERR_INVALID_ARG;
  if (nnz == 0) return HSS_OK;
  if (!values || !perm || !values_t) return HSS_ERR_INVALID_ARG;
  const size_t vb = (size_t)nnz * dsize(dt);
  if (overlap(values, vb, values_t, vb)) return HSS_ERR_INVALID_ARG;
  return hss::launch_gather_values(dt, nnz, values, perm, values_t, stream);
}

hss_status hss_transpose(int32_t dt, int32_t rows, int32_t cols, const void* src, void* dst, hipStream_t stream) {
  if (!valid_dtype(dt) || rows < 1 || cols < 1 || (int64_t)rows * cols >= kLimit || !src || !dst)
    return HSS_ERR_INVALID_ARG;
  if ((rows + 31) / 32 > 65535) return HSS_ERR_INVALID_ARG;
  const size_t bytes = (size_t)rows * cols * dsize(dt);
  if (overlap(src, bytes, dst, bytes)) return HSS_ERR_INVALID_ARG;
  return hss::launch_transpose(dt, rows, cols, src, dst, stream);
}

hss_status hss_nm24_to_csr(int32_t m, int32_t n, const uint32_t* nm_meta, int32_t* row_ptr, int32_t* col_idx,
                           hipStream_t stream) {
  if (m < 1 || n < 4 || n % 4 != 0 || (int64_t)m * n >= kLimit || !nm_meta || !row_ptr || !col_idx)
    return HSS_ERR_INVALID_ARG;
  const size_t cb = (size_t)m * (n / 2) * 4, rb = (size_t)(m + 1) * 4;
  if (overlap(row_ptr, rb, col_idx, cb)) return HSS_ERR_INVALID_ARG;
  return hss::launch_nm_to_csr(m, n, nm_meta, row_ptr, col_idx, stream);
}
