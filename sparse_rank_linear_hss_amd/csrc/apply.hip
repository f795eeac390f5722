// hss_apply dispatch: Y = X S^T + (X V) U^T.
//
// [HSS] page "LLMの階層的スパース+低ランク圧縮", section "実装と運用パターン": the
// forward pass of the compressed layer is the sparse product plus two small
// dense products through the factors.
//
// Paths:
//   decode (decode.hip)  up to 8 columns per launch: one fused kernel that
//                        streams S, U and V^T once (HBM-bound regime); fp32
//                        and narrow batches.
//   mfma (mfma.hip)      bf16 2:4 beyond 64 columns, CSR beyond 128: the
//                        low-rank products are dense contractions and run on
//                        the matrix cores, S expanded into the same GEMM.
//   dense-and-sparse     HSS_DQ4 matrices (decode.hip, k_decode_dq): the
//                        quantised dense part and the CSR outliers, up to 8
//                        columns per pass, no workspace.
//   gather SpMM          bf16 CSR from 3 to 128 columns (and beyond where S
//   (spmm.hip)           cannot be densified): S read once, X^T rows
//                        gathered per entry, T from a small prologue.
//   sparse matrix cores  bf16 2:4 from 2 to 64 columns (n % 128 == 0): S's
//   (nm_mma.hip)         values and metadata fed to v_smfmac as stored, T
//                        from a small prologue.
//
// HSS_OPT_BATCH_ROUTE (hss_set_option; first value from the environment
// variable HSS_CSR_BATCH_ROUTE) forces the route of a bf16 batch (where that
// route supports it), for measuring one against another.
#include "hss_internal.h"

namespace hss {

void launch_decode(const hss_matrix* A, int bc, const void* X, void* Y, void* ws, hipStream_t s);
void launch_decode_group(const hss_matrix* const* A, int G, int bc, const void* X, void* const* Y, void* ws,
                         hipStream_t s);
size_t decode_ctl_bytes();
size_t decode_t_bytes(const hss_matrix* A);
int decode_max_cols(const hss_matrix* A);
int decode_dq_max_cols(const hss_matrix* A);
void launch_decode_dq(const hss_matrix* A, int bc, const void* X, void* Y, hipStream_t s);
static bool is_dq(const hss_matrix* A) { return (A->flags & HSS_DQ4) != 0; }
static bool is_hier(const hss_matrix* A) { return (A->flags & HSS_HIER2) != 0; }
static size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }

// A block-structured (HSS_HIER2) matrix takes the fused decode kernel with
// its compact factors; the batched routes read flat factors, expanded per
// call into the workspace (m x r and r x n, zeros outside the blocks).
static size_t hier_flat_bytes(const hss_matrix* A) {
  const size_t es = A->dtype == HSS_F32 ? 4 : 2;
  return a256((size_t)A->m * A->r * es) + a256((size_t)A->r * A->n * es);
}
static hss_matrix flat_view(const hss_matrix* A, void* Uf, void* Vtf) {
  hss_matrix F = *A;
  F.flags &= ~HSS_HIER2;
  F.U = Uf;
  F.Vt = Vtf;
  return F;
}

static constexpr int kDecodeCols = 8;

bool mfma_supported(const hss_matrix* A, int b);
size_t mfma_ws_bytes(const hss_matrix* A, int b);
hss_status launch_mfma(const hss_matrix* A, int b, const void* X, void* Y, void* ws, hipStream_t s);

bool spmm_supported(const hss_matrix* A, int b);
size_t spmm_ws_bytes(const hss_matrix* A, int b);
hss_status launch_spmm(const hss_matrix* A, int b, const void* X, void* Y, void* ws, hipStream_t s);

bool nm_mma_supported(const hss_matrix* A, int b);
size_t nm_mma_ws_bytes(const hss_matrix* A, int b);
hss_status launch_nm_mma(const hss_matrix* A, int b, const void* X, void* Y, void* ws, hipStream_t s);

enum Route { R_DECODE = 0, R_SPMM = 1, R_MFMA = 2, R_NM = 3 };

// Default batch range of the 2:4 route on the sparse matrix cores.
// Measured on the 11008 x 4096 rank-64 layer (decode / densify vs sparse
// matrix cores, us, 16-call graphs): b = 2 decode 20.0 vs 21.6 (three runs:
// the decode passes won by 1.5-2.0); b = 3 decode 25.3 vs 18.5; b = 8 decode
// 49.5 vs 22.5; b = 16 densify 47.2 vs 23.9; b = 32 densify 48.5 vs 25.8;
// b = 64 densify 61.4 vs 44.5.
static constexpr int kNmMinColsDefault = 3;

// Default batch range of the gather SpMM for bf16 CSR: below it the fused
// decode passes, above it S densified for the matrix cores.  Measured on the
// 4096 x 4096 5 % rank-256 layer (decode / densify vs gather): b = 2 decode
// 10.3 vs 11.1 us; b = 3 decode 12.2 vs 11.2 us; b = 4 decode 12.7 vs 11.3
// us; b = 8 decode 20.1 vs 11.7 us; b = 16 39.8 vs 14.3 us; b = 32 densify
// 52.8 vs 20.7 us; b = 64 169 / 58.4 vs 30.0 us; b = 128 densify 64.8 vs
// 41.0 us; b = 256 densify 77.3 vs 61.5 us.  The 8192 x 8192 3 % rank-512
// layer: b = 64 densify 137 vs 68 us, b = 128 151 vs 102 us, b = 256 164 vs
// 178 us (its U part, m r b on the vector units, is 4 times the 4096^2
// layer's), so the gather stops at 128.
static constexpr int kSpmmMinCols = 3, kSpmmMaxCols = 128;

// X: the call's input (the sparse matrix cores need it 16-byte aligned), or
// null when sizing a workspace.
static Route batch_route(const hss_matrix* A0, int b, const void* X) {
  if (b < 2) return R_DECODE;  // one column: always the fused decode kernel
  const hss_matrix F = is_hier(A0) ? flat_view(A0, nullptr, nullptr) : *A0;  // routes decide on shapes only
  const hss_matrix* A = &F;
  const bool sp = spmm_supported(A, b), mf = mfma_supported(A, b);
  const bool nm = nm_mma_supported(A, b) && (uintptr_t)X % 16 == 0;
  switch (option(HSS_OPT_BATCH_ROUTE)) {
    case 1: return R_DECODE;
    case 2: if (sp) return R_SPMM; break;
    case 3: if (mf) return R_MFMA; break;
    case 4: if (nm) return R_NM; break;
    default: break;
  }
  if (nm && b >= kNmMinColsDefault) return R_NM;
  if (sp && b >= kSpmmMinCols && (b <= kSpmmMaxCols || !mf)) return R_SPMM;
  if (mf) return R_MFMA;
  return R_DECODE;
}

// Layout: [decode control region | decode T words or MFMA buffers].  The
// control region persists between calls; everything after it is per-call
// scratch, so both paths can share one workspace.
size_t apply_ws_bytes(const hss_matrix* A0, int b) {
  if (is_dq(A0)) return 0;
  // every route the call may take (the route can be forced at call time)
  const size_t dec = decode_t_bytes(A0);
  const hss_matrix F = is_hier(A0) ? flat_view(A0, nullptr, nullptr) : *A0;
  const hss_matrix* A = &F;
  const size_t mf = mfma_supported(A, b) ? mfma_ws_bytes(A, b) : 0;
  const size_t sp = spmm_supported(A, b) ? spmm_ws_bytes(A, b) : 0;
  const size_t nm = nm_mma_supported(A, b) ? nm_mma_ws_bytes(A, b) : 0;
  size_t mx = mf > sp ? mf : sp;
  mx = mx > nm ? mx : nm;
  if (is_hier(A0) && b >= 2) mx += hier_flat_bytes(A0);
  return decode_ctl_bytes() + (dec > mx ? dec : mx);
}

// Workspace bytes of the route this call takes (hss_apply_workspace_size
// covers every route a call could be forced onto).
size_t apply_route_ws_bytes(const hss_matrix* A0, int b, const void* X) {
  if (is_dq(A0)) return 0;
  const hss_matrix F = is_hier(A0) ? flat_view(A0, nullptr, nullptr) : *A0;
  const hss_matrix* A = &F;
  const size_t flat = is_hier(A0) ? hier_flat_bytes(A0) : 0;
  switch (batch_route(A0, b, X)) {
    case R_NM: return decode_ctl_bytes() + flat + nm_mma_ws_bytes(A, b);
    case R_MFMA: return decode_ctl_bytes() + flat + mfma_ws_bytes(A, b);
    case R_SPMM: return decode_ctl_bytes() + flat + spmm_ws_bytes(A, b);
    default: return decode_ctl_bytes() + decode_t_bytes(A0);
  }
}

hss_status launch_apply(const hss_matrix* A, int b, const void* X, void* Y, void* ws,
                        hipStream_t stream) {
  if (is_dq(A)) {
    const size_t es = A->dtype == HSS_F32 ? 4 : 2;
    const int cols = decode_dq_max_cols(A);
    if (cols == 0) return HSS_ERR_UNSUPPORTED;
    for (int c0 = 0; c0 < b; c0 += cols) {
      const int bc = b - c0 < cols ? b - c0 : cols;
      launch_decode_dq(A, bc, static_cast<const char*>(X) + (size_t)c0 * A->n * es,
                       static_cast<char*>(Y) + (size_t)c0 * A->m * es, stream);
    }
    return hipGetLastError() == hipSuccess ? HSS_OK : HSS_ERR_HIP;
  }
  const Route route = batch_route(A, b, X);
  char* scratch = static_cast<char*>(ws) + decode_ctl_bytes();
  hss_matrix F;
  if (route != R_DECODE && is_hier(A)) {
    const size_t es = A->dtype == HSS_F32 ? 4 : 2;
    void* Uf = A->r > 0 ? scratch : nullptr;
    void* Vtf = A->r > 0 ? scratch + a256((size_t)A->m * A->r * es) : nullptr;
    const hss_status st = launch_hier_expand(A, Uf, Vtf, stream);
    if (st != HSS_OK) return st;
    scratch += hier_flat_bytes(A);
    F = flat_view(A, Uf, Vtf);
    A = &F;
  }
  if (route == R_NM) return launch_nm_mma(A, b, X, Y, scratch, stream);
  if (route == R_MFMA) return launch_mfma(A, b, X, Y, scratch, stream);
  if (route == R_SPMM) return launch_spmm(A, b, X, Y, scratch, stream);
  const size_t es = A->dtype == HSS_F32 ? 4 : 2;
  const int cols = decode_max_cols(A);
  if (cols == 0) return HSS_ERR_UNSUPPORTED;
  for (int c0 = 0; c0 < b; c0 += cols) {
    const int bc = b - c0 < cols ? b - c0 : cols;
    launch_decode(A, bc, static_cast<const char*>(X) + (size_t)c0 * A->n * es,
                  static_cast<char*>(Y) + (size_t)c0 * A->m * es, ws, stream);
  }
  return hipGetLastError() == hipSuccess ? HSS_OK : HSS_ERR_HIP;
}

// Every byte of p[0 .. bytes) set to zero by plain vector stores (a kernel,
// not a memset, so it may be captured into a graph): the aligned middle as
// 16-byte stores, the unaligned head and tail bytewise.
__global__ __launch_bounds__(256) void k_zero_fill(unsigned char* p, size_t bytes) {
  const size_t head = min(bytes, (size_t)((16u - ((uintptr_t)p & 15u)) & 15u));
  const size_t nvec = (bytes - head) / 16, tail0 = head + nvec * 16;
  const size_t tid = (size_t)blockIdx.x * blockDim.x + threadIdx.x, nth = (size_t)gridDim.x * blockDim.x;
  u32x4* v = reinterpret_cast<u32x4*>(p + head);
  for (size_t i = tid; i < nvec; i += nth) v[i] = u32x4{0u, 0u, 0u, 0u};
  if (tid < head) p[tid] = 0;
  if (tid < bytes - tail0) p[tail0 + tid] = 0;
}

hss_status launch_zero_fill(void* p, size_t bytes, hipStream_t s) {
  const size_t vec = bytes / 16 + 1;
  const unsigned blocks = (unsigned)(vec / 256 + 1 < 2048 ? vec / 256 + 1 : 2048);
  hipLaunchKernelGGL(k_zero_fill, dim3(blocks), dim3(256), 0, s, static_cast<unsigned char*>(p), bytes);
  return hipGetLastError() == hipSuccess ? HSS_OK : HSS_ERR_HIP;
}

// Grouped apply of G matrices sharing X.  Decode batches: one fused launch
// per pass over all G matrices (their T words side by side after the control
// region).  Matrix-core batches: one apply per matrix, in order.
size_t apply_group_ws_bytes(const hss_matrix* const* A, int G, int b) {
  size_t dec = 0, one = 0;
  for (int g = 0; g < G; ++g) {
    if (is_dq(A[g])) continue;  // the dense-and-sparse kernel uses no workspace
    dec += decode_t_bytes(A[g]);
    const size_t a = apply_ws_bytes(A[g], b) - decode_ctl_bytes();
    one = one > a ? one : a;
  }
  return decode_ctl_bytes() + (dec > one ? dec : one);
}

hss_status launch_apply_group(const hss_matrix* const* A, int G, int b, const void* X, void* const* Y, void* ws,
                              hipStream_t stream) {
  bool any_mfma = false;  // (or dense-and-sparse: those run one by one too)
  for (int g = 0; g < G; ++g) any_mfma = any_mfma || batch_route(A[g], b, X) != R_DECODE || is_dq(A[g]);
  if (any_mfma) {
    for (int g = 0; g < G; ++g) {
      const hss_status st = launch_apply(A[g], b, X, Y[g], ws, stream);
      if (st != HSS_OK) return st;
    }
    return HSS_OK;
  }
  const size_t es = A[0]->dtype == HSS_F32 ? 4 : 2;
  int cols = kDecodeCols;
  for (int g = 0; g < G; ++g) {
    const int c = decode_max_cols(A[g]);
    cols = cols < c ? cols : c;
  }
  if (cols == 0) return HSS_ERR_UNSUPPORTED;
  for (int c0 = 0; c0 < b; c0 += cols) {
    const int bc = b - c0 < cols ? b - c0 : cols;
    void* Yc[8];
    for (int g = 0; g < G; ++g) Yc[g] = static_cast<char*>(Y[g]) + (size_t)c0 * A[g]->m * es;
    launch_decode_group(A, G, bc, static_cast<const char*>(X) + (size_t)c0 * A[0]->n * es, Yc, ws, stream);
  }
  return hipGetLastError() == hipSuccess ? HSS_OK : HSS_ERR_HIP;
}

}  // namespace hss
