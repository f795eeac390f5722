// Backward pass of the HSS layer: gradients of S's stored values, U and V^T
// (bf16 CSR and 2:4 layers, fp32 gradients), and the pieces of the
// transposed layer whose forward apply gives the input gradient.
//
// [HSS] page "LLMの階層的スパース+低ランク圧縮", section "実装と運用パターン"
// (the backward formulas): the gradients of S, U and V are computed
// separately; S's is the upstream gradient times the input, kept on S's
// stored positions; U's and V's go through the other factor.  In this
// library's orientation (Y = X A^T, A = S + U V^T, G = dL/dY, b x m):
//
//   T^T = (X V)^T   r x ldt   launch_tt_gemm (matrix cores, bf16)
//   P^T = (G U)^T   r x ldt   GEMM: A = G (b x m), B = U^T (r x m)
//   dU  = G^T T     m x r     GEMM over the batch: A = T^T, B = G^T (m x ldt)
//   dV^T = P^T X    r x n     GEMM over the batch: A = X^T (n x ldt), B = P^T
//   dS_p = sum_c G[c][i_p] X[c][j_p]                  k_sddmm (vector units), or
//          for large batches dA = G^T X on the matrix cores, then k_ds_gather
//
// The input gradient dX = G A is the forward apply of A^T = S^T + V U^T:
// hss_csr_transpose (S^T's pattern, once per pattern, on the host),
// hss_gather_values (its values, on the device) and hss_transpose (U^T and
// V from the stored factors) build it; hss_apply then runs on it.
#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "hss_internal.h"

namespace hss {

void launch_tt_gemm(const hss_matrix* A, int b, const void* X, uint16_t* Tt, int ldt, float* part, hipStream_t s);
size_t tt_gemm_part_bytes(const hss_matrix* A, int b, int ldt);
void launch_gemm_bf16(int M, int N, int K, const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, void* C,
                      int64_t ldc, bool out_bf16, float* part, hipStream_t s);
size_t gemm_bf16_part_bytes(int M, int N, int K, int64_t ldc);
void launch_xt(const uint16_t* X, int b, int n, int ldt, uint16_t* Xt, hipStream_t s);

static size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }
static int round8(int x) { return (x + 7) & ~7; }

// ---------------------------------------------------------------------------
// dS, sparse form: one wave per row i; each stored entry's dot product over
// the batch is split across LP lanes (16 bytes = 8 batch values of G^T[i]
// and X^T[j] per lane and step), the 64 / LP lane groups taking entries
// p0 + s + SL u (u < 4: four entries in flight, sharing the G^T piece).  The
// LP partial sums meet in an xor butterfly (fixed order).
// ---------------------------------------------------------------------------
static constexpr int kSdUnroll = 4;

// S's stored positions: CSR (int32 or 16-bit columns) or 2:4 (row i holds
// n / 2 entries, entry 2g + s the s-th kept column of group g, from the
// nibble at bits 4 (g % 8) of metadata word g / 8).
enum : int { PAT_CSR32 = 0, PAT_CSR16 = 1, PAT_NM24 = 2 };

struct SPattern {
  const int32_t* row_ptr;  // CSR
  const void* col;         // CSR columns
  const uint32_t* meta;    // 2:4 metadata, m x ceil(n / 32)
  int n;
};

template <int PAT>
__device__ __forceinline__ void pat_row(const SPattern& P, int i, int64_t& rs, int64_t& re) {
  if constexpr (PAT == PAT_NM24) {
    rs = (int64_t)i * (P.n >> 1);
    re = rs + (P.n >> 1);
  } else {
    rs = P.row_ptr[i];
    re = P.row_ptr[i + 1];
  }
}

template <int PAT>
__device__ __forceinline__ int pat_col(const SPattern& P, int i, int64_t rs, int64_t p) {
  if constexpr (PAT == PAT_CSR32) {
    return static_cast<const int32_t*>(P.col)[p];
  } else if constexpr (PAT == PAT_CSR16) {
    return static_cast<const uint16_t*>(P.col)[p];
  } else {
    const int q = (int)(p - rs), g = q >> 1;
    const uint32_t w = P.meta[(int64_t)i * ((P.n + 31) >> 5) + (g >> 3)];
    const uint32_t nib = (w >> (4 * (g & 7))) & 15u;
    return 4 * g + (int)((q & 1) ? (nib >> 2) & 3u : nib & 3u);
  }
}

template <int LP, int PAT>
__global__ __launch_bounds__(256) void k_sddmm(SPattern P, const uint16_t* __restrict__ Gt,
                                               const uint16_t* __restrict__ Xt, int m, int n, int ldt,
                                               float* __restrict__ dS) {
  constexpr int SL = 64 / LP, UE = kSdUnroll;
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (i >= m) return;  // wave-uniform
  const int lane = lane_id(), q0 = lane % LP, s = lane / LP;
  const int pieces = ldt >> 3;
  int64_t rs, re;
  pat_row<PAT>(P, i, rs, re);
  const uint16_t* __restrict__ grow = Gt + (int64_t)i * ldt;
  // X^T through a bounded buffer resource: a column index outside [0, n)
  // reads zeros instead of memory past X^T
  const __amdgpu_buffer_rsrc_t rx =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(Xt), 0, (int)((int64_t)n * ldt * 2), 0x00020000);
  for (int64_t p0 = rs + s; p0 < re; p0 += SL * UE) {
    int j[UE];
    float acc[UE];
    // unconditional loads (past the row: its last entry again, dropped at the
    // store), so the four are in flight together
#pragma unroll
    for (int u = 0; u < UE; ++u) {
      const int64_t p = p0 + u * SL;
      j[u] = pat_col<PAT>(P, i, rs, p < re ? p : re - 1);
      acc[u] = 0.f;
    }
    for (int q = q0; q < pieces; q += LP) {
      const u32x4 gv = *reinterpret_cast<const u32x4*>(grow + 8 * q);
      u32x4 xv[UE];
#pragma unroll
      for (int u = 0; u < UE; ++u)
        xv[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, (j[u] * ldt + 8 * q) * 2, 0, 0));
      const float g[8] = {bf16lo(gv.x), bf16hi(gv.x), bf16lo(gv.y), bf16hi(gv.y),
                          bf16lo(gv.z), bf16hi(gv.z), bf16lo(gv.w), bf16hi(gv.w)};
#pragma unroll
      for (int u = 0; u < UE; ++u) {
        float t = acc[u];
        t = fmaf(g[0], bf16lo(xv[u].x), t); t = fmaf(g[1], bf16hi(xv[u].x), t);
        t = fmaf(g[2], bf16lo(xv[u].y), t); t = fmaf(g[3], bf16hi(xv[u].y), t);
        t = fmaf(g[4], bf16lo(xv[u].z), t); t = fmaf(g[5], bf16hi(xv[u].z), t);
        t = fmaf(g[6], bf16lo(xv[u].w), t); t = fmaf(g[7], bf16hi(xv[u].w), t);
        acc[u] = t;
      }
    }
#pragma unroll
    for (int u = 0; u < UE; ++u) {
#pragma unroll
      for (int off = 1; off < LP; off <<= 1) acc[u] += __shfl_xor(acc[u], off, 64);
      const int64_t p = p0 + u * SL;
      if (p < re && q0 == 0) dS[p] = acc[u];
    }
  }
}

// dS, dense form: dS[p] = dA[i][column of p] from dA = G^T X (m x n fp32,
// computed on the matrix cores); one wave per row, coalesced along the row.
template <int PAT>
__global__ __launch_bounds__(256) void k_ds_gather(SPattern P, const float* __restrict__ dA, int m, int n,
                                                   float* __restrict__ dS) {
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (i >= m) return;
  const float* __restrict__ row = dA + (int64_t)i * n;
  int64_t rs, re;
  pat_row<PAT>(P, i, rs, re);
  for (int64_t p = rs + lane_id(); p < re; p += 64) {
    const int j = pat_col<PAT>(P, i, rs, p);
    dS[p] = (j >= 0 && j < n) ? row[j] : 0.f;
  }
}

// The CSR form of a 2:4 pattern (row_ptr[i] = i n / 2; columns from the
// metadata), for building the transposed layer.
__global__ __launch_bounds__(256) void k_nm_to_csr(const uint32_t* __restrict__ meta, int m, int n,
                                                   int32_t* __restrict__ row_ptr, int32_t* __restrict__ col) {
  SPattern P = {};
  P.meta = meta;
  P.n = n;
  const int64_t total = (int64_t)m * (n >> 1);
  for (int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x; p < total; p += (int64_t)gridDim.x * 256) {
    const int i = (int)(p / (n >> 1));
    col[p] = pat_col<PAT_NM24>(P, i, (int64_t)i * (n >> 1), p);
  }
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i <= m; i += (int64_t)gridDim.x * 256)
    row_ptr[i] = (int32_t)(i * (n >> 1));
}

hss_status launch_nm_to_csr(int m, int n, const uint32_t* meta, int32_t* row_ptr, int32_t* col, hipStream_t s) {
  const int64_t total = (int64_t)m * (n >> 1);
  const unsigned grid = (unsigned)std::min<int64_t>((total + 255) / 256, 8192);
  hipLaunchKernelGGL(k_nm_to_csr, dim3(grid), dim3(256), 0, s, meta, m, n, row_ptr, col);
  return hipGetLastError() == hipSuccess ? HSS_OK : HSS_ERR_HIP;
}

template <int PAT>
static void launch_sddmm_pat(int lp, const SPattern& P, const uint16_t* Gt, const uint16_t* Xt, int m, int n, int ldt,
                             float* dS, hipStream_t s) {
  const dim3 grid((unsigned)((m + 3) / 4)), block(256);
  switch (lp) {
    case 1: hipLaunchKernelGGL((k_sddmm<1, PAT>), grid, block, 0, s, P, Gt, Xt, m, n, ldt, dS); break;
    case 2: hipLaunchKernelGGL((k_sddmm<2, PAT>), grid, block, 0, s, P, Gt, Xt, m, n, ldt, dS); break;
    case 4: hipLaunchKernelGGL((k_sddmm<4, PAT>), grid, block, 0, s, P, Gt, Xt, m, n, ldt, dS); break;
    case 8: hipLaunchKernelGGL((k_sddmm<8, PAT>), grid, block, 0, s, P, Gt, Xt, m, n, ldt, dS); break;
    case 16: hipLaunchKernelGGL((k_sddmm<16, PAT>), grid, block, 0, s, P, Gt, Xt, m, n, ldt, dS); break;
    case 32: hipLaunchKernelGGL((k_sddmm<32, PAT>), grid, block, 0, s, P, Gt, Xt, m, n, ldt, dS); break;
    default: hipLaunchKernelGGL((k_sddmm<64, PAT>), grid, block, 0, s, P, Gt, Xt, m, n, ldt, dS); break;
  }
}

// ---------------------------------------------------------------------------
// Workspace: X^T, G^T, U^T, T^T, P^T and the GEMMs' split-K partials.
// ---------------------------------------------------------------------------
// dS route: the dense form from this batch on (or HSS_OPT_GRAD_DS_ROUTE:
// 1 sampled, 2 dense).  Measured on the 8192 x 8192 3 % layer (sampled vs
// dense, ms): b = 256 0.101 vs 0.127, b = 512 0.203 vs 0.170, b = 2048 1.15
// vs 0.41.
static constexpr int kDenseDsMinB = 512;

static bool ds_dense(int b) {
  const int forced = option(HSS_OPT_GRAD_DS_ROUTE);
  if (forced == 1) return false;
  if (forced == 2) return true;
  return b >= kDenseDsMinB;
}

struct GradPlan {
  int ldt, ldu;
  size_t xt, gt, ut, tt, pt, da, part, total;
};

static GradPlan plan_grad(const hss_matrix* A, int b) {
  GradPlan p;
  const int m = A->m, n = A->n, r = A->r;
  p.ldt = round8(b);
  p.ldu = round8(m);
  size_t off = 0;
  p.xt = off; off += al256((size_t)n * p.ldt * 2);
  p.gt = off; off += al256((size_t)m * p.ldt * 2);
  p.ut = off; off += al256((size_t)(r > 0 ? r : 1) * p.ldu * 2);
  p.tt = off; off += al256((size_t)(r > 0 ? r : 1) * p.ldt * 2);
  p.pt = off; off += al256((size_t)(r > 0 ? r : 1) * p.ldt * 2);
  p.da = off; off += ds_dense(b) ? al256((size_t)m * n * 4) : 0;
  size_t part = 0;
  if (r > 0) {
    part = std::max(part, tt_gemm_part_bytes(A, b, p.ldt));
    part = std::max(part, gemm_bf16_part_bytes(b, r, m, p.ldt));  // P^T
    part = std::max(part, gemm_bf16_part_bytes(r, m, b, r));      // dU
    part = std::max(part, gemm_bf16_part_bytes(n, r, b, n));      // dV^T
  }
  if (ds_dense(b)) part = std::max(part, gemm_bf16_part_bytes(n, m, b, n));  // dA
  p.part = off; off += al256(part);
  p.total = off;
  return p;
}

size_t grad_ws_bytes(const hss_matrix* A, int b) { return plan_grad(A, b).total; }

hss_status launch_grad(const hss_matrix* A, int b, const void* X, const void* G, float* dS, float* dU, float* dVt,
                       void* ws, hipStream_t s) {
  const GradPlan p = plan_grad(A, b);
  char* base = static_cast<char*>(ws);
  uint16_t* Xt = reinterpret_cast<uint16_t*>(base + p.xt);
  uint16_t* Gt = reinterpret_cast<uint16_t*>(base + p.gt);
  uint16_t* Ut = reinterpret_cast<uint16_t*>(base + p.ut);
  uint16_t* Tt = reinterpret_cast<uint16_t*>(base + p.tt);
  uint16_t* Pt = reinterpret_cast<uint16_t*>(base + p.pt);
  float* part = reinterpret_cast<float*>(base + p.part);
  const int m = A->m, n = A->n, r = A->r;
  const uint16_t* Xb = static_cast<const uint16_t*>(X);
  const uint16_t* Gb = static_cast<const uint16_t*>(G);
  const int64_t stored = A->fmt == HSS_FMT_2OF4 ? (int64_t)m * (n / 2) : A->nnz;
  const bool want_s = dS && stored > 0, want_u = dU && r > 0, want_v = dVt && r > 0;
  if (want_v || want_s) launch_xt(Xb, b, n, p.ldt, Xt, s);
  if (want_u || want_s) launch_xt(Gb, b, m, p.ldt, Gt, s);
  if (want_u) {
    launch_tt_gemm(A, b, X, Tt, p.ldt, part, s);
    launch_gemm_bf16(r, m, b, Tt, p.ldt, Gt, p.ldt, dU, r, false, part, s);
  }
  if (want_v) {
    launch_xt(static_cast<const uint16_t*>(A->U), m, r, p.ldu, Ut, s);
    launch_gemm_bf16(b, r, m, Gb, m, Ut, p.ldu, Pt, p.ldt, true, part, s);
    launch_gemm_bf16(n, r, b, Xt, p.ldt, Pt, p.ldt, dVt, n, false, part, s);
  }
  if (want_s) {
    SPattern P = {};
    P.row_ptr = A->row_ptr;
    P.col = A->col_idx;
    P.meta = A->nm_meta;
    P.n = n;
    const int pat = A->fmt == HSS_FMT_2OF4 ? PAT_NM24 : ((A->flags & HSS_COL16) ? PAT_CSR16 : PAT_CSR32);
    if (ds_dense(b)) {
      float* dA = reinterpret_cast<float*>(base + p.da);
      launch_gemm_bf16(n, m, b, Xt, p.ldt, Gt, p.ldt, dA, n, false, part, s);
      const dim3 grid((unsigned)((m + 3) / 4));
      if (pat == PAT_NM24)
        hipLaunchKernelGGL(k_ds_gather<PAT_NM24>, grid, dim3(256), 0, s, P, dA, m, n, dS);
      else if (pat == PAT_CSR16)
        hipLaunchKernelGGL(k_ds_gather<PAT_CSR16>, grid, dim3(256), 0, s, P, dA, m, n, dS);
      else
        hipLaunchKernelGGL(k_ds_gather<PAT_CSR32>, grid, dim3(256), 0, s, P, dA, m, n, dS);
    } else {
      int lp = 1;
      while (lp < 64 && lp * 2 <= (p.ldt >> 3)) lp *= 2;
      if (pat == PAT_NM24)
        launch_sddmm_pat<PAT_NM24>(lp, P, Gt, Xt, m, n, p.ldt, dS, s);
      else if (pat == PAT_CSR16)
        launch_sddmm_pat<PAT_CSR16>(lp, P, Gt, Xt, m, n, p.ldt, dS, s);
      else
        launch_sddmm_pat<PAT_CSR32>(lp, P, Gt, Xt, m, n, p.ldt, dS, s);
    }
  }
  return hipGetLastError() == hipSuccess ? HSS_OK : HSS_ERR_HIP;
}

// ---------------------------------------------------------------------------
// The transposed layer.
// ---------------------------------------------------------------------------

// S^T's CSR pattern on the host: a counting sort by column, rows visited in
// ascending order, so each row of S^T lists its entries by original row;
// perm[q] = the storage index in S of S^T's q-th entry.
hss_status csr_transpose_host(int m, int n, const int32_t* row_ptr, const int32_t* col_idx, int32_t* row_ptr_t,
                              int32_t* col_idx_t, int32_t* perm) {
  const int64_t nnz = row_ptr[m];
  std::vector<int64_t> next(n + 1, 0);
  for (int64_t p = 0; p < nnz; ++p) ++next[col_idx[p] + 1];
  for (int j = 0; j < n; ++j) next[j + 1] += next[j];
  for (int j = 0; j <= n; ++j) row_ptr_t[j] = (int32_t)next[j];
  for (int i = 0; i < m; ++i)
    for (int64_t p = row_ptr[i]; p < row_ptr[i + 1]; ++p) {
      const int64_t q = next[col_idx[p]]++;
      col_idx_t[q] = i;
      perm[q] = (int32_t)p;
    }
  return HSS_OK;
}

template <typename T>
__global__ __launch_bounds__(256) void k_gather(const T* __restrict__ src, const int32_t* __restrict__ perm,
                                                int64_t count, T* __restrict__ dst) {
  for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < count; q += (int64_t)gridDim.x * 256)
    dst[q] = src[perm[q]];
}

hss_status launch_gather_values(int dt, int64_t nnz, const void* values, const int32_t* perm, void* values_t,
                                hipStream_t s) {
  if (nnz == 0) return HSS_OK;
  const unsigned grid = (unsigned)std::min<int64_t>((nnz + 255) / 256, 8192);
  if (dt == HSS_F32)
    hipLaunchKernelGGL(k_gather<uint32_t>, dim3(grid), dim3(256), 0, s, static_cast<const uint32_t*>(values), perm,
                       nnz, static_cast<uint32_t*>(values_t));
  else
    hipLaunchKernelGGL(k_gather<uint16_t>, dim3(grid), dim3(256), 0, s, static_cast<const uint16_t*>(values), perm,
                       nnz, static_cast<uint16_t*>(values_t));
  return hipGetLastError() == hipSuccess ? HSS_OK : HSS_ERR_HIP;
}

// dst (cols x rows) = src (rows x cols)^T, bits copied.  32 x 32 tiles
// through LDS so that both the reads and the writes run along rows.
template <typename T>
__global__ __launch_bounds__(256) void k_transpose(const T* __restrict__ src, int rows, int cols, T* __restrict__ dst) {
  __shared__ T tile[32][33];
  const int tr = blockIdx.y * 32, tc = blockIdx.x * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
#pragma unroll
  for (int k = 0; k < 32; k += 8) {
    const int r = tr + ty + k, c = tc + tx;
    if (r < rows && c < cols) tile[ty + k][tx] = src[(int64_t)r * cols + c];
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 32; k += 8) {
    const int c = tc + ty + k, r = tr + tx;
    if (r < rows && c < cols) dst[(int64_t)c * rows + r] = tile[tx][ty + k];
  }
}

hss_status launch_transpose(int dt, int rows, int cols, const void* src, void* dst, hipStream_t s) {
  const dim3 grid((unsigned)((cols + 31) / 32), (unsigned)((rows + 31) / 32));
  if (dt == HSS_F32)
    hipLaunchKernelGGL(k_transpose<uint32_t>, grid, dim3(256), 0, s, static_cast<const uint32_t*>(src), rows, cols,
                       static_cast<uint32_t*>(dst));
  else
    hipLaunchKernelGGL(k_transpose<uint16_t>, grid, dim3(256), 0, s, static_cast<const uint16_t*>(src), rows, cols,
                       static_cast<uint16_t*>(dst));
  return hipGetLastError() == hipSuccess ? HSS_OK : HSS_ERR_HIP;
}

}  // namespace hss
