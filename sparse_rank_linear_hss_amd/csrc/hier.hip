// Hierarchical variant: Reverse Cuthill-McKee order (host), concentration
// ratio (device) and the packing of 2 x 2 block low-rank factors into flat
// factors that the apply kernels read (device).
//
// [HSS] page "LLMの階層的スパース+低ランク圧縮", section "順列と階層的整列"
// (vision rewrite "置換と階層的整列"): rho = sum of |W| over the diagonal blocks
// over the sum of |W|; a Reverse Cuthill-McKee order of rows and columns
// pulls the large entries to the diagonal; the 2 x 2 block factorisation
// then keeps a higher rank on the diagonal blocks than off them.
//
// One level of 2 x 2 blocks (rows split at m / 2, columns at n / 2) with
// block (bi, bj) = U_b Vt_b of the permuted residual is, in the original
// order, U_cat Vt_cat with R = r00 + r01 + r10 + r11 columns:
//   U_cat[perm[i]][o_b + l] = U_b[i - row0(bi)][l]  for the two blocks of i's row half,
//   Vt_cat[o_b + l][perm[j]] = Vt_b[l][j - col0(bj)] for the columns of block b's column half,
// zero elsewhere (o_b: the column offset of block b in the order 00, 01, 10,
// 11).  The apply kernels then run unchanged (a rank-R layer); the zeros cost
// twice the factor bytes of the blocks themselves.
#include <algorithm>
#include <vector>

#include "hss_internal.h"

namespace hss {

// ---------------------------------------------------------------------------
// RCM (host): breadth-first from the lowest-degree (then lowest-index)
// unvisited node of each component, unvisited neighbours queued by (degree,
// index) ascending, the visit order reversed; graph = the symmetric pattern
// without self-loops.
// ---------------------------------------------------------------------------
hss_status rcm_order_host(int n, const int32_t* row_ptr, const int32_t* col_idx, int32_t* perm) {
  std::vector<std::vector<int32_t>> nbr(n);
  for (int i = 0; i < n; ++i) {
    for (int64_t p = row_ptr[i]; p < row_ptr[i + 1]; ++p) {
      const int32_t j = col_idx[p];
      if (j == i) continue;
      nbr[i].push_back(j);
      nbr[j].push_back(i);
    }
  }
  std::vector<int32_t> deg(n);
  for (int i = 0; i < n; ++i) {
    auto& v = nbr[i];
    std::sort(v.begin(), v.end());
    v.erase(std::unique(v.begin(), v.end()), v.end());
    deg[i] = (int32_t)v.size();
  }
  auto less = [&](int32_t a, int32_t b) { return deg[a] != deg[b] ? deg[a] < deg[b] : a < b; };
  std::vector<int32_t> by_deg(n);
  for (int i = 0; i < n; ++i) by_deg[i] = i;
  std::sort(by_deg.begin(), by_deg.end(), less);
  std::vector<char> seen(n, 0);
  std::vector<int32_t> order;
  order.reserve(n);
  std::vector<int32_t> cand;
  size_t next = 0;
  while ((int)order.size() < n) {
    while (seen[by_deg[next]]) ++next;
    const int32_t start = by_deg[next];
    seen[start] = 1;
    size_t head = order.size();
    order.push_back(start);
    while (head < order.size()) {
      const int32_t u = order[head++];
      cand.clear();
      for (int32_t v : nbr[u])
        if (!seen[v]) cand.push_back(v);
      std::sort(cand.begin(), cand.end(), less);
      for (int32_t v : cand) {
        seen[v] = 1;
        order.push_back(v);
      }
    }
  }
  for (int i = 0; i < n; ++i) perm[i] = order[n - 1 - i];
  return HSS_OK;
}

// ---------------------------------------------------------------------------
// Concentration ratio (device).  Fixed grid and fixed-order reductions in
// fp64, so the result does not depend on scheduling.
// ---------------------------------------------------------------------------
static constexpr int kRhoBlocks = 1024;

__global__ __launch_bounds__(256) void k_inverse_perm(const int32_t* __restrict__ perm, int n, int32_t* inv) {
  for (int a = blockIdx.x * 256 + threadIdx.x; a < n; a += gridDim.x * 256) {
    const int32_t p = perm[a];
    if (p >= 0 && p < n) inv[p] = a;
  }
}

template <int DT>
__global__ __launch_bounds__(256) void k_rho_partial(const typename Elem<DT>::bits_t* __restrict__ W, int m, int n,
                                                     const int32_t* __restrict__ inv, double* part) {
  __shared__ double sd[256], st[256];
  const int m1 = m / 2, n1 = n / 2;
  const int64_t total = (int64_t)m * n;
  double d = 0.0, a = 0.0;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
    const int i = (int)(e / n), j = (int)(e - (int64_t)i * n);
    const int pi = inv ? inv[i] : i, pj = inv ? inv[j] : j;
    const double v = fabs((double)Elem<DT>::to_f(W[e]));
    a += v;
    if ((pi < m1) == (pj < n1)) d += v;
  }
  sd[threadIdx.x] = d;
  st[threadIdx.x] = a;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) {
      sd[threadIdx.x] += sd[threadIdx.x + s];
      st[threadIdx.x] += st[threadIdx.x + s];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    part[2 * blockIdx.x] = sd[0];
    part[2 * blockIdx.x + 1] = st[0];
  }
}

// 64 threads: thread t adds partials t, t + 64, ... in order, then a fixed
// pairwise tree through LDS; the same bits on every call.
__global__ __launch_bounds__(64) void k_rho_final(const double* __restrict__ part, int blocks, double* out) {
  __shared__ double sd[64], st[64];
  const int t = threadIdx.x;
  double d = 0.0, a = 0.0;
  for (int b = t; b < blocks; b += 64) {
    d += part[2 * b];
    a += part[2 * b + 1];
  }
  sd[t] = d;
  st[t] = a;
  __syncthreads();
  for (int s = 32; s > 0; s >>= 1) {
    if (t < s) {
      sd[t] += sd[t + s];
      st[t] += st[t + s];
    }
    __syncthreads();
  }
  if (t == 0) {
    out[0] = st[0] > 0.0 ? sd[0] / st[0] : 0.0;
    out[1] = sd[0];
    out[2] = st[0];
  }
}

size_t concentration_ws_bytes(int n) { return sizeof(double) * 2 * kRhoBlocks + sizeof(int32_t) * (size_t)n; }

hss_status launch_concentration(int dt, int m, int n, const void* W, const int32_t* perm, double* out, void* ws,
                                hipStream_t s) {
  double* part = static_cast<double*>(ws);
  int32_t* inv = nullptr;
  if (perm) {
    inv = reinterpret_cast<int32_t*>(part + 2 * kRhoBlocks);
    hipLaunchKernelGGL(k_inverse_perm, dim3((unsigned)std::min(4096, (n + 255) / 256)), dim3(256), 0, s, perm, n,
                       inv);
  }
  if (dt == HSS_F32)
    hipLaunchKernelGGL(k_rho_partial<HSS_F32>, dim3(kRhoBlocks), dim3(256), 0, s,
                       static_cast<const uint32_t*>(W), m, n, inv, part);
  else
    hipLaunchKernelGGL(k_rho_partial<HSS_BF16>, dim3(kRhoBlocks), dim3(256), 0, s,
                       static_cast<const uint16_t*>(W), m, n, inv, part);
  hipLaunchKernelGGL(k_rho_final, dim3(1), dim3(64), 0, s, part, kRhoBlocks, out);
  return hipGetLastError() == hipSuccess ? HSS_OK : HSS_ERR_HIP;
}

// ---------------------------------------------------------------------------
// Packing of the 2 x 2 block factors (device): pure data movement.  A
// permutation entry out of [0, n) is skipped (its output row / column keeps
// whatever it held): the caller passes a permutation.
// ---------------------------------------------------------------------------
struct HierBlocks {
  const void* U[4];
  const void* Vt[4];
  int r[4];
  int off[5];  // column offsets of the blocks in U_cat (off[4] = R)
};

template <typename T>
__global__ __launch_bounds__(256) void k_pack_u(HierBlocks hb, int m, const int32_t* __restrict__ perm, T* Ucat) {
  const int R = hb.off[4], m1 = m / 2;
  const int64_t total = (int64_t)m * R;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
    const int i = (int)(e / R), c = (int)(e - (int64_t)i * R);
    int b = 0;
    while (c >= hb.off[b + 1]) ++b;
    const int bi = b >> 1;  // row half of block b (order 00, 01, 10, 11)
    const int half = i < m1 ? 0 : 1;
    T v = 0;
    if (bi == half) {
      const int ii = i - (half ? m1 : 0);
      v = static_cast<const T*>(hb.U[b])[(int64_t)ii * hb.r[b] + (c - hb.off[b])];
    }
    const int row = perm ? perm[i] : i;
    if (row >= 0 && row < m) Ucat[(int64_t)row * R + c] = v;
  }
}

template <typename T>
__global__ __launch_bounds__(256) void k_pack_vt(HierBlocks hb, int n, const int32_t* __restrict__ perm, T* Vtcat) {
  const int R = hb.off[4], n1 = n / 2;
  const int64_t total = (int64_t)R * n;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
    const int c = (int)(e / n), j = (int)(e - (int64_t)c * n);
    int b = 0;
    while (c >= hb.off[b + 1]) ++b;
    const int bj = b & 1;  // column half of block b
    const int half = j < n1 ? 0 : 1;
    T v = 0;
    if (bj == half) {
      const int jj = j - (half ? n1 : 0), w = half ? n - n1 : n1;
      v = static_cast<const T*>(hb.Vt[b])[(int64_t)(c - hb.off[b]) * w + jj];
    }
    const int col = perm ? perm[j] : j;
    if (col >= 0 && col < n) Vtcat[(int64_t)c * n + col] = v;
  }
}

hss_status launch_hier_pack(int dt, int m, int n, const int32_t* r, const void* const* U, const void* const* Vt,
                            const int32_t* perm, void* Ucat, void* Vtcat, hipStream_t s) {
  HierBlocks hb = {};
  hb.off[0] = 0;
  for (int b = 0; b < 4; ++b) {
    hb.U[b] = U[b];
    hb.Vt[b] = Vt[b];
    hb.r[b] = r[b];
    hb.off[b + 1] = hb.off[b] + r[b];
  }
  const int R = hb.off[4];
  if (R == 0) return HSS_OK;
  const unsigned gu = (unsigned)std::min<int64_t>(((int64_t)m * R + 255) / 256, 8192);
  const unsigned gv = (unsigned)std::min<int64_t>(((int64_t)R * n + 255) / 256, 8192);
  if (dt == HSS_F32) {
    hipLaunchKernelGGL(k_pack_u<uint32_t>, dim3(gu), dim3(256), 0, s, hb, m, perm, static_cast<uint32_t*>(Ucat));
    hipLaunchKernelGGL(k_pack_vt<uint32_t>, dim3(gv), dim3(256), 0, s, hb, n, perm, static_cast<uint32_t*>(Vtcat));
  } else {
    hipLaunchKernelGGL(k_pack_u<uint16_t>, dim3(gu), dim3(256), 0, s, hb, m, perm, static_cast<uint16_t*>(Ucat));
    hipLaunchKernelGGL(k_pack_vt<uint16_t>, dim3(gv), dim3(256), 0, s, hb, n, perm, static_cast<uint16_t*>(Vtcat));
  }
  return hipGetLastError() == hipSuccess ? HSS_OK : HSS_ERR_HIP;
}

// ---------------------------------------------------------------------------
// Compact form of the block term (HSS_HIER2), in the blocks' own order: U_c
// row i holds the factors of the two blocks of i's row half side by side
// (ru = r00 + r01 = r10 + r11 values), V^T_c row o_b + l holds row l of
// block b's V^T over its column half only, rows n - n/2 long.  Nothing is
// zero but the unread last value of a first-half row when n is odd.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void k_pack_compact_u(HierBlocks hb, int m, T* Uc) {
  const int ru = hb.r[0] + hb.r[1], m1 = m / 2;
  const int64_t total = (int64_t)m * ru;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
    const int i = (int)(e / ru), k = (int)(e - (int64_t)i * ru);
    const int half = i < m1 ? 0 : 1, ii = i - (half ? m1 : 0);
    const int b0 = 2 * half, b = k < hb.r[b0] ? b0 : b0 + 1, kk = b == b0 ? k : k - hb.r[b0];
    Uc[e] = static_cast<const T*>(hb.U[b])[(int64_t)ii * hb.r[b] + kk];
  }
}

template <typename T>
__global__ __launch_bounds__(256) void k_pack_compact_vt(HierBlocks hb, int n, T* Vtc) {
  const int R = hb.off[4], n1 = n / 2, ld = hier_vt_ld(n);
  const int64_t total = (int64_t)R * ld;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
    const int c = (int)(e / ld), j = (int)(e - (int64_t)c * ld);
    int b = 0;
    while (c >= hb.off[b + 1]) ++b;
    const int w = (b & 1) ? n - n1 : n1;  // columns of block b's half
    Vtc[e] = j < w ? static_cast<const T*>(hb.Vt[b])[(int64_t)(c - hb.off[b]) * w + j] : T(0);
  }
}

hss_status launch_hier_pack_compact(int dt, int m, int n, const int32_t* r, const void* const* U,
                                    const void* const* Vt, void* Uc, void* Vtc, hipStream_t s) {
  HierBlocks hb = {};
  hb.off[0] = 0;
  for (int b = 0; b < 4; ++b) {
    hb.U[b] = U[b];
    hb.Vt[b] = Vt[b];
    hb.r[b] = r[b];
    hb.off[b + 1] = hb.off[b] + r[b];
  }
  const int R = hb.off[4], ru = r[0] + r[1];
  if (R == 0) return HSS_OK;
  const unsigned gu = (unsigned)std::min<int64_t>(((int64_t)m * ru + 255) / 256, 8192);
  const unsigned gv = (unsigned)std::min<int64_t>(((int64_t)R * hier_vt_ld(n) + 255) / 256, 8192);
  if (dt == HSS_F32) {
    if (ru > 0) hipLaunchKernelGGL(k_pack_compact_u<uint32_t>, dim3(gu), dim3(256), 0, s, hb, m, static_cast<uint32_t*>(Uc));
    hipLaunchKernelGGL(k_pack_compact_vt<uint32_t>, dim3(gv), dim3(256), 0, s, hb, n, static_cast<uint32_t*>(Vtc));
  } else {
    if (ru > 0) hipLaunchKernelGGL(k_pack_compact_u<uint16_t>, dim3(gu), dim3(256), 0, s, hb, m, static_cast<uint16_t*>(Uc));
    hipLaunchKernelGGL(k_pack_compact_vt<uint16_t>, dim3(gv), dim3(256), 0, s, hb, n, static_cast<uint16_t*>(Vtc));
  }
  return hipGetLastError() == hipSuccess ? HSS_OK : HSS_ERR_HIP;
}

// The compact factors of an HSS_HIER2 matrix expanded into flat factors of
// the same basis (U_f m x R, V^T_f R x n, zeros outside each block), for the
// batched routes: U_f[i][c] = U_c[i][c - h ru] when column c belongs to the
// blocks of i's row half h (c in [h ru, (h + 1) ru)), V^T_f[l][j] =
// V^T_c[l][j - bj n/2] when column j lies in the column half bj of row l's
// block.
template <typename T>
__global__ __launch_bounds__(256) void k_expand_u(const T* __restrict__ Uc, int m, int ru, T* Uf) {
  const int R = 2 * ru, m1 = m / 2;
  const int64_t total = (int64_t)m * R;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
    const int i = (int)(e / R), c = (int)(e - (int64_t)i * R);
    const int h = i < m1 ? 0 : 1;
    Uf[e] = (c >= h * ru && c < (h + 1) * ru) ? Uc[(int64_t)i * ru + (c - h * ru)] : T(0);
  }
}

template <typename T>
__global__ __launch_bounds__(256) void k_expand_vt(const T* __restrict__ Vtc, int n, int R, int l1, int l2, int l3,
                                                   T* Vtf) {
  const int n1 = n / 2, ld = hier_vt_ld(n);
  const int64_t total = (int64_t)R * n;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
    const int l = (int)(e / n), j = (int)(e - (int64_t)l * n);
    const int bj = ((l >= l1 && l < l2) || l >= l3) ? 1 : 0;  // column half of row l's block
    const int jj = j - (bj ? n1 : 0);
    Vtf[e] = ((j >= n1) == (bj == 1)) ? Vtc[(int64_t)l * ld + jj] : T(0);
  }
}

hss_status launch_hier_expand(const hss_matrix* A, void* Uf, void* Vtf, hipStream_t s) {
  const int m = A->m, n = A->n, R = A->r, ru = A->hier_r[0] + A->hier_r[1];
  if (R == 0) return HSS_OK;
  const int l1 = A->hier_r[0], l2 = l1 + A->hier_r[1], l3 = l2 + A->hier_r[2];
  const unsigned gu = (unsigned)std::min<int64_t>(((int64_t)m * R + 255) / 256, 8192);
  const unsigned gv = (unsigned)std::min<int64_t>(((int64_t)R * n + 255) / 256, 8192);
  if (A->dtype == HSS_F32) {
    hipLaunchKernelGGL(k_expand_u<uint32_t>, dim3(gu), dim3(256), 0, s, static_cast<const uint32_t*>(A->U), m, ru,
                       static_cast<uint32_t*>(Uf));
    hipLaunchKernelGGL(k_expand_vt<uint32_t>, dim3(gv), dim3(256), 0, s, static_cast<const uint32_t*>(A->Vt), n, R,
                       l1, l2, l3, static_cast<uint32_t*>(Vtf));
  } else {
    hipLaunchKernelGGL(k_expand_u<uint16_t>, dim3(gu), dim3(256), 0, s, static_cast<const uint16_t*>(A->U), m, ru,
                       static_cast<uint16_t*>(Uf));
    hipLaunchKernelGGL(k_expand_vt<uint16_t>, dim3(gv), dim3(256), 0, s, static_cast<const uint16_t*>(A->Vt), n, R,
                       l1, l2, l3, static_cast<uint16_t*>(Vtf));
  }
  return hipGetLastError() == hipSuccess ? HSS_OK : HSS_ERR_HIP;
}

// S' = P S P^T on the host: row i of S' is row perm[i] of S with every
// column j renamed pos[j] (pos = perm's inverse) and the row sorted by the
// new columns; from[q] = S's storage index of S''s entry q.
hss_status csr_permute_host(int n, const int32_t* row_ptr, const int32_t* col_idx, const int32_t* perm,
                            const int32_t* pos, int32_t* row_ptr_p, int32_t* col_idx_p, int32_t* from) {
  std::vector<std::pair<int32_t, int32_t>> row;
  int64_t q = 0;
  row_ptr_p[0] = 0;
  for (int i = 0; i < n; ++i) {
    const int src = perm[i];
    row.clear();
    for (int64_t p = row_ptr[src]; p < row_ptr[src + 1]; ++p) row.emplace_back(pos[col_idx[p]], (int32_t)p);
    std::sort(row.begin(), row.end());
    for (const auto& e : row) {
      col_idx_p[q] = e.first;
      from[q] = e.second;
      ++q;
    }
    row_ptr_p[i + 1] = (int32_t)q;
  }
  return HSS_OK;
}

}  // namespace hss
