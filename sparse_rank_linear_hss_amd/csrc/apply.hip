// Apply: Y = X S^T + (X V) U^T.
//
// [HSS] page "LLMの階層的スパース+低ランク圧縮", section "実装と運用パターン": the
// forward pass of the compressed layer is the sparse product plus two small
// dense products through the factors.  Decode (few columns) streams the
// compressed weights once and is bound by HBM bandwidth (the SqueezeLLM
// explainer page aibr.jp/archives/208940, section "1.概要と位置づけ", makes the
// same point: single-batch inference is limited by memory bandwidth).
//
// Small-batch path (bc <= 16 columns of X per pass):
//   k_lr_t      T[c][l] = sum_j Vt[l][j] X[c][j]: one block per factor row l,
//               contiguous 16-byte reads of Vt and X, fp32 accumulation.
//   k_rows_*    one wave per output row i: the row's sparse entries (CSR or
//               2:4 with the 4-bit metadata decoded in registers) against X,
//               plus U[i][:] . T[:][c], one wave reduction, one store per column.
#include "hss_internal.h"

namespace hss {

template <int DT> struct Out;
template <> struct Out<HSS_F32> {
  __device__ __forceinline__ static uint32_t pack(float f) { return __float_as_uint(f); }
};
template <> struct Out<HSS_BF16> {
  __device__ __forceinline__ static uint16_t pack(float f) { return f32_to_bf16(f); }
};

template <int DT>
__device__ __forceinline__ float ld(const typename Elem<DT>::bits_t* p) {
  return Elem<DT>::to_f(*p);
}

// Unpack a 16-byte vector into fp32 values (4 for fp32, 8 for bf16).
template <int DT> struct V16;
template <> struct V16<HSS_F32> {
  static constexpr int N = 4;
  __device__ __forceinline__ static void get(const u32x4& v, float (&o)[4]) {
    o[0] = __uint_as_float(v.x); o[1] = __uint_as_float(v.y);
    o[2] = __uint_as_float(v.z); o[3] = __uint_as_float(v.w);
  }
};
template <> struct V16<HSS_BF16> {
  static constexpr int N = 8;
  __device__ __forceinline__ static void get(const u32x4& v, float (&o)[8]) {
    o[0] = bf16lo(v.x); o[1] = bf16hi(v.x); o[2] = bf16lo(v.y); o[3] = bf16hi(v.y);
    o[4] = bf16lo(v.z); o[5] = bf16hi(v.z); o[6] = bf16lo(v.w); o[7] = bf16hi(v.w);
  }
};

// T[c][l] for one l per block; bc <= BC columns.
template <int DT, int BC, bool VEC>
__global__ __launch_bounds__(256) void k_lr_t(const typename Elem<DT>::bits_t* __restrict__ Vt,
                                              const typename Elem<DT>::bits_t* __restrict__ X,
                                              int n, int r, int bc, float* __restrict__ T) {
  using bits_t = typename Elem<DT>::bits_t;
  __shared__ float red[4][BC];
  const int l = blockIdx.x;
  const int t = threadIdx.x;
  const bits_t* v = Vt + (int64_t)l * n;
  float acc[BC];
#pragma unroll
  for (int c = 0; c < BC; ++c) acc[c] = 0.f;
  int jt = 0;  // first column of the scalar tail
  if constexpr (VEC) {
    constexpr int NV = V16<DT>::N;
    const int nvec = n / NV;
    for (int q = t; q < nvec; q += 256) {
      float vv[NV];
      V16<DT>::get(__builtin_nontemporal_load(reinterpret_cast<const u32x4*>(v) + q), vv);
#pragma unroll
      for (int c = 0; c < BC; ++c) {
        if (c < bc) {
          float xv[NV];
          V16<DT>::get(*(reinterpret_cast<const u32x4*>(X + (int64_t)c * n) + q), xv);
#pragma unroll
          for (int e = 0; e < NV; ++e) acc[c] = fmaf(vv[e], xv[e], acc[c]);
        }
      }
    }
    jt = nvec * NV;
  }
  for (int j = jt + t; j < n; j += 256) {
    const float vj = ld<DT>(v + j);
#pragma unroll
    for (int c = 0; c < BC; ++c)
      if (c < bc) acc[c] = fmaf(vj, ld<DT>(X + (int64_t)c * n + j), acc[c]);
  }
  const int w = t >> 6;
#pragma unroll
  for (int c = 0; c < BC; ++c) {
    const float s = wave_sum(acc[c]);
    if (lane_id() == 0) red[w][c] = s;
  }
  __syncthreads();
  if (t < bc) T[(int64_t)t * r + l] = (red[0][t] + red[1][t]) + (red[2][t] + red[3][t]);
}

// Low-rank epilogue of one row: acc[c] += sum_l U[i][l] T[c][l] (lane-strided l).
template <int DT, int BC>
__device__ __forceinline__ void lowrank_row(const typename Elem<DT>::bits_t* __restrict__ Ur, int r,
                                            int bc, const float* __restrict__ T, float (&acc)[BC]) {
  for (int l = lane_id(); l < r; l += HSS_WAVE) {
    const float u = ld<DT>(Ur + l);
#pragma unroll
    for (int c = 0; c < BC; ++c)
      if (c < bc) acc[c] = fmaf(u, T[(int64_t)c * r + l], acc[c]);
  }
}

template <int DT, int BC>
__device__ __forceinline__ void finish_row(float (&acc)[BC], int bc, int m, int row,
                                           typename Elem<DT>::bits_t* __restrict__ Y) {
  const int lane = lane_id();
#pragma unroll
  for (int c = 0; c < BC; ++c) {
    const float s = wave_sum(acc[c]);
    if (c < bc && lane == c) Y[(int64_t)c * m + row] = Out<DT>::pack(s);
  }
}

// CSR rows, one wave per row.
template <int DT, int BC>
__global__ __launch_bounds__(256) void k_rows_csr(int m, int n, int r, int bc,
                                                  const int32_t* __restrict__ row_ptr,
                                                  const int32_t* __restrict__ col_idx,
                                                  const typename Elem<DT>::bits_t* __restrict__ vals,
                                                  const typename Elem<DT>::bits_t* __restrict__ U,
                                                  const float* __restrict__ T,
                                                  const typename Elem<DT>::bits_t* __restrict__ X,
                                                  typename Elem<DT>::bits_t* __restrict__ Y) {
  const int row = uniform(blockIdx.x * 4 + (int)(threadIdx.x >> 6));
  if (row >= m) return;
  const int start = uniform(row_ptr[row]);
  const int end = uniform(row_ptr[row + 1]);
  float acc[BC];
#pragma unroll
  for (int c = 0; c < BC; ++c) acc[c] = 0.f;
  for (int p = start + lane_id(); p < end; p += HSS_WAVE) {
    const int col = __builtin_nontemporal_load(col_idx + p);
    const float v = Elem<DT>::to_f(__builtin_nontemporal_load(vals + p));
#pragma unroll
    for (int c = 0; c < BC; ++c)
      if (c < bc) acc[c] = fmaf(v, ld<DT>(X + (int64_t)c * n + col), acc[c]);
  }
  if (r > 0) lowrank_row<DT, BC>(U + (int64_t)row * r, r, bc, T, acc);
  finish_row<DT, BC>(acc, bc, m, row, Y);
}

// 2:4 rows, one wave per row; lane handles whole metadata words (32 columns).
template <int DT, int BC>
__global__ __launch_bounds__(256) void k_rows_24(int m, int n, int r, int bc,
                                                 const typename Elem<DT>::bits_t* __restrict__ nmv,
                                                 const uint32_t* __restrict__ meta,
                                                 const typename Elem<DT>::bits_t* __restrict__ U,
                                                 const float* __restrict__ T,
                                                 const typename Elem<DT>::bits_t* __restrict__ X,
                                                 typename Elem<DT>::bits_t* __restrict__ Y) {
  using bits_t = typename Elem<DT>::bits_t;
  const int row = uniform(blockIdx.x * 4 + (int)(threadIdx.x >> 6));
  if (row >= m) return;
  const int words = (n + 31) >> 5;
  const uint32_t* Mr = meta + (int64_t)row * words;
  const bits_t* Vr = nmv + (int64_t)row * (n >> 1);
  float acc[BC];
#pragma unroll
  for (int c = 0; c < BC; ++c) acc[c] = 0.f;
  for (int w = lane_id(); w < words; w += HSS_WAVE) {
    const uint32_t mw = __builtin_nontemporal_load(Mr + w);
    const int c0 = w * 32;
    const int ng = min(8, (n - c0) >> 2);
    for (int g = 0; g < ng; ++g) {
      const uint32_t nib = (mw >> (4 * g)) & 15u;
      const int j0 = c0 + 4 * g + (int)(nib & 3u);
      const int j1 = c0 + 4 * g + (int)(nib >> 2);
      const float v0 = Elem<DT>::to_f(__builtin_nontemporal_load(Vr + (c0 >> 1) + 2 * g));
      const float v1 = Elem<DT>::to_f(__builtin_nontemporal_load(Vr + (c0 >> 1) + 2 * g + 1));
#pragma unroll
      for (int c = 0; c < BC; ++c) {
        if (c < bc) {
          const bits_t* Xc = X + (int64_t)c * n;
          acc[c] = fmaf(v0, ld<DT>(Xc + j0), acc[c]);
          acc[c] = fmaf(v1, ld<DT>(Xc + j1), acc[c]);
        }
      }
    }
  }
  if (r > 0) lowrank_row<DT, BC>(U + (int64_t)row * r, r, bc, T, acc);
  finish_row<DT, BC>(acc, bc, m, row, Y);
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
static constexpr int kMaxCols = 16;  // columns per small-batch pass

size_t apply_ws_bytes(const hss_matrix* A, int /*b*/) {
  const size_t t_bytes = sizeof(float) * (size_t)kMaxCols * (size_t)(A->r > 0 ? A->r : 1);
  return 256 + ((t_bytes + 255) / 256) * 256;
}

template <int DT, int BC>
static void launch_pass(const hss_matrix* A, int bc, const typename Elem<DT>::bits_t* X,
                        typename Elem<DT>::bits_t* Y, float* T, hipStream_t s) {
  using bits_t = typename Elem<DT>::bits_t;
  const int m = A->m, n = A->n, r = A->r;
  const bits_t* U = static_cast<const bits_t*>(A->U);
  const bits_t* Vt = static_cast<const bits_t*>(A->Vt);
  if (r > 0) {
    const bool vec = ((uintptr_t)Vt % 16) == 0 && ((uintptr_t)X % 16) == 0 &&
                     ((size_t)n * sizeof(bits_t)) % 16 == 0;
    if (vec)
      hipLaunchKernelGGL((k_lr_t<DT, BC, true>), dim3(r), dim3(256), 0, s, Vt, X, n, r, bc, T);
    else
      hipLaunchKernelGGL((k_lr_t<DT, BC, false>), dim3(r), dim3(256), 0, s, Vt, X, n, r, bc, T);
  }
  const unsigned grid = (unsigned)((m + 3) / 4);
  if (A->fmt == HSS_FMT_CSR)
    hipLaunchKernelGGL((k_rows_csr<DT, BC>), dim3(grid), dim3(256), 0, s, m, n, r, bc, A->row_ptr,
                       A->col_idx, static_cast<const bits_t*>(A->values), U, T, X, Y);
  else
    hipLaunchKernelGGL((k_rows_24<DT, BC>), dim3(grid), dim3(256), 0, s, m, n, r, bc,
                       static_cast<const bits_t*>(A->nm_values), A->nm_meta, U, T, X, Y);
}

template <int DT>
static hss_status apply_t(const hss_matrix* A, int b, const void* Xv, void* Yv, void* ws,
                          hipStream_t s) {
  using bits_t = typename Elem<DT>::bits_t;
  const bits_t* X = static_cast<const bits_t*>(Xv);
  bits_t* Y = static_cast<bits_t*>(Yv);
  float* T = reinterpret_cast<float*>(static_cast<char*>(ws) + 256);
  for (int c0 = 0; c0 < b; c0 += kMaxCols) {
    const int bc = b - c0 < kMaxCols ? b - c0 : kMaxCols;
    const bits_t* Xc = X + (int64_t)c0 * A->n;
    bits_t* Yc = Y + (int64_t)c0 * A->m;
    if (bc == 1) launch_pass<DT, 1>(A, bc, Xc, Yc, T, s);
    else if (bc == 2) launch_pass<DT, 2>(A, bc, Xc, Yc, T, s);
    else if (bc <= 4) launch_pass<DT, 4>(A, bc, Xc, Yc, T, s);
    else if (bc <= 8) launch_pass<DT, 8>(A, bc, Xc, Yc, T, s);
    else launch_pass<DT, 16>(A, bc, Xc, Yc, T, s);
  }
  return hipGetLastError() == hipSuccess ? HSS_OK : HSS_ERR_HIP;
}

hss_status launch_apply(const hss_matrix* A, int b, const void* X, void* Y, void* ws,
                        hipStream_t stream) {
  if (A->dtype == HSS_F32) return apply_t<HSS_F32>(A, b, X, Y, ws, stream);
  return apply_t<HSS_BF16>(A, b, X, Y, ws, stream);
}

}  // namespace hss
