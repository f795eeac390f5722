// Batched apply (b >= 16 columns, bf16) on the matrix cores.
//
// [HSS] page "LLMの階層的スパース+低ランク圧縮", section "実装と運用パターン": the
// forward pass is the sparse product plus two small dense products; the same
// section notes that on compute-bound hardware (large batches) the sparse
// product's low arithmetic intensity limits the gain.  With b >= 16 columns
// both low-rank products are dense contractions, so they run on MFMA:
//
//   T^T (b x r)  = X (b x n) . Vt^T              one GEMM, A = Vt, B = X
//   Y   (b x m)  = [X | T^T] . [S | U]^T          one GEMM over K = n + r:
//                  segment 1: A = S densified into LDS chunk by chunk
//                  (2:4: metadata expanded in registers; CSR: entries of
//                  each row scattered from per-chunk row pointers),
//                  segment 2: A = U, B = T^T.
//
// One kernel, k_gemm: C = A . B^T with A (M x K) and B (N x K) both
// K-contiguous, fp32 accumulation in v_mfma_f32_32x32x16_bf16, output stored
// N-major (C[n * ldc + m]) so that Y (b x m) and T^T (b x r) come out in the
// layout their consumers read.  Tile 128 x 128 (4 waves of 64 x 64), K in
// chunks of 128 staged through LDS.  When there are too few tiles to fill the
// chip the K chunks are split across blocks; fp32 partials are then summed in
// a fixed order by k_reduce (deterministic, no float atomics).
#include <algorithm>

#include "hss_internal.h"

namespace hss {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

enum : int { A_DENSE = 0, A_NM24 = 1, A_CSR = 2 };
enum : int { OUT_BF16 = 0, OUT_F32 = 1, OUT_PARTIAL = 2 };

static constexpr int kBM = 128, kBN = 128, kKC = 128;
static constexpr int kLdsStride = kKC + 8;  // bf16 elements per LDS row (16-byte pad)

struct GemmArgs {
  int M, N;
  int K1, K2;            // K segments: [0, K1) then [K1, K1 + K2)
  int nch1, nch;         // chunks in segment 1, total chunks
  int chunks_per_split;  // gridDim.z splits of the chunk range
  int a1_mode;
  const uint16_t* A1;  int64_t lda1;   // dense A, segment 1 (M x K1)
  const uint16_t* nmv; const uint32_t* meta;            // 2:4 S (K1 % 32 == 0)
  const int32_t* col_idx; const uint16_t* vals; const int32_t* cptr; int ncp;  // CSR S
  const uint16_t* B1;  int64_t ldb1;   // N x K1
  const uint16_t* A2;  int64_t lda2;   // M x K2
  const uint16_t* B2;  int64_t ldb2;   // N x K2
  void* C; int64_t ldc; int out_mode;  // C[n * ldc + m]; partials: + z * N * ldc
  int vec_a1, vec_b1, vec_a2, vec_b2;  // 16-byte loads allowed (K % 8 == 0, aligned rows)
};

// Stage a 128 x 128 chunk of a dense K-contiguous operand (rows r0.., cols k0..)
// into LDS; rows >= R or cols >= K are zero.
__device__ __forceinline__ void stage_dense(uint16_t* __restrict__ lds, const uint16_t* __restrict__ src,
                                            int64_t ld, int r0, int R, int k0, int K, int vec) {
  const int t = threadIdx.x;
  if (vec) {
    u32x4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {  // issue all 8 loads first (clamped, always valid)
      const int q = t + 256 * i;
      const int row = q >> 4, kq = (q & 15) * 8;
      const int rr = min(r0 + row, R - 1), kk = min(k0 + kq, K - 8);
      v[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + rr * ld + kk));
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int q = t + 256 * i;
      const int row = q >> 4, kq = (q & 15) * 8;
      const bool ok = r0 + row < R && k0 + kq < K;
      const u32x4 z = {0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(lds + row * kLdsStride + kq) = ok ? v[i] : z;
    }
  } else {
    for (int q = t; q < kBM * kKC; q += 256) {
      const int row = q / kKC, kq = q % kKC;
      const bool ok = r0 + row < R && k0 + kq < K;
      lds[row * kLdsStride + kq] = ok ? src[(int64_t)(r0 + row) * ld + k0 + kq] : (uint16_t)0;
    }
  }
}

// Stage a 2:4 chunk: rows r0.., columns k0..k0+127 (4 metadata words per row).
__device__ __forceinline__ void stage_nm24(uint16_t* __restrict__ lds, const uint16_t* __restrict__ nmv,
                                           const uint32_t* __restrict__ meta, int r0, int R, int k0, int K) {
  const int t = threadIdx.x;
  const int words = K >> 5;
  uint32_t mw[2];
  u32x4 v[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = t + 256 * i;  // (row, word) item
    const int row = q >> 2, wd = (k0 >> 5) + (q & 3);
    const int rr = min(r0 + row, R - 1), wc = min(wd, words - 1);
    mw[i] = __builtin_nontemporal_load(meta + (int64_t)rr * words + wc);
    const u32x4* vp = reinterpret_cast<const u32x4*>(nmv + (int64_t)rr * (K >> 1) + wc * 16);
    v[i][0] = __builtin_nontemporal_load(vp);
    v[i][1] = __builtin_nontemporal_load(vp + 1);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = t + 256 * i;
    const int row = q >> 2, wd = (k0 >> 5) + (q & 3);
    const bool ok = r0 + row < R && wd < words;
    const uint32_t vw[8] = {v[i][0].x, v[i][0].y, v[i][0].z, v[i][0].w,
                            v[i][1].x, v[i][1].y, v[i][1].z, v[i][1].w};
    uint32_t out[16];  // 32 bf16 of the dense row segment
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      const uint32_t nib = ok ? (mw[i] >> (4 * g)) & 15u : 0u;
      const uint32_t i0 = nib & 3u, i1 = nib >> 2;
      const uint32_t v0 = ok ? (vw[g] & 0xffffu) : 0u, v1 = ok ? (vw[g] >> 16) : 0u;
      uint32_t e[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) e[p] = (p == (int)i0) ? v0 : ((p == (int)i1) ? v1 : 0u);
      out[2 * g] = e[0] | (e[1] << 16);
      out[2 * g + 1] = e[2] | (e[3] << 16);
    }
    u32x4* dst = reinterpret_cast<u32x4*>(lds + row * kLdsStride + (q & 3) * 32);
#pragma unroll
    for (int h = 0; h < 4; ++h) dst[h] = u32x4{out[4 * h], out[4 * h + 1], out[4 * h + 2], out[4 * h + 3]};
  }
}

// Stage a CSR chunk: zero the tile, then each of the 128 rows scatters its
// entries with columns in [k0, k0 + 128), found through cptr (row pointers per
// chunk).  Two threads per row, four entries each per pass.
__device__ __forceinline__ void stage_csr(uint16_t* __restrict__ lds, const GemmArgs& g, int r0, int chunk) {
  const int t = threadIdx.x;
  u32x4* l4 = reinterpret_cast<u32x4*>(lds);
  for (int q = t; q < kBM * kLdsStride / 8; q += 256) l4[q] = u32x4{0u, 0u, 0u, 0u};
  __syncthreads();
  const int row = t & 127, h = t >> 7;
  if (r0 + row < g.M) {
    const int* cp = g.cptr + (int64_t)(r0 + row) * g.ncp + chunk;
    const int p0 = cp[0], p1 = cp[1];
    const int k0 = chunk * kKC;
    for (int e = p0 + h; e < p1; e += 8) {
      int col[4];
      uint16_t val[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int ej = min(e + 2 * j, p1 - 1);
        col[j] = g.col_idx[ej];
        val[j] = g.vals[ej];
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int kc = col[j] - k0;  // in [0, 128) for ascending columns; guarded anyway
        if (e + 2 * j < p1 && kc >= 0 && kc < kKC) lds[row * kLdsStride + kc] = val[j];
      }
    }
  }
}

__global__ __launch_bounds__(256) void k_gemm(GemmArgs g) {
  __shared__ __align__(16) uint16_t As[kBM * kLdsStride];
  __shared__ __align__(16) uint16_t Bs[kBN * kLdsStride];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int m0 = blockIdx.x * kBM, n0 = blockIdx.y * kBN;
  const int c_begin = blockIdx.z * g.chunks_per_split;
  const int c_end = min(c_begin + g.chunks_per_split, g.nch);

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  for (int c = c_begin; c < c_end; ++c) {
    __syncthreads();  // previous chunk's MFMA reads are done
    if (c < g.nch1) {
      const int k0 = c * kKC;
      if (g.a1_mode == A_DENSE)
        stage_dense(As, g.A1, g.lda1, m0, g.M, k0, g.K1, g.vec_a1);
      else if (g.a1_mode == A_NM24)
        stage_nm24(As, g.nmv, g.meta, m0, g.M, k0, g.K1);
      else
        stage_csr(As, g, m0, c);
      stage_dense(Bs, g.B1, g.ldb1, n0, g.N, k0, g.K1, g.vec_b1);
    } else {
      const int k0 = (c - g.nch1) * kKC;
      stage_dense(As, g.A2, g.lda2, m0, g.M, k0, g.K2, g.vec_a2);
      stage_dense(Bs, g.B2, g.ldb2, n0, g.N, k0, g.K2, g.vec_b2);
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < kKC / 16; ++s) {
      const int kk = s * 16 + 8 * (lane >> 5);
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        af[i] = *reinterpret_cast<const bf16x8*>(As + (wm * 64 + i * 32 + (lane & 31)) * kLdsStride + kk);
        bfr[i] = *reinterpret_cast<const bf16x8*>(Bs + (wn * 64 + i * 32 + (lane & 31)) * kLdsStride + kk);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  }

  // Epilogue: lane holds D[8*(v/4) + 4*(lane/32) + v%4][lane%32] of each 32x32 block.
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + wn * 64 + j * 32 + (lane & 31);
      if (n >= g.N) continue;
#pragma unroll
      for (int vg = 0; vg < 4; ++vg) {
        const int m = m0 + wm * 64 + i * 32 + 8 * vg + 4 * (lane >> 5);
        float a4[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) a4[p] = acc[i][j][4 * vg + p];
        if (g.out_mode == OUT_BF16) {
          uint16_t* C = static_cast<uint16_t*>(g.C) + (int64_t)n * g.ldc;
#pragma unroll
          for (int p = 0; p < 4; ++p)
            if (m + p < g.M) C[m + p] = f32_to_bf16(a4[p]);
        } else {
          float* C = static_cast<float*>(g.C) + (int64_t)blockIdx.z * g.N * g.ldc + (int64_t)n * g.ldc;
#pragma unroll
          for (int p = 0; p < 4; ++p)
            if (m + p < g.M) C[m + p] = a4[p];
        }
      }
    }
  }
}

// out[n * ldc + m] = sum_z P[z][n][m] (z ascending), as bf16 or fp32.
__global__ __launch_bounds__(256) void k_reduce(const float* __restrict__ P, int splits, int M, int N,
                                                int64_t ldc, void* out, int out_bf16) {
  const int64_t total = (int64_t)N * ldc;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total; idx += (int64_t)gridDim.x * 256) {
    if (idx % ldc >= M) continue;
    float s = 0.f;
    for (int z = 0; z < splits; ++z) s += P[(int64_t)z * total + idx];
    if (out_bf16)
      static_cast<uint16_t*>(out)[idx] = f32_to_bf16(s);
    else
      static_cast<float*>(out)[idx] = s;
  }
}

// cptr[i * ncp + c] = first entry of row i whose column is >= c * 128
// (c = 0 .. ncp - 1; the last one is the row end).  Columns ascend in a row.
__global__ __launch_bounds__(256) void k_chunk_ptr(const int32_t* __restrict__ row_ptr,
                                                   const int32_t* __restrict__ col_idx, int m, int ncp,
                                                   int32_t* __restrict__ cptr) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)m * ncp) return;
  const int i = (int)(idx / ncp), c = (int)(idx % ncp);
  int lo = row_ptr[i], hi = row_ptr[i + 1];
  if (c < ncp - 1) {
    const int key = c * kKC;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (col_idx[mid] < key) lo = mid + 1; else hi = mid;
    }
  } else {
    lo = hi;
  }
  cptr[idx] = lo;
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
static inline int cdiv(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }
static inline size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Splits so that tiles * splits reaches ~256 blocks, at least 2 chunks each.
static int choose_splits(int tiles, int nch) {
  int s = 1;
  while (tiles * s < 256 && s * 2 <= nch / 2) s *= 2;
  return s;
}

struct MfmaPlan {
  int r, b;
  int t_splits, y_splits;
  size_t tb_off, cptr_off, part_off, total;
};

static MfmaPlan plan_mfma(const hss_matrix* A, int b) {
  MfmaPlan p;
  p.r = A->r; p.b = b;
  const int m = A->m, n = A->n, r = A->r;
  const int nch_t = cdiv(n, kKC);
  p.t_splits = r > 0 ? choose_splits(cdiv(r, kBM) * cdiv(b, kBN), nch_t) : 0;
  const int nch_y = cdiv(n, kKC) + (r > 0 ? cdiv(r, kKC) : 0);
  p.y_splits = choose_splits(cdiv(m, kBM) * cdiv(b, kBN), nch_y);
  size_t off = 0;
  p.tb_off = off;   off += align256(sizeof(uint16_t) * (size_t)b * (r > 0 ? r : 1));
  p.cptr_off = off; off += align256(sizeof(int32_t) * (size_t)m * (cdiv(n, kKC) + 1));
  p.part_off = off;
  const size_t part_t = p.t_splits > 1 ? sizeof(float) * (size_t)p.t_splits * b * r : 0;
  const size_t part_y = p.y_splits > 1 ? sizeof(float) * (size_t)p.y_splits * b * m : 0;
  off += align256(part_t > part_y ? part_t : part_y);
  p.total = off;
  return p;
}

bool mfma_supported(const hss_matrix* A, int b) {
  if (A->dtype != HSS_BF16 || b < 16) return false;
  if (A->fmt == HSS_FMT_2OF4 && (A->n % 32 != 0 || (uintptr_t)A->nm_values % 16 || (uintptr_t)A->nm_meta % 4))
    return false;
  return true;
}

size_t mfma_ws_bytes(const hss_matrix* A, int b) { return plan_mfma(A, b).total; }

static void run_gemm(GemmArgs g, int splits, float* part, hipStream_t s) {
  const int tm = cdiv(g.M, kBM), tn = cdiv(g.N, kBN);
  g.chunks_per_split = cdiv(g.nch, splits);
  void* final_out = g.C;
  const int64_t final_ldc = g.ldc;
  const int final_bf16 = g.out_mode == OUT_BF16;
  if (splits > 1) {
    g.C = part;
    g.out_mode = OUT_PARTIAL;
  }
  hipLaunchKernelGGL(k_gemm, dim3(tm, tn, splits), dim3(256), 0, s, g);
  if (splits > 1) {
    const int64_t total = (int64_t)g.N * final_ldc;
    const unsigned grid = (unsigned)std::min<int64_t>((total + 255) / 256, 4096);
    hipLaunchKernelGGL(k_reduce, dim3(grid), dim3(256), 0, s, part, splits, g.M, g.N, final_ldc, final_out,
                       final_bf16);
  }
}

static int aligned16(const void* p, int64_t ld) { return ((uintptr_t)p % 16 == 0) && (ld % 8 == 0); }

hss_status launch_mfma(const hss_matrix* A, int b, const void* X, void* Y, void* ws, hipStream_t s) {
  const MfmaPlan p = plan_mfma(A, b);
  char* base = static_cast<char*>(ws);
  uint16_t* Tb = reinterpret_cast<uint16_t*>(base + p.tb_off);
  int32_t* cptr = reinterpret_cast<int32_t*>(base + p.cptr_off);
  float* part = reinterpret_cast<float*>(base + p.part_off);
  const int m = A->m, n = A->n, r = A->r;
  const uint16_t* Xb = static_cast<const uint16_t*>(X);

  // T^T (b x r) = X . Vt^T
  if (r > 0) {
    GemmArgs g = {};
    g.M = r; g.N = b; g.K1 = n; g.K2 = 0;
    g.nch1 = g.nch = cdiv(n, kKC);
    g.a1_mode = A_DENSE;
    g.A1 = static_cast<const uint16_t*>(A->Vt); g.lda1 = n;
    g.B1 = Xb; g.ldb1 = n;
    g.C = Tb; g.ldc = r; g.out_mode = OUT_BF16;
    g.vec_a1 = aligned16(g.A1, n) && n % 8 == 0;
    g.vec_b1 = aligned16(Xb, n) && n % 8 == 0;
    run_gemm(g, p.t_splits, part, s);
  }
  // Y (b x m) = [X | T^T] . [S | U]^T
  GemmArgs g = {};
  g.M = m; g.N = b; g.K1 = n; g.K2 = r;
  g.nch1 = cdiv(n, kKC);
  g.nch = g.nch1 + (r > 0 ? cdiv(r, kKC) : 0);
  g.B1 = Xb; g.ldb1 = n;
  g.vec_b1 = aligned16(Xb, n) && n % 8 == 0;
  if (A->fmt == HSS_FMT_2OF4) {
    g.a1_mode = A_NM24;
    g.nmv = static_cast<const uint16_t*>(A->nm_values);
    g.meta = A->nm_meta;
  } else {
    g.a1_mode = A_CSR;
    g.col_idx = A->col_idx;
    g.vals = static_cast<const uint16_t*>(A->values);
    g.cptr = cptr;
    g.ncp = cdiv(n, kKC) + 1;
    const int64_t items = (int64_t)m * g.ncp;
    hipLaunchKernelGGL(k_chunk_ptr, dim3((unsigned)((items + 255) / 256)), dim3(256), 0, s, A->row_ptr,
                       A->col_idx, m, g.ncp, cptr);
  }
  if (r > 0) {
    g.A2 = static_cast<const uint16_t*>(A->U); g.lda2 = r;
    g.B2 = Tb; g.ldb2 = r;
    g.vec_a2 = aligned16(g.A2, r) && r % 8 == 0;
    g.vec_b2 = aligned16(Tb, r) && r % 8 == 0;
  }
  g.C = Y; g.ldc = m; g.out_mode = OUT_BF16;
  run_gemm(g, p.y_splits, part, s);
  return hipGetLastError() == hipSuccess ? HSS_OK : HSS_ERR_HIP;
}

}  // namespace hss
