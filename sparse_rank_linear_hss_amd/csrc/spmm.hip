// Batched CSR apply on the vector units (gather SpMM), bf16 layers.
//
// [HSS] page "LLMの階層的スパース+低ランク圧縮", section "実装と運用パターン": the
// forward pass is one sparse product plus two small dense products through
// the factors; section "2段階階層的スパース+低ランク圧縮" (vision rewrite):
// W ~ S + U V^T.  Here, for b columns:
//
//   T^T = (X V)^T                   (r x ldt, bf16) k_spmm_prep on the vector
//                                   units for b <= 64, else launch_tt_gemm on
//                                   the matrix cores
//   X^T                             (n x ldt) a plain transpose (k_spmm_prep's
//                                   other blocks, or k_xt)
//   Y[c][i] = sum_p S_ip X^T[col_p][c] + sum_l U[i][l] T^T[l][c]   k_spmm
//
// This is the alternative to densifying S into a dense GEMM operand: it
// reads S once and gathers, for every stored entry, one row of X^T (the
// entry's column across the batch tile) from L2, so its cost grows with
// nnz * b instead of m * n.  One wave owns one output row; within it, G
// lanes cover the batch tile's 8 G columns (16 bytes = 8 bf16 each) and the
// 64 / G lane groups ("slots") take every (64 / G)-th entry of the row.  The
// U part uses the same layout, with T's tile staged transposed in LDS.  The
// slot partial sums are added by an xor butterfly in a fixed order, so the
// result does not depend on scheduling.
#include <algorithm>

#include "hss_internal.h"

namespace hss {

void launch_tt_gemm(const hss_matrix* A, int b, const void* X, uint16_t* Tt, int ldt, float* part, hipStream_t s);
bool t_mfma_supported(const hss_matrix* A, const void* X);
void launch_t_mfma(const hss_matrix* A, int b, const void* X, uint16_t* T, int sl, int sc, hipStream_t s);
size_t tt_gemm_part_bytes(const hss_matrix* A, int b, int ldt);

static constexpr int kSpWaves = 8;            // rows (waves) per block
static constexpr int kSpLdsMax = 64 * 1024;   // LDS for the T tile
static constexpr int kSpLdsPref = 32 * 1024;  // ... preferred (more blocks per CU)
static constexpr int kPrepCb4MaxB = 16;       // T passes of 4 columns up to this batch
// k_spmm_prep's block: 512 threads (a 4096-column row in one step of 8
// columns each, all its loads in flight together) while the T passes take
// at most kPrepWideMaxBlocks blocks, else 256 (more blocks per CU).  11008 x
// 4096 rank 64 (64 .. 256 pass blocks), whole 2:4 calls, 256 vs 512
// threads: b = 2 18.3 vs 17.9 us, b = 32 25.8 vs 25.2 us; 4096^2 rank 256
// (256 .. 1024 pass blocks), gather calls: b = 3 11.1 vs 10.9 us, b = 16
// 14.3 vs 14.7 us, b = 64 30.0 vs 33.3 us.
static constexpr int kPrepWideMaxBlocks = 256;
static constexpr int kSpMaxG = 8;             // batch tile <= 64 columns
static constexpr int kSpDepth = 4;            // entries per lane in flight
static constexpr int kSpVecMaxB = 64;         // T on the vector units up to this batch, and
static constexpr int kPrepMaxTBlocks = 1024;  // while its passes take at most this many blocks;
                                              // beyond, T by k_nm_t where it can
// (4096^2 rank 256, passes of 16 columns side by side vs k_nm_t: b = 48 29.0
// vs 33.5 us, b = 64 30.0 vs 33.1 us; 8192^2 rank 512, 2048 pass blocks at
// b = 64: 77.7 vs 74.2 us.)

static size_t align256_(size_t x) { return (x + 255) & ~(size_t)255; }
static int cdiv_(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

struct SpmmArgs {
  const int32_t* row_ptr;
  const void* col;       // int32 or uint16 column indices
  const uint16_t* val;   // bf16 bits
  int64_t nnz;
  const uint16_t* U;     // m x r
  const uint16_t* Tt;    // r x ldt (columns past b unused)
  const uint16_t* Xt;    // n x ldt
  uint16_t* Y;           // b x m
  int m, n, r, b, ldt;
};

// X^T (n x ldt, zero columns past b) from X (b x n).  Thread t covers column
// j = t % n and the 8-column group t / n: eight 2-byte reads coalesced along
// j, one 16-byte store.
__global__ __launch_bounds__(256) void k_xt(const uint16_t* __restrict__ X, int b, int n, int ldt,
                                            uint16_t* __restrict__ Xt);

// One X^T work item of k_xt: column j, 8-column group cg.
__device__ __forceinline__ void xt_item(const uint16_t* __restrict__ X, int b, int n, int ldt, int64_t t,
                                        uint16_t* __restrict__ Xt) {
  const int cg = (int)(t / n), j = (int)(t - (int64_t)cg * n);
  uint32_t w[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int c = cg * 8 + 2 * k;
    const uint32_t lo = c < b ? X[(int64_t)c * n + j] : 0u;
    const uint32_t hi = c + 1 < b ? X[(int64_t)(c + 1) * n + j] : 0u;
    w[k] = lo | hi << 16;
  }
  const u32x4 v = {w[0], w[1], w[2], w[3]};
  *reinterpret_cast<u32x4*>(Xt + (int64_t)j * ldt + cg * 8) = v;
}

__global__ __launch_bounds__(256) void k_xt(const uint16_t* __restrict__ X, int b, int n, int ldt,
                                            uint16_t* __restrict__ Xt) {
  const int64_t total = (int64_t)n * (ldt >> 3);
  for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < total; t += (int64_t)gridDim.x * 256)
    xt_item(X, b, n, ldt, t, Xt);
}

// Prologue for b <= 64 in one launch.  Blocks 0 .. r-1: T^T row l = V^T[l] .
// X^T (b values), the block's threads striding over n (8 columns per step
// with 16-byte loads when VEC), CB batch columns per pass (4, 8 or 16: one
// X load per column and step); each column's sum
// is reduced within waves by DPP and the NTH / 64 wave sums added in order,
// so the result does not depend on scheduling; stored as bf16 at
// T[l * sl + c * sc] (sl = ldt, sc = 1: T^T; sl = 1, sc = row stride: T).
// Blocks r and up: X^T, as k_xt.
template <bool VEC, int CB, int NTH>
__global__ __launch_bounds__(NTH) void k_spmm_prep(const uint16_t* __restrict__ X, const uint16_t* __restrict__ Vt,
                                                   int b, int n, int r, int ldt, int sl, int sc,
                                                   uint16_t* __restrict__ Tt, uint16_t* __restrict__ Xt) {
  if ((int)blockIdx.x >= r) {
    if (blockIdx.y > 0) return;  // X^T once
    const int64_t total = (int64_t)n * (ldt >> 3);
    const int64_t nb = gridDim.x - r;
    for (int64_t t = (int64_t)(blockIdx.x - r) * NTH + threadIdx.x; t < total; t += nb * NTH)
      xt_item(X, b, n, ldt, t, Xt);
    return;
  }
  constexpr int kPrepWaves = NTH / 64;
  __shared__ float red[kPrepWaves][16];
  const int l = blockIdx.x, wave = threadIdx.x >> 6;
  const uint16_t* __restrict__ vrow = Vt + (int64_t)l * n;
  // pass blockIdx.y, and every gridDim.y-th after it
  for (int cb = CB * (int)blockIdx.y; cb < b; cb += CB * (int)gridDim.y) {
    float acc[CB];
#pragma unroll
    for (int cc = 0; cc < CB; ++cc) acc[cc] = 0.f;
    if constexpr (VEC) {
      // all CB + 1 loads of a step are unconditional (rows past b re-read row
      // b - 1 and are dropped after), so they are in flight together: a load
      // under a branch would be waited for inside it
      for (int j = 8 * threadIdx.x; j < n; j += 8 * NTH) {
        const u32x4 vv = *reinterpret_cast<const u32x4*>(vrow + j);
        u32x4 xx[CB];
#pragma unroll
        for (int cc = 0; cc < CB; ++cc)
          xx[cc] = *reinterpret_cast<const u32x4*>(X + (int64_t)min(cb + cc, b - 1) * n + j);
        const float vf[8] = {bf16lo(vv.x), bf16hi(vv.x), bf16lo(vv.y), bf16hi(vv.y),
                             bf16lo(vv.z), bf16hi(vv.z), bf16lo(vv.w), bf16hi(vv.w)};
#pragma unroll
        for (int cc = 0; cc < CB; ++cc) {
          float t = acc[cc];
          t = fmaf(vf[0], bf16lo(xx[cc].x), t); t = fmaf(vf[1], bf16hi(xx[cc].x), t);
          t = fmaf(vf[2], bf16lo(xx[cc].y), t); t = fmaf(vf[3], bf16hi(xx[cc].y), t);
          t = fmaf(vf[4], bf16lo(xx[cc].z), t); t = fmaf(vf[5], bf16hi(xx[cc].z), t);
          t = fmaf(vf[6], bf16lo(xx[cc].w), t); t = fmaf(vf[7], bf16hi(xx[cc].w), t);
          acc[cc] = t;
        }
      }
    } else {
      for (int j = threadIdx.x; j < n; j += NTH) {
        const float vf = bf16lo(vrow[j]);
#pragma unroll
        for (int cc = 0; cc < CB; ++cc)
          if (cb + cc < b) acc[cc] = fmaf(vf, bf16lo(X[(int64_t)(cb + cc) * n + j]), acc[cc]);
      }
    }
#pragma unroll
    for (int cc = 0; cc < CB; ++cc) {
      const float w = wave_sum(acc[cc]);
      if ((threadIdx.x & 63) == 0) red[wave][cc] = w;
    }
    __syncthreads();
    if (threadIdx.x < CB && cb + (int)threadIdx.x < b) {
      const int cc = threadIdx.x;
      float sum = red[0][cc];
#pragma unroll
      for (int w = 1; w < kPrepWaves; ++w) sum += red[w][cc];
      Tt[(int64_t)l * sl + (int64_t)(cb + cc) * sc] = f32_to_bf16(sum);
    }
    __syncthreads();
  }
}

__device__ __forceinline__ void fma8(float (&acc)[8], float v, const u32x4& x) {
  acc[0] = fmaf(v, bf16lo(x.x), acc[0]);
  acc[1] = fmaf(v, bf16hi(x.x), acc[1]);
  acc[2] = fmaf(v, bf16lo(x.y), acc[2]);
  acc[3] = fmaf(v, bf16hi(x.y), acc[3]);
  acc[4] = fmaf(v, bf16lo(x.z), acc[4]);
  acc[5] = fmaf(v, bf16hi(x.z), acc[5]);
  acc[6] = fmaf(v, bf16lo(x.w), acc[6]);
  acc[7] = fmaf(v, bf16hi(x.w), acc[7]);
}

// acc += v x (8 columns) when on, else acc unchanged (a masked entry adds
// nothing, whatever its x).
__device__ __forceinline__ void fma8_if(float (&acc)[8], float v, const u32x4& x, bool on) {
  float t[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) t[k] = acc[k];
  fma8(t, v, x);
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = on ? t[k] : acc[k];
}

template <typename CT>
__device__ __forceinline__ int load_col(__amdgpu_buffer_rsrc_t rc, int64_t p) {
  if constexpr (sizeof(CT) == 4)
    return (int)__builtin_amdgcn_raw_buffer_load_b32(rc, (int)(p * 4), 0, 0);
  else
    return (int)__builtin_amdgcn_raw_buffer_load_b16(rc, (int)(p * 2), 0, 0);
}

// Grid: x = row blocks of kSpWaves rows, y = batch tiles of 8 G columns.
// Dynamic LDS: r x 8G bf16 (T's tile, transposed).
template <int G, typename CT>
__global__ __launch_bounds__(kSpWaves * 64) void k_spmm(SpmmArgs a) {
  // entries per lane in flight: 8 with 32 slots (16 columns: a 4096-wide
  // 5 % row then needs one round of loads per lane; measured 17.0 -> 15.7
  // us), else 4 (8 was slower at 32-128 columns)
  constexpr int BT = 8 * G, S = 64 / G, D = G == 2 ? 2 * kSpDepth : kSpDepth;
  extern __shared__ uint16_t ts[];
  const int c0 = blockIdx.y * BT;
  const int r = a.r;
  const int wave = threadIdx.x >> 6, lane = lane_id();
  const int i = blockIdx.x * kSpWaves + wave;
  const bool live = i < a.m;  // wave-uniform
  const int g = lane % G, s = lane / G;

  // This wave's row bounds, then the first D entries of each lane and the
  // first D values of its U row, issued before the T tile's staging and
  // barrier so that their round trips overlap it.  The loads are
  // unconditional (buffer resources: past an array's end they read zeros;
  // past the row they read entries of the next one, masked out below).
  const int64_t rs = live ? a.row_ptr[i] : 0, re = live ? a.row_ptr[i + 1] : 0;
  const __amdgpu_buffer_rsrc_t rc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(a.col), 0, (int)(a.nnz * sizeof(CT)), 0x00020000);
  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.val), 0, (int)(a.nnz * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t ru =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.U), 0, (int)((int64_t)a.m * r * 2), 0x00020000);
  int64_t p = rs + s;
  int c1[D];
  float v1[D], u1[D];
#pragma unroll
  for (int k = 0; k < D; ++k) {
    c1[k] = load_col<CT>(rc, p + k * S);
    v1[k] = bf16lo(__builtin_amdgcn_raw_buffer_load_b16(rv, (int)((p + k * S) * 2), 0, 0));
    u1[k] = bf16lo(__builtin_amdgcn_raw_buffer_load_b16(ru, (int)(((int64_t)(live ? i : 0) * r + s + k * S) * 2), 0, 0));
  }

  // T tile -> LDS: ts[l * BT + c] = T^T[l][c0 + c], 16-byte pieces, four
  // loads in flight per thread before their stores.  Columns at or past b
  // (inside the last 8-column piece, or a whole piece past ldt) feed only
  // accumulators that are never stored.
  {
    constexpr int NT = kSpWaves * 64;
    const int pieces = r * G;
    const __amdgpu_buffer_rsrc_t rt = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(a.Tt), 0, (int)((int64_t)r * a.ldt * 2), 0x00020000);
    for (int q0 = threadIdx.x; q0 < pieces; q0 += 4 * NT) {
      u32x4 v[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int q = q0 + k * NT;
        const int l = q / G, pc = q - l * G;
        v[k] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                             rt, (l * a.ldt + c0 + 8 * pc) * 2, 0, 0));
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int q = q0 + k * NT;
        if (q < pieces) *reinterpret_cast<u32x4*>(ts + q * 8) = v[k];
      }
    }
  }
  __syncthreads();
  if (!live) return;  // no barrier follows
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};

  // sparse part: entries p = rs + s + S t in order -- the prefetched D
  // (masked past the row), then D per lane in flight (the column loads, then
  // the gathers), then the row's tail one at a time
  if (re > rs) {
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(a.Xt), 0, (int)((int64_t)a.n * a.ldt * 2), 0x00020000);
    const int xoff = (c0 + 8 * g) * 2;
    {
      u32x4 x[D];
#pragma unroll
      for (int k = 0; k < D; ++k)
        x[k] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, c1[k] * a.ldt * 2 + xoff, 0, 0));
#pragma unroll
      for (int k = 0; k < D; ++k) fma8_if(acc, v1[k], x[k], p + k * S < re);
      p += D * S;
    }
    for (; p + (D - 1) * S < re; p += D * S) {
      int c[D];
      float v[D];
#pragma unroll
      for (int k = 0; k < D; ++k) {
        c[k] = load_col<CT>(rc, p + k * S);
        v[k] = bf16lo(__builtin_amdgcn_raw_buffer_load_b16(rv, (int)((p + k * S) * 2), 0, 0));
      }
      u32x4 x[D];
#pragma unroll
      for (int k = 0; k < D; ++k)
        x[k] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, c[k] * a.ldt * 2 + xoff, 0, 0));
#pragma unroll
      for (int k = 0; k < D; ++k) fma8(acc, v[k], x[k]);
    }
    for (; p < re; p += S) {
      const int c = load_col<CT>(rc, p);
      const float v = bf16lo(__builtin_amdgcn_raw_buffer_load_b16(rv, (int)(p * 2), 0, 0));
      const u32x4 x = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, c * a.ldt * 2 + xoff, 0, 0));
      fma8(acc, v, x);
    }
  }
  // low-rank part: l = s + S t in order, U from memory (the first D
  // prefetched), T from LDS
  if (r > 0) {
    {
      u32x4 x[D];
#pragma unroll
      for (int k = 0; k < D; ++k) {
        const int l = s + k * S;
        x[k] = *reinterpret_cast<const u32x4*>(ts + (l < r ? l : r - 1) * BT + 8 * g);
      }
#pragma unroll
      for (int k = 0; k < D; ++k) fma8_if(acc, u1[k], x[k], s + k * S < r);
    }
    const uint16_t* __restrict__ ur = a.U + (int64_t)i * r;
    int l = s + D * S;
    for (; l + (D - 1) * S < r; l += D * S) {
      float u[D];
      u32x4 x[D];
#pragma unroll
      for (int k = 0; k < D; ++k) {
        u[k] = bf16lo(ur[l + k * S]);
        x[k] = *reinterpret_cast<const u32x4*>(ts + (l + k * S) * BT + 8 * g);
      }
#pragma unroll
      for (int k = 0; k < D; ++k) fma8(acc, u[k], x[k]);
    }
    for (; l < r; l += S) fma8(acc, bf16lo(ur[l]), *reinterpret_cast<const u32x4*>(ts + l * BT + 8 * g));
  }
  // sum over the slots (lanes with the same g), same bits in every lane
#pragma unroll
  for (int off = G; off < 64; off <<= 1) {
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] += __shfl_xor(acc[k], off, 64);
  }
  if (s == 0) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int c = c0 + 8 * g + k;
      if (c < a.b) a.Y[(int64_t)c * a.m + i] = f32_to_bf16(acc[k]);
    }
  }
}

// X^T (n x ldt, zero columns past b) of X (b x n): also used by the backward
// pass for G^T and U^T.
void launch_xt(const uint16_t* X, int b, int n, int ldt, uint16_t* Xt, hipStream_t s) {
  const int64_t work = (int64_t)n * (ldt >> 3);
  if (work == 0) return;
  hipLaunchKernelGGL(k_xt, dim3((unsigned)std::min<int64_t>(cdiv_(work, 256), 4096)), dim3(256), 0, s, X, b, n, ldt,
                     Xt);
}

// Batch tile: the smallest of 8, 16, 32, 64 columns that covers b (64 beyond),
// shrunk until T's tile fits the LDS budget.
// Batch tile 8 G: the widest that covers b and whose T tile takes at most
// kSpLdsPref of LDS (8192^2 rank 512, whose 64-column tile takes 64 KB: 4
// tiles of 32 columns at b = 64 / 128 took 67.7 / 103 us against 74.1 / 112
// with 2 / 1 tiles of 64; 4096^2 rank 256: 29.6 / 45.2 against 30.0 / 41.0).
static int spmm_g(const hss_matrix* A, int b) {
  int g = b <= 8 ? 1 : (b <= 16 ? 2 : (b <= 32 ? 4 : kSpMaxG));
  while (g > 1 && (size_t)A->r * 8 * g * 2 > kSpLdsPref) g >>= 1;
  return g;
}

static int spmm_ldt(int b) { return (b + 7) & ~7; }

bool spmm_supported(const hss_matrix* A, int b) {
  if (A->flags & HSS_DQ4) return false;
  if (A->fmt != HSS_FMT_CSR || A->dtype != HSS_BF16 || b < 1) return false;
  if ((size_t)A->r * 8 * 2 > kSpLdsMax) return false;                    // T tile of 8 columns must fit
  if ((int64_t)A->n * spmm_ldt(b) * 2 >= ((int64_t)1 << 31)) return false; // 32-bit buffer offsets
  if (A->nnz * 4 >= ((int64_t)1 << 31)) return false;
  if ((int64_t)A->m * A->r * 2 >= ((int64_t)1 << 31)) return false;  // U through a 32-bit buffer offset
  return true;
}

struct SpmmPlan {
  size_t tt_off, xt_off, part_off, total;
};

static SpmmPlan plan_spmm(const hss_matrix* A, int b) {
  SpmmPlan p;
  const int ldt = spmm_ldt(b);
  size_t off = 0;
  p.tt_off = off;   off += align256_(sizeof(uint16_t) * (size_t)ldt * (A->r > 0 ? A->r : 1));
  p.xt_off = off;   off += align256_(sizeof(uint16_t) * (size_t)A->n * ldt);
  p.part_off = off; off += align256_(tt_gemm_part_bytes(A, b, ldt));
  p.total = off;
  return p;
}

size_t spmm_ws_bytes(const hss_matrix* A, int b) { return plan_spmm(A, b).total; }

// Columns per T pass of k_spmm_prep: narrower passes load fewer X rows per
// step and run side by side.
static int prep_cb(int b) { return b <= kPrepCb4MaxB ? 4 : (b <= 32 ? 8 : 16); }

// Blocks the T passes of k_spmm_prep take for b columns.
int64_t prep_t_blocks(int r, int b) { return (int64_t)r * ((b + prep_cb(b) - 1) / prep_cb(b)); }

// k_spmm_prep with the pass width prep_cb(b).
template <bool VEC, int NTH>
static void launch_prep_vn(dim3 grid, const uint16_t* X, const uint16_t* Vt, int b, int n, int r, int ldt, int sl,
                           int sc, uint16_t* T, uint16_t* Xt, hipStream_t s) {
  if (prep_cb(b) == 4)
    hipLaunchKernelGGL((k_spmm_prep<VEC, 4, NTH>), grid, dim3(NTH), 0, s, X, Vt, b, n, r, ldt, sl, sc, T, Xt);
  else if (prep_cb(b) == 8)
    hipLaunchKernelGGL((k_spmm_prep<VEC, 8, NTH>), grid, dim3(NTH), 0, s, X, Vt, b, n, r, ldt, sl, sc, T, Xt);
  else
    hipLaunchKernelGGL((k_spmm_prep<VEC, 16, NTH>), grid, dim3(NTH), 0, s, X, Vt, b, n, r, ldt, sl, sc, T, Xt);
}

template <bool VEC>
static void launch_prep_v(dim3 grid, const uint16_t* X, const uint16_t* Vt, int b, int n, int r, int ldt, int sl,
                          int sc, uint16_t* T, uint16_t* Xt, hipStream_t s) {
  if (prep_t_blocks(r, b) <= kPrepWideMaxBlocks)
    launch_prep_vn<VEC, 512>(grid, X, Vt, b, n, r, ldt, sl, sc, T, Xt, s);
  else
    launch_prep_vn<VEC, 256>(grid, X, Vt, b, n, r, ldt, sl, sc, T, Xt, s);
}

// Grid: rank rows (then X^T blocks) along x, the passes of CB columns along
// y, so a block computes one pass (the passes run side by side).
static void launch_prep(bool vec, unsigned grid, const uint16_t* X, const uint16_t* Vt, int b, int n, int r, int ldt,
                        int sl, int sc, uint16_t* T, uint16_t* Xt, hipStream_t s) {
  const int cb = prep_cb(b);
  const dim3 g(grid, (unsigned)((b + cb - 1) / cb));
  if (vec)
    launch_prep_v<true>(g, X, Vt, b, n, r, ldt, sl, sc, T, Xt, s);
  else
    launch_prep_v<false>(g, X, Vt, b, n, r, ldt, sl, sc, T, Xt, s);
}

template <int G>
static void launch_spmm_g(const SpmmArgs& a, bool col16, hipStream_t s) {
  const dim3 grid((unsigned)cdiv_(a.m, kSpWaves), (unsigned)cdiv_(a.b, 8 * G));
  const size_t lds = (size_t)a.r * 8 * G * 2;
  if (col16)
    hipLaunchKernelGGL((k_spmm<G, uint16_t>), grid, dim3(kSpWaves * 64), lds, s, a);
  else
    hipLaunchKernelGGL((k_spmm<G, int32_t>), grid, dim3(kSpWaves * 64), lds, s, a);
}

hss_status launch_spmm(const hss_matrix* A, int b, const void* X, void* Y, void* ws, hipStream_t s) {
  const SpmmPlan p = plan_spmm(A, b);
  char* base = static_cast<char*>(ws);
  SpmmArgs a = {};
  a.row_ptr = A->row_ptr;
  a.col = A->col_idx;
  a.val = static_cast<const uint16_t*>(A->values);
  a.nnz = A->nnz;
  a.U = static_cast<const uint16_t*>(A->U);
  a.Tt = reinterpret_cast<uint16_t*>(base + p.tt_off);
  a.Xt = reinterpret_cast<uint16_t*>(base + p.xt_off);
  a.Y = static_cast<uint16_t*>(Y);
  a.m = A->m; a.n = A->n; a.r = A->r; a.b = b; a.ldt = spmm_ldt(b);
  const uint16_t* Xb = static_cast<const uint16_t*>(X);
  const int64_t work = (int64_t)A->n * (a.ldt >> 3);
  const int xt_blocks = A->nnz > 0 ? (int)std::min<int64_t>(cdiv_(work, 256), 1024) : 0;
  const bool t_vec = b <= kSpVecMaxB && prep_t_blocks(A->r, b) <= kPrepMaxTBlocks;
  if (!t_vec && t_mfma_supported(A, X)) {
    // T on the matrix cores, X^T by k_xt
    launch_t_mfma(A, b, X, const_cast<uint16_t*>(a.Tt), a.ldt, 1, s);
    if (xt_blocks > 0)
      hipLaunchKernelGGL(k_xt, dim3((unsigned)std::min<int64_t>(cdiv_(work, 256), 4096)), dim3(256), 0, s, Xb, b,
                         A->n, a.ldt, const_cast<uint16_t*>(a.Xt));
  } else if (b <= kSpVecMaxB) {
    // T and X^T in one launch
    const bool vec = A->n % 8 == 0 && (uintptr_t)X % 16 == 0 && (A->r == 0 || (uintptr_t)A->Vt % 16 == 0);
    const unsigned grid = (unsigned)(A->r + xt_blocks);
    if (grid > 0)
      launch_prep(vec, grid, Xb, static_cast<const uint16_t*>(A->Vt), b, A->n, A->r, a.ldt, a.ldt, 1,
                  const_cast<uint16_t*>(a.Tt), const_cast<uint16_t*>(a.Xt), s);
  } else {
    if (xt_blocks > 0)
      hipLaunchKernelGGL(k_xt, dim3((unsigned)std::min<int64_t>(cdiv_(work, 256), 4096)), dim3(256), 0, s, Xb, b,
                         A->n, a.ldt, const_cast<uint16_t*>(a.Xt));
    if (A->r > 0)
      launch_tt_gemm(A, b, X, const_cast<uint16_t*>(a.Tt), a.ldt, reinterpret_cast<float*>(base + p.part_off), s);
  }
  const bool col16 = (A->flags & HSS_COL16) != 0;
  switch (spmm_g(A, b)) {
    case 1: launch_spmm_g<1>(a, col16, s); break;
    case 2: launch_spmm_g<2>(a, col16, s); break;
    case 4: launch_spmm_g<4>(a, col16, s); break;
    default: launch_spmm_g<8>(a, col16, s); break;
  }
  return hipGetLastError() == hipSuccess ? HSS_OK : HSS_ERR_HIP;
}

// T = X V (b x r, bf16, row c at T + c * ldt, ldt >= r) on the vector units
// alone (k_spmm_prep's T blocks), b <= 64.
void launch_t_vec(const hss_matrix* A, int b, const void* X, int ldt, uint16_t* T, hipStream_t s) {
  if (A->r == 0) return;
  const uint16_t* Xb = static_cast<const uint16_t*>(X);
  const uint16_t* Vt = static_cast<const uint16_t*>(A->Vt);
  const bool vec = A->n % 8 == 0 && (uintptr_t)X % 16 == 0 && (uintptr_t)A->Vt % 16 == 0;
  launch_prep(vec, (unsigned)A->r, Xb, Vt, b, A->n, A->r, 8, 1, ldt, T, nullptr, s);
}

}  // namespace hss
