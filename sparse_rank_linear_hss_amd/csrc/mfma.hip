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
//                  segment 1: A = S, either 2:4 expanded in registers on its
//                  way to LDS, or CSR densified beforehand into a bf16 buffer
//                  in the workspace (m n zeros written, then the entries);
//                  segment 2: A = U, B = T^T.
//
// One kernel, k_gemm<BN, AMODE>: C = A . B^T with A (M x K) and B (N x K)
// both K-contiguous, fp32 accumulation in v_mfma_f32_32x32x16_bf16, output
// stored N-major (C[n * ldc + m]) so that Y (b x m) and T^T (b x r) come out
// in the layout their consumers read.  Tile 128 x BN (BN = 32, 64 or 128, the
// smallest covering b), K in chunks of 128 staged through LDS, the next
// chunk's global loads in flight during the current chunk's MFMA loop.  When
// there are too few tiles to fill the chip the K chunks are split across
// blocks; fp32 partials are then summed in a fixed order by k_reduce
// (deterministic, no float atomics).
#include <algorithm>

#include "hss_internal.h"

namespace hss {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 (lo in the low half) with gfx950's packed
// conversion: round to nearest even, NaN stays NaN -- the same bits as
// f32_to_bf16 for every other input, in one instruction instead of six.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
typedef float f32x16 __attribute__((ext_vector_type(16)));

enum : int { A_DENSE = 0, A_NM24 = 1 };
enum : int { OUT_BF16 = 0, OUT_F32 = 1, OUT_PARTIAL = 2 };

static constexpr int kBM = 128, kKC = 128;
static constexpr int kLdsStride = kKC + 8;  // bf16 elements per LDS row (16-byte pad: conflict-free reads)

struct GemmArgs {
  int M, N;
  int K1, K2;            // K segments: [0, K1) then [K1, K1 + K2)
  int nch1, nch;         // chunks in segment 1, total chunks
  int chunks_per_split;  // gridDim.z splits of the chunk range
  const uint16_t* A1;  int64_t lda1;   // dense A, segment 1 (M x K1)
  const uint16_t* nmv; const uint32_t* meta;            // 2:4 A, segment 1 (K1 % 32 == 0)
  const uint16_t* B1;  int64_t ldb1;   // N x K1
  const uint16_t* A2;  int64_t lda2;   // M x K2
  const uint16_t* B2;  int64_t ldb2;   // N x K2
  void* C; int64_t ldc; int out_mode;  // C[n * ldc + m]; partials: + z * N * ldc
  int vec_a1, vec_b1, vec_a2, vec_b2;  // 16-byte loads allowed (K % 8 == 0, aligned rows)
  int tiles_m, tiles_n;                // k_gemm_h: tiles per dimension (1-D grid of tiles_m * tiles_n * splits)
};

// Wave layout of a kBM x BN tile: WM x WN waves, each a (FM x FN) grid of
// 32 x 32 MFMA blocks.  BN is the batch tile (32, 64 or 128).
template <int BN>
struct TileShape {
  static constexpr int WM = BN >= 64 ? 2 : 4;
  static constexpr int WN = 4 / WM;
  static constexpr int FM = kBM / WM / 32;
  static constexpr int FN = BN / WN / 32;
  static constexpr int BV = BN * kKC / 8 / 256;  // 16-byte B vectors per thread per chunk
};

// A 128 x 128 chunk of a dense K-contiguous operand in registers: thread t
// holds 16-byte vectors q = t + 256 i (row q / 16, columns 8 (q % 16) ..).
// Loads use clamped (always valid) addresses; out-of-range parts are zeroed
// when written to LDS.
template <int NVEC>
struct DenseRegs {
  u32x4 v[NVEC];
};

template <int NVEC>
__device__ __forceinline__ void dense_load(DenseRegs<NVEC>& d, const uint16_t* __restrict__ src, int64_t ld,
                                           int r0, int R, int k0, int K) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < NVEC; ++i) {
    const int q = t + 256 * i;
    const int row = q >> 4, kq = (q & 15) * 8;
    const int rr = min(r0 + row, R - 1), kk = min(k0 + kq, K - 8);
    d.v[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + rr * ld + kk));
  }
}

template <int NVEC>
__device__ __forceinline__ void dense_store(uint16_t* __restrict__ lds, const DenseRegs<NVEC>& d, int r0, int R,
                                            int k0, int K) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < NVEC; ++i) {
    const int q = t + 256 * i;
    const int row = q >> 4, kq = (q & 15) * 8;
    const bool ok = r0 + row < R && k0 + kq < K;
    const u32x4 z = {0u, 0u, 0u, 0u};
    *reinterpret_cast<u32x4*>(lds + row * kLdsStride + kq) = ok ? d.v[i] : z;
  }
}

// Unaligned or odd-K operands: element-wise copy straight to LDS (no prefetch).
__device__ __forceinline__ void scalar_stage(uint16_t* __restrict__ lds, const uint16_t* __restrict__ src, int64_t ld,
                                             int rows, int r0, int R, int k0, int K) {
  for (int q = threadIdx.x; q < rows * kKC; q += 256) {
    const int row = q / kKC, kq = q % kKC;
    const bool ok = r0 + row < R && k0 + kq < K;
    lds[row * kLdsStride + kq] = ok ? src[(int64_t)(r0 + row) * ld + k0 + kq] : (uint16_t)0;
  }
}

// A 2:4 chunk in registers: thread t holds (row, word) items q = t + 256 i,
// row q / 4, word (k0 / 32) + q % 4: the metadata word and its 16 values.
struct NmRegs {
  uint32_t mw[2];
  u32x4 v[2][2];
};

__device__ __forceinline__ void nm_load(NmRegs& d, const uint16_t* __restrict__ nmv, const uint32_t* __restrict__ meta,
                                        int r0, int R, int k0, int K) {
  const int t = threadIdx.x;
  const int words = K >> 5;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = t + 256 * i;
    const int row = q >> 2, wd = (k0 >> 5) + (q & 3);
    const int rr = min(r0 + row, R - 1), wc = min(wd, words - 1);
    d.mw[i] = __builtin_nontemporal_load(meta + (int64_t)rr * words + wc);
    const u32x4* vp = reinterpret_cast<const u32x4*>(nmv + (int64_t)rr * (K >> 1) + wc * 16);
    d.v[i][0] = __builtin_nontemporal_load(vp);
    d.v[i][1] = __builtin_nontemporal_load(vp + 1);
  }
}

// Expand each item to its 32 dense columns (kept values at the positions the
// 2-bit indices name, zeros elsewhere).
__device__ __forceinline__ void nm_store(uint16_t* __restrict__ lds, const NmRegs& d, int r0, int R, int k0, int K) {
  const int t = threadIdx.x;
  const int words = K >> 5;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = t + 256 * i;
    const int row = q >> 2, wd = (k0 >> 5) + (q & 3);
    const bool ok = r0 + row < R && wd < words;
    const uint32_t vw[8] = {d.v[i][0].x, d.v[i][0].y, d.v[i][0].z, d.v[i][0].w,
                            d.v[i][1].x, d.v[i][1].y, d.v[i][1].z, d.v[i][1].w};
    uint32_t out[16];
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      const uint32_t nib = ok ? (d.mw[i] >> (4 * g)) & 15u : 0u;
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

// C (N-major) = A . B^T over this block's chunk range.  The next chunk's
// global loads are issued before the current chunk's MFMA loop, so their
// latency overlaps the matrix-core work (one LDS buffer, two barriers per
// chunk).
template <int BN, int AMODE>
__global__ __launch_bounds__(256) void k_gemm(GemmArgs g) {
  using TS = TileShape<BN>;
  __shared__ __align__(16) uint16_t As[kBM * kLdsStride];
  __shared__ __align__(16) uint16_t Bs[BN * kLdsStride];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int wm = w / TS::WN, wn = w % TS::WN;
  const int m0 = blockIdx.x * kBM, n0 = blockIdx.y * BN;
  const int c_begin = blockIdx.z * g.chunks_per_split;
  const int c_end = min(c_begin + g.chunks_per_split, g.nch);

  f32x16 acc[TS::FM][TS::FN];
#pragma unroll
  for (int i = 0; i < TS::FM; ++i)
#pragma unroll
    for (int j = 0; j < TS::FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  DenseRegs<8> ra;   // A chunk (dense)
  NmRegs rn;         // A chunk (2:4)
  DenseRegs<TS::BV> rb;

  // which operands a chunk uses
  auto seg1 = [&](int c) { return c < g.nch1; };
  auto a_vec = [&](int c) { return seg1(c) ? (AMODE == A_NM24 ? 1 : g.vec_a1) : g.vec_a2; };
  auto b_vec = [&](int c) { return seg1(c) ? g.vec_b1 : g.vec_b2; };

  auto issue = [&](int c) {
    if (seg1(c)) {
      const int k0 = c * kKC;
      if constexpr (AMODE == A_NM24) nm_load(rn, g.nmv, g.meta, m0, g.M, k0, g.K1);
      else if (g.vec_a1) dense_load(ra, g.A1, g.lda1, m0, g.M, k0, g.K1);
      if (g.vec_b1) dense_load(rb, g.B1, g.ldb1, n0, g.N, k0, g.K1);
    } else {
      const int k0 = (c - g.nch1) * kKC;
      if (g.vec_a2) dense_load(ra, g.A2, g.lda2, m0, g.M, k0, g.K2);
      if (g.vec_b2) dense_load(rb, g.B2, g.ldb2, n0, g.N, k0, g.K2);
    }
  };
  auto store = [&](int c) {
    if (seg1(c)) {
      const int k0 = c * kKC;
      if constexpr (AMODE == A_NM24) nm_store(As, rn, m0, g.M, k0, g.K1);
      else if (g.vec_a1) dense_store(As, ra, m0, g.M, k0, g.K1);
      else scalar_stage(As, g.A1, g.lda1, kBM, m0, g.M, k0, g.K1);
      if (g.vec_b1) dense_store(Bs, rb, n0, g.N, k0, g.K1);
      else scalar_stage(Bs, g.B1, g.ldb1, BN, n0, g.N, k0, g.K1);
    } else {
      const int k0 = (c - g.nch1) * kKC;
      if (g.vec_a2) dense_store(As, ra, m0, g.M, k0, g.K2);
      else scalar_stage(As, g.A2, g.lda2, kBM, m0, g.M, k0, g.K2);
      if (g.vec_b2) dense_store(Bs, rb, n0, g.N, k0, g.K2);
      else scalar_stage(Bs, g.B2, g.ldb2, BN, n0, g.N, k0, g.K2);
    }
  };
  (void)a_vec; (void)b_vec;

  if (c_begin < c_end) issue(c_begin);
  for (int c = c_begin; c < c_end; ++c) {
    __syncthreads();  // the previous chunk's MFMA reads are done
    store(c);
    __syncthreads();
    if (c + 1 < c_end) issue(c + 1);
#pragma unroll
    for (int s = 0; s < kKC / 16; ++s) {
      const int kk = s * 16 + 8 * (lane >> 5);
      bf16x8 af[TS::FM], bfr[TS::FN];
#pragma unroll
      for (int i = 0; i < TS::FM; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(As + (wm * TS::FM * 32 + i * 32 + (lane & 31)) * kLdsStride + kk);
#pragma unroll
      for (int j = 0; j < TS::FN; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8*>(Bs + (wn * TS::FN * 32 + j * 32 + (lane & 31)) * kLdsStride + kk);
#pragma unroll
      for (int i = 0; i < TS::FM; ++i)
#pragma unroll
        for (int j = 0; j < TS::FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  }

  // Epilogue: lane holds D[8*(v/4) + 4*(lane/32) + v%4][lane%32] of each 32x32 block.
#pragma unroll
  for (int i = 0; i < TS::FM; ++i) {
#pragma unroll
    for (int j = 0; j < TS::FN; ++j) {
      const int n = n0 + wn * TS::FN * 32 + j * 32 + (lane & 31);
      if (n >= g.N) continue;
#pragma unroll
      for (int vg = 0; vg < 4; ++vg) {
        const int m = m0 + wm * TS::FM * 32 + i * 32 + 8 * vg + 4 * (lane >> 5);
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

// ---------------------------------------------------------------------------
// Large tiles for big batches (prefill): 256 (M) x 128 (N) per block, each
// wave a 128 x 64 quarter (4 x 2 MFMA blocks, 128 accumulators), K in stages
// of 64 through one padded LDS buffer, the next stage's global loads in
// flight during the current stage's MFMA loop.  The wave tile reads 6 KiB of
// LDS per 8 MFMAs (the 64 x 64 tiles above: 4 KiB per 4), and a block is
// small enough (55 KiB LDS) for two to share a CU.  Dense operands whose rows
// allow 16-byte loads (K % 8 == 0).
// ---------------------------------------------------------------------------
static constexpr int kGM = 256, kGN = 128, kGK = 64;
static constexpr int kGStride = kGK + 8;  // bf16 per LDS row (16-byte pad: conflict-free fragment reads)

struct BigRegs {
  u32x4 a[8], b[4];
};

// Stage s: segment 1 (A1, B1) for s < nst1, else segment 2.  Thread t holds
// A vectors q = t + 256 i (row q / 8, columns 8 (q % 8) ..) and B likewise.
__device__ __forceinline__ void big_load(BigRegs& r, const GemmArgs& g, int nst1, int s, int m0, int n0) {
  const int t = threadIdx.x;
  const bool seg1 = s < nst1;
  const int k0 = (seg1 ? s : s - nst1) * kGK;
  const int K = seg1 ? g.K1 : g.K2;
  const uint16_t* __restrict__ A = seg1 ? g.A1 : g.A2;
  const uint16_t* __restrict__ B = seg1 ? g.B1 : g.B2;
  const int64_t lda = seg1 ? g.lda1 : g.lda2, ldb = seg1 ? g.ldb1 : g.ldb2;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int q = t + 256 * i;
    const int kk = min(k0 + (q & 7) * 8, K - 8);
    r.a[i] = __builtin_nontemporal_load(
        reinterpret_cast<const u32x4*>(A + (int64_t)min(m0 + (q >> 3), g.M - 1) * lda + kk));
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = t + 256 * i;
    const int kk = min(k0 + (q & 7) * 8, K - 8);
    r.b[i] = __builtin_nontemporal_load(
        reinterpret_cast<const u32x4*>(B + (int64_t)min(n0 + (q >> 3), g.N - 1) * ldb + kk));
  }
}

__device__ __forceinline__ void big_store(uint16_t* __restrict__ As, uint16_t* __restrict__ Bs, const BigRegs& r,
                                          const GemmArgs& g, int nst1, int s, int m0, int n0) {
  const int t = threadIdx.x;
  const bool seg1 = s < nst1;
  const int k0 = (seg1 ? s : s - nst1) * kGK;
  const int K = seg1 ? g.K1 : g.K2;
  const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int q = t + 256 * i, row = q >> 3, kq = (q & 7) * 8;
    *reinterpret_cast<u32x4*>(As + row * kGStride + kq) = (k0 + kq < K && m0 + row < g.M) ? r.a[i] : z;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = t + 256 * i, row = q >> 3, kq = (q & 7) * 8;
    *reinterpret_cast<u32x4*>(Bs + row * kGStride + kq) = (k0 + kq < K && n0 + row < g.N) ? r.b[i] : z;
  }
}

__global__ __launch_bounds__(256, 2) void k_gemm_big(GemmArgs g) {
  __shared__ __align__(16) uint16_t As[kGM * kGStride];
  __shared__ __align__(16) uint16_t Bs[kGN * kGStride];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int m0 = blockIdx.x * kGM, n0 = blockIdx.y * kGN;
  const int nst1 = (g.K1 + kGK - 1) / kGK;
  const int nst = nst1 + (g.K2 + kGK - 1) / kGK;
  const int s_begin = blockIdx.z * g.chunks_per_split;
  const int s_end = min(s_begin + g.chunks_per_split, nst);

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  BigRegs r;
  if (s_begin < s_end) big_load(r, g, nst1, s_begin, m0, n0);
  for (int s = s_begin; s < s_end; ++s) {
    __syncthreads();  // the previous stage's fragment reads are done
    big_store(As, Bs, r, g, nst1, s, m0, n0);
    __syncthreads();
    if (s + 1 < s_end) big_load(r, g, nst1, s + 1, m0, n0);
#pragma unroll
    for (int ks = 0; ks < kGK / 16; ++ks) {
      const int kk = ks * 16 + 8 * (lane >> 5);
      bf16x8 af[4], bfr[2];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(As + (wm * 128 + i * 32 + (lane & 31)) * kGStride + kk);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8*>(Bs + (wn * 64 + j * 32 + (lane & 31)) * kGStride + kk);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  }

#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + wn * 64 + j * 32 + (lane & 31);
      if (n >= g.N) continue;
#pragma unroll
      for (int vg = 0; vg < 4; ++vg) {
        const int m = m0 + wm * 128 + i * 32 + 8 * vg + 4 * (lane >> 5);
        if (g.out_mode == OUT_BF16) {
          uint16_t* C = static_cast<uint16_t*>(g.C) + (int64_t)n * g.ldc;
#pragma unroll
          for (int p = 0; p < 4; ++p)
            if (m + p < g.M) C[m + p] = f32_to_bf16(acc[i][j][4 * vg + p]);
        } else {
          float* C = static_cast<float*>(g.C) + (int64_t)blockIdx.z * g.N * g.ldc + (int64_t)n * g.ldc;
#pragma unroll
          for (int p = 0; p < 4; ++p)
            if (m + p < g.M) C[m + p] = acc[i][j][4 * vg + p];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Large tiles for big batches (prefill), k_gemm_h<FM, FN>: 4 waves, each a
// (32 FM) x (32 FN) part (FM x FN MFMA blocks) of a (64 FM) x (64 FN) tile;
// FM = FN = 4 gives 256 x 256 tiles with 128 x 128 per wave, where a wave
// reads 8 fragments from LDS per 16 MFMAs.  K runs in stages of 32: each
// stage is loaded into registers (buffer loads: one 32-bit offset per row,
// rows past the end read as zeros) while the one before it is computed,
// written to the other of two LDS buffers, and costs one barrier.  Rows of a
// stage are 64 bytes; chunk c (8 bf16) of row r sits at slot c ^ h_swz(r),
// so that the stores and the fragment reads do not conflict on LDS banks.
// Needs K1 and K2 multiples of 32 and 16-byte aligned rows.
// ---------------------------------------------------------------------------
static constexpr int kHK = 32;

template <int FM, int FN>
struct HTile {
  static constexpr int TM = 64 * FM, TN = 64 * FN;  // block tile
  static constexpr int STAGE = (TM + TN) * kHK;      // bf16 per LDS buffer: A rows, then B rows
};

// Slot of 16-byte chunk c of LDS row r is c ^ h_swz(r).  A fragment read
// (ds_read_b128, lane l: row base + l % 32, one chunk) must put the lanes the
// LDS serves together on distinct banks: 8 consecutive rows in a 128-byte
// bank window, or 16 in a 256-byte one.  Rows are 64 bytes, so rows r and
// r + 2 (r + 4) share a window position and need different slots;
// ((r >> 1) & 3) ^ ((r >> 3) & 1) gives that for both group sizes (the
// former (r >> 1) & 3 repeated every 8 rows: 88-94 % of the LDS cycles of the
// prefill GEMMs were bank conflicts by SQ_LDS_BANK_CONFLICT).  Stores (4 lanes
// per row, rows in order) fill whole windows and do not conflict.
__device__ __forceinline__ int h_swz(int r) { return ((r >> 1) & 3) ^ ((r >> 3) & 1); }

template <int FM, int FN>
struct HRegs {
  u32x4 a[FM], b[FN];  // thread t: chunks q = t + 256 i (row q / 4, chunk q % 4) of A and of B
};

// The four operands as buffer resources (32-bit offsets, one register per
// row instead of a 64-bit pointer; rows past the end read as zeros).
struct HOps {
  __amdgpu_buffer_rsrc_t a1, b1, a2, b2;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t h_rsrc(const uint16_t* p, int rows, int64_t ld) {
  const int64_t bytes = p ? (int64_t)rows * ld * 2 : 0;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p), 0, (int)bytes, 0x00020000);
}

// Stage s: rows r0 + (t >> 2) + 64 i, columns k0 + 8 (t & 3) .. of A and B.
template <int FM, int FN>
__device__ __forceinline__ void h_load(HRegs<FM, FN>& r, const GemmArgs& g, const HOps& ops, int nst1, int s, int m0,
                                       int n0) {
  const int t = threadIdx.x;
  const bool seg1 = s < nst1;
  const int k0 = (seg1 ? s : s - nst1) * kHK;
  const int lda = (int)(seg1 ? g.lda1 : g.lda2), ldb = (int)(seg1 ? g.ldb1 : g.ldb2);
  const uint32_t koff = 2u * (uint32_t)(k0 + 8 * (t & 3));
  const uint32_t arow = 2u * (uint32_t)(m0 + (t >> 2)) * (uint32_t)lda + koff;
  const uint32_t brow = 2u * (uint32_t)(n0 + (t >> 2)) * (uint32_t)ldb + koff;
  const uint32_t astep = 128u * (uint32_t)lda, bstep = 128u * (uint32_t)ldb;  // 64 rows
#pragma unroll
  for (int i = 0; i < FM; ++i)
    r.a[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(seg1 ? ops.a1 : ops.a2, arow + i * astep, 0, 0));
#pragma unroll
  for (int i = 0; i < FN; ++i)
    r.b[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(seg1 ? ops.b1 : ops.b2, brow + i * bstep, 0, 0));
}

template <int FM, int FN>
__device__ __forceinline__ void h_store(uint16_t* __restrict__ buf, const HRegs<FM, FN>& r) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int row = (t >> 2) + 64 * i, c = t & 3;
    *reinterpret_cast<u32x4*>(buf + row * kHK + 8 * (c ^ h_swz(row))) = r.a[i];
  }
#pragma unroll
  for (int i = 0; i < FN; ++i) {
    const int row = (t >> 2) + 64 * i, c = t & 3;
    *reinterpret_cast<u32x4*>(buf + HTile<FM, FN>::TM * kHK + row * kHK + 8 * (c ^ h_swz(row))) = r.b[i];
  }
}

// The MFMAs of one stage.
template <int FM, int FN>
__device__ __forceinline__ void h_compute(const uint16_t* __restrict__ buf, int wm, int wn, f32x16 (&acc)[FM][FN]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int ks = 0; ks < kHK / 16; ++ks) {
    const int c = 2 * ks + (lane >> 5);
    bf16x8 af[FM], bfr[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int row = wm * 32 * FM + 32 * i + (lane & 31);
      af[i] = *reinterpret_cast<const bf16x8*>(buf + row * kHK + 8 * (c ^ h_swz(row)));
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int row = wn * 32 * FN + 32 * j + (lane & 31);
      bfr[j] = *reinterpret_cast<const bf16x8*>(buf + HTile<FM, FN>::TM * kHK + row * kHK + 8 * (c ^ h_swz(row)));
    }
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
  }
}

// Tile of block b in a 1-D grid of G = tiles_m * tiles_n * splits blocks.
// Blocks are dealt to the 8 XCDs round robin (b % 8), each XCD with its own
// L2, so each XCD gets a contiguous range of tile numbers (when G % 8 == 0),
// and tile numbers run down groups of 8 tiles along M before moving along N
// (split z outermost): the blocks of one XCD then share their A and B slabs
// in its L2 instead of each fetching them from memory.
__device__ __forceinline__ void h_tile_of(int b, int tiles_m, int tiles_n, int G, int& tm, int& tn, int& tz) {
  const int t = G % 8 == 0 ? (b % 8) * (G / 8) + b / 8 : b;
  const int per_z = tiles_m * tiles_n;
  tz = t / per_z;
  const int u = t - tz * per_z;
  const int group = 8 * tiles_n;  // tiles in a group of 8 M-tiles
  const int first_m = (u / group) * 8;
  const int gm = min(tiles_m - first_m, 8);
  const int v = u - (u / group) * group;
  tm = first_m + v % gm;
  tn = v / gm;
}

template <int FM, int FN>
__global__ __launch_bounds__(256, (FM * FN >= 16 ? 1 : 2)) void k_gemm_h(GemmArgs g) {
  using TL = HTile<FM, FN>;
  constexpr bool DEEP = FM * FN < 8;  // two stages in registers
  __shared__ __align__(16) uint16_t hb0[TL::STAGE], hb1[TL::STAGE];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w >> 1, wn = w & 1;
  int tm, tn, tz;
  h_tile_of(blockIdx.x, g.tiles_m, g.tiles_n, (int)gridDim.x, tm, tn, tz);
  const int m0 = tm * TL::TM, n0 = tn * TL::TN;
  const int nst1 = g.K1 / kHK;
  const int nst = nst1 + g.K2 / kHK;
  const int s_begin = tz * g.chunks_per_split;
  const int s_end = min(s_begin + g.chunks_per_split, nst);
  // An AGPR named in an (empty) asm makes the compiler treat the kernel as
  // one that uses AGPRs, so the MFMAs keep their accumulators there;
  // otherwise they are selected with VGPR accumulators, which do not fit.
  asm volatile("" ::: "a0");
  HOps ops;
  ops.a1 = h_rsrc(g.A1, g.M, g.lda1);
  ops.b1 = h_rsrc(g.B1, g.N, g.ldb1);
  ops.a2 = h_rsrc(g.A2, g.M, g.lda2);
  ops.b2 = h_rsrc(g.B2, g.N, g.ldb2);

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  // Stage s_begin + d sits in LDS buffer d % 2.  Two register sets hold the
  // next two stages, so every stage's loads have two stages of MFMA work to
  // land in (one was not enough to cover a memory round trip on the short-K
  // products).  Loads past the end reload the last stage (unconditional, so
  // the compiler keeps one copy of each register set), and their stores fill
  // a buffer nobody reads.
  if (DEEP && s_begin < s_end) {
    const int last = s_end - 1;
    HRegs<FM, FN> r0, r1;
    h_load<FM, FN>(r0, g, ops, nst1, s_begin, m0, n0);
    h_store<FM, FN>(hb0, r0);
    h_load<FM, FN>(r0, g, ops, nst1, min(s_begin + 1, last), m0, n0);
    h_load<FM, FN>(r1, g, ops, nst1, min(s_begin + 2, last), m0, n0);
    __syncthreads();
    // Pairs of stages, then an odd last one: no exit from the middle of the
    // loop body.  With one, the compiler moved accumulators between AGPRs
    // and VGPRs on every iteration (the 128 x 128 tile then took 88 VGPRs +
    // 128 AGPRs, now 82 + 64; the 128 x 256 tile spilled).  The 128 x 256
    // tile with two register sets, which now fits (128 + 128), measured no
    // faster: 28.5 against 27.2 us for the K = 512 product of the 8192^2
    // prefill, 305 against 299 us with the dense S.
    int s = s_begin;
    for (; s + 1 < s_end; s += 2) {
      // stage s in hb0, s + 1 in r0, s + 2 in r1
      h_compute<FM, FN>(hb0, wm, wn, acc);
      h_store<FM, FN>(hb1, r0);
      h_load<FM, FN>(r0, g, ops, nst1, min(s + 3, last), m0, n0);
      __syncthreads();
      h_compute<FM, FN>(hb1, wm, wn, acc);
      h_store<FM, FN>(hb0, r1);
      h_load<FM, FN>(r1, g, ops, nst1, min(s + 4, last), m0, n0);
      __syncthreads();
    }
    if (s < s_end) {  // stage s, in hb0; the barrier frees hb0 for the output staging
      h_compute<FM, FN>(hb0, wm, wn, acc);
      __syncthreads();
    }
  } else if (!DEEP && s_begin < s_end) {
    // one register set (128 x 256 tiles: two measured no faster; 256 x 256:
    // a second set does not fit beside the 256 accumulators)
    const int last = s_end - 1;
    HRegs<FM, FN> r;
    h_load<FM, FN>(r, g, ops, nst1, s_begin, m0, n0);
    h_store<FM, FN>(hb0, r);
    h_load<FM, FN>(r, g, ops, nst1, min(s_begin + 1, last), m0, n0);
    __syncthreads();
    for (int s = s_begin; s < s_end; ++s) {
      const int odd = (s - s_begin) & 1;
      h_compute<FM, FN>(odd ? hb1 : hb0, wm, wn, acc);
      h_store<FM, FN>(odd ? hb0 : hb1, r);
      h_load<FM, FN>(r, g, ops, nst1, min(s + 2, last), m0, n0);
      __syncthreads();
    }
  }

  // Output.  bf16: each wave stages 32 columns n x its 32 FM rows m of C at
  // a time in its own part of LDS (16-byte chunk cm of row n at
  // cm ^ (n % 4 FM)), then writes every row n as 64 FM contiguous bytes in
  // 16-byte stores.  fp32 partials: 16-byte stores of 4 consecutive m
  // straight from the accumulators.
  const int mw0 = m0 + wm * 32 * FM, nw0 = n0 + wn * 32 * FN;
  if (g.out_mode == OUT_BF16) {
    constexpr int CH = 4 * FM;       // 16-byte chunks per staged row
    constexpr int RPI = 64 / CH;     // rows per read instruction
    static_assert(4 * 32 * 32 * FM <= TL::STAGE, "staging fits one LDS buffer");
    uint16_t* stage = hb0 + w * 32 * 32 * FM;  // hb0 is free: the loop ended on a barrier
    uint16_t* C = static_cast<uint16_t*>(g.C);
    const bool vec_out = ((uintptr_t)C % 16 == 0) && (g.ldc % 8 == 0);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int nl = lane & 31, h = lane >> 5;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int vg = 0; vg < 4; ++vg) {
          const int cm = 4 * i + vg;
          u32x2 v2;
          v2.x = pack_bf16x2(acc[i][j][4 * vg], acc[i][j][4 * vg + 1]);
          v2.y = pack_bf16x2(acc[i][j][4 * vg + 2], acc[i][j][4 * vg + 3]);
          *reinterpret_cast<u32x2*>(stage + nl * 8 * CH + 8 * (cm ^ (nl % CH)) + 4 * h) = v2;
        }
#pragma unroll
      for (int q = 0; q < 32 / RPI; ++q) {
        const int nl2 = RPI * q + lane / CH, cm = lane % CH;
        const u32x4 v = *reinterpret_cast<const u32x4*>(stage + nl2 * 8 * CH + 8 * (cm ^ (nl2 % CH)));
        const int n = nw0 + 32 * j + nl2, m = mw0 + 8 * cm;
        if (n < g.N) {
          uint16_t* dst = C + (int64_t)n * g.ldc + m;
          if (vec_out && m + 8 <= g.M) {
            *reinterpret_cast<u32x4*>(dst) = v;
          } else {
            const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (m + e < g.M) dst[e] = (uint16_t)(w4[e >> 1] >> (16 * (e & 1)));
          }
        }
      }
    }
  } else {
    float* C = static_cast<float*>(g.C) + (int64_t)tz * g.N * g.ldc;
    const bool vec_out = ((uintptr_t)C % 16 == 0) && (g.ldc % 4 == 0);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int n = nw0 + j * 32 + (lane & 31);
        if (n >= g.N) continue;
#pragma unroll
        for (int vg = 0; vg < 4; ++vg) {
          const int m = mw0 + i * 32 + 8 * vg + 4 * (lane >> 5);
          float* dst = C + (int64_t)n * g.ldc + m;
          if (vec_out && m + 4 <= g.M) {
            float4 v;
            v.x = acc[i][j][4 * vg]; v.y = acc[i][j][4 * vg + 1];
            v.z = acc[i][j][4 * vg + 2]; v.w = acc[i][j][4 * vg + 3];
            *reinterpret_cast<float4*>(dst) = v;
          } else {
#pragma unroll
            for (int p = 0; p < 4; ++p)
              if (m + p < g.M) dst[p] = acc[i][j][4 * vg + p];
          }
        }
      }
  }
}

// Dense bf16 copy D (m x n, row-major) of a CSR matrix, one wave per row,
// kDensSeg columns at a time: the wave zeroes its segment in LDS, its lanes
// scatter the row's entries that fall in the segment, and the segment goes out
// in 16-byte stores, so D is written once.  (Zeroing the row in memory and
// scattering the entries over it wrote every row twice, the second time in
// 2-byte stores: 51 us for the 8192^2 layer.)  Segment 1 of the batched apply
// then reads S as a dense operand.
static constexpr int kDensSeg = 4096;  // columns per segment: 8 KiB of LDS per wave
template <typename COL>
__global__ __launch_bounds__(256) void k_csr_densify(const int32_t* __restrict__ row_ptr,
                                                     const COL* __restrict__ col_idx,
                                                     const uint16_t* __restrict__ vals, int m, int n,
                                                     uint16_t* __restrict__ D) {
  __shared__ __align__(16) uint16_t seg[4][kDensSeg];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int row = blockIdx.x * 4 + w;
  if (row >= m) return;  // no block-wide barrier below
  uint16_t* Dr = D + (int64_t)row * n;  // n % 8 == 0, D 16-byte aligned
  uint16_t* L = seg[w];
  const int p0 = row_ptr[row], p1 = row_ptr[row + 1];
  const u32x4 z = {0u, 0u, 0u, 0u};
  for (int c0 = 0; c0 < n; c0 += kDensSeg) {
    const int len = min(kDensSeg, n - c0);  // a multiple of 8
    for (int j = 8 * lane; j < len; j += 512) *reinterpret_cast<u32x4*>(L + j) = z;
    // A wave's LDS accesses complete in issue order; the empty asm keeps the
    // compiler from moving the 2-byte entry stores above the zeros, and the
    // 16-byte reads below above the entry stores.
    asm volatile("" ::: "memory");
    for (int p = p0 + lane; p < p1; p += 64) {
      const int c = (int)col_idx[p] - c0;
      if ((unsigned)c < (unsigned)len) L[c] = vals[p];
    }
    asm volatile("" ::: "memory");
    for (int j = 8 * lane; j < len; j += 512)
      *reinterpret_cast<u32x4*>(Dr + c0 + j) = *reinterpret_cast<const u32x4*>(L + j);
    asm volatile("" ::: "memory");  // the next segment's zeros after these reads
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

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
static inline int cdiv(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }
static inline size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Batch tile: the smallest of 32, 64, 128 that covers b (larger b tiles by 128).
static int batch_tile(int b) { return b <= 32 ? 32 : (b <= 64 ? 64 : 128); }

// Splits so that tiles * splits reaches ~`target` blocks, at least 2 chunks each.
static int choose_splits(int tiles, int nch, int target = 256) {
  int s = 1;
  while (tiles * s < target && s * 2 <= nch / 2) s *= 2;
  return s;
}

// Kernel choice for one GEMM (M x N outputs, K = K1 + K2): k_gemm_h for
// dense 16-byte-aligned operands with K segments in whole stages of 32 and
// M, N >= 128 -- 128 x 256 tiles when there are at least 64 of them, else
// 128 x 128, with K split until there are ~256 blocks (one per CU); else
// 256 x 128 tiles (k_gemm_big) for dense aligned operands and N >= 256; else
// k_gemm<BN>.  Measured on the 8192^2 rank-512 layer at b = 2048: the
// 2048 x 8192 products take 23 us (K 512) and 238 us (K 8704, 49 % of the
// bf16 MFMA peak) with 128 x 256 tiles, 26 and 249 us with 256 x 256; the
// 2048 x 512 one (K 8192, operands in cache) 25.9 us with 128 x 128 tiles
// split 4 ways, 26.6 split 8 ways (which also gives k_reduce twice the
// partials to read), 31.0 split 16 ways, 40.5 with 128 x 256 tiles split 4.
enum : int { G_SMALL = 0, G_BIG = 1, G_H = 2 };
struct GemmCfg {
  int kind;
  int bn, splits;
  int fm, fn;  // k_gemm_h tile: (64 fm) x (64 fn)
};

static GemmCfg gemm_cfg(int M, int N, int K1, int K2, bool big_ok, bool h_ok) {
  GemmCfg c;
  if (h_ok && M >= 128 && N >= 128 && K1 % kHK == 0 && K2 % kHK == 0) {
    c.kind = G_H;
    c.fm = 2;
    c.fn = N >= 256 && cdiv(M, 128) * cdiv(N, 256) >= 64 ? 4 : 2;
    c.bn = 64 * c.fn;
    c.splits = choose_splits(cdiv(M, 64 * c.fm) * cdiv(N, 64 * c.fn), K1 / kHK + K2 / kHK, 256);
  } else if (big_ok && N >= 256) {
    c.fm = c.fn = 0;
    c.kind = G_BIG;
    c.bn = kGN;
    c.splits = choose_splits(cdiv(M, kGM) * cdiv(N, kGN), cdiv(K1, kGK) + cdiv(K2, kGK));
  } else {
    c.fm = c.fn = 0;
    c.kind = G_SMALL;
    c.bn = batch_tile(N);
    c.splits = choose_splits(cdiv(M, kBM) * cdiv(N, c.bn), cdiv(K1, kKC) + cdiv(K2, kKC));
  }
  return c;
}

// fp32 partials of one GEMM: enough for every kernel choice (operand
// alignment, which decides between them, is known only at launch).
static size_t gemm_part_bytes(int M, int N, int K1, int K2) {
  size_t mx = 0;
  for (int kind = 0; kind < 3; ++kind) {
    const GemmCfg c = gemm_cfg(M, N, K1, K2, kind >= G_BIG, kind == G_H);
    if (c.splits > 1) mx = std::max(mx, sizeof(float) * (size_t)c.splits * N * M);
  }
  return mx;
}

struct MfmaPlan {
  size_t tb_off, dense_off, part_off, total;
};

static bool csr_empty(const hss_matrix* A) { return A->fmt == HSS_FMT_CSR && A->nnz == 0; }

static MfmaPlan plan_mfma(const hss_matrix* A, int b) {
  MfmaPlan p;
  const int m = A->m, n = A->n, r = A->r;
  const int k1 = csr_empty(A) ? 0 : n;
  size_t off = 0;
  p.tb_off = off;    off += align256(sizeof(uint16_t) * (size_t)b * (r > 0 ? r : 1));
  p.dense_off = off;
  if (A->fmt == HSS_FMT_CSR && k1 > 0) off += align256(sizeof(uint16_t) * (size_t)m * n);
  p.part_off = off;
  const size_t part_t = r > 0 ? gemm_part_bytes(r, b, n, 0) : 0;
  const size_t part_y = gemm_part_bytes(m, b, k1, r);
  off += align256(std::max(part_t, part_y));
  p.total = off;
  return p;
}

// Matrix cores from 16 columns (2:4) or 24 (CSR: up to 16 columns, two fused
// decode passes with X in LDS beat densifying S -- measured 43 vs 49 us on
// the 4096 x 4096 5 % layer).
bool mfma_supported(const hss_matrix* A, int b) {
  if (A->flags & HSS_DQ4) return false;  // dense-and-sparse: its own fused kernel
  if (A->dtype != HSS_BF16 || b < (A->fmt == HSS_FMT_CSR ? 24 : 16)) return false;
  if (A->fmt == HSS_FMT_CSR && A->n % 8 != 0) return false;  // dense copy written in 16-byte rows
  if (A->fmt == HSS_FMT_2OF4 && (A->n % 32 != 0 || (uintptr_t)A->nm_values % 16 || (uintptr_t)A->nm_meta % 4))
    return false;
  return true;
}

size_t mfma_ws_bytes(const hss_matrix* A, int b) { return plan_mfma(A, b).total; }

template <int BN>
static void launch_gemm_bn(const GemmArgs& g, int amode, int splits, hipStream_t s) {
  const dim3 grid(cdiv(g.M, kBM), cdiv(g.N, BN), splits);
  if (amode == A_NM24)
    hipLaunchKernelGGL((k_gemm<BN, A_NM24>), grid, dim3(256), 0, s, g);
  else
    hipLaunchKernelGGL((k_gemm<BN, A_DENSE>), grid, dim3(256), 0, s, g);
}

static int aligned16(const void* p, int64_t ld) { return ((uintptr_t)p % 16 == 0) && (ld % 8 == 0); }

// Operand rows * ld bf16 fit the 32-bit byte offsets of k_gemm_h's buffer loads.
static bool fits_u31(int rows, int64_t ld) { return (int64_t)rows * ld * 2 < ((int64_t)1 << 31); }

static void run_gemm(GemmArgs g, int amode, float* part, hipStream_t s) {
  const bool big_ok = amode == A_DENSE && (g.K1 == 0 || (g.vec_a1 && g.vec_b1)) &&
                      (g.K2 == 0 || (g.vec_a2 && g.vec_b2));
  const bool h_ok = big_ok && (g.K1 == 0 || (fits_u31(g.M, g.lda1) && fits_u31(g.N, g.ldb1))) &&
                    (g.K2 == 0 || (fits_u31(g.M, g.lda2) && fits_u31(g.N, g.ldb2)));
  const GemmCfg c = gemm_cfg(g.M, g.N, g.K1, g.K2, big_ok, h_ok);
  g.chunks_per_split = cdiv(g.nch, c.splits);
  if (c.kind == G_BIG) g.chunks_per_split = cdiv(cdiv(g.K1, kGK) + cdiv(g.K2, kGK), c.splits);
  if (c.kind == G_H) g.chunks_per_split = cdiv(g.K1 / kHK + g.K2 / kHK, c.splits);
  void* final_out = g.C;
  const int64_t final_ldc = g.ldc;
  const int final_bf16 = g.out_mode == OUT_BF16;
  if (c.splits > 1) {
    g.C = part;
    g.out_mode = OUT_PARTIAL;
  }
  if (c.kind == G_H) {
    g.tiles_m = cdiv(g.M, 64 * c.fm);
    g.tiles_n = cdiv(g.N, 64 * c.fn);
    const dim3 grid((unsigned)(g.tiles_m * g.tiles_n * c.splits));
    if (c.fn == 4)
      hipLaunchKernelGGL((k_gemm_h<2, 4>), grid, dim3(256), 0, s, g);
    else
      hipLaunchKernelGGL((k_gemm_h<2, 2>), grid, dim3(256), 0, s, g);
  }
  else if (c.kind == G_BIG)
    hipLaunchKernelGGL(k_gemm_big, dim3(cdiv(g.M, kGM), cdiv(g.N, kGN), c.splits), dim3(256), 0, s, g);
  else if (c.bn == 32) launch_gemm_bn<32>(g, amode, c.splits, s);
  else if (c.bn == 64) launch_gemm_bn<64>(g, amode, c.splits, s);
  else launch_gemm_bn<128>(g, amode, c.splits, s);
  if (c.splits > 1) {
    const int64_t total = (int64_t)g.N * final_ldc;
    const unsigned grid = (unsigned)std::min<int64_t>((total + 255) / 256, 4096);
    hipLaunchKernelGGL(k_reduce, dim3(grid), dim3(256), 0, s, part, c.splits, g.M, g.N, final_ldc, final_out,
                       final_bf16);
  }
}

// T (b x r, bf16, row c = X[c] . V) on the matrix cores; `part` holds the
// split-K partials (sized by plan_mfma).
static void launch_t_gemm(const hss_matrix* A, int b, const void* X, uint16_t* Tb, float* part, hipStream_t s) {
  const int n = A->n, r = A->r;
  const uint16_t* Xb = static_cast<const uint16_t*>(X);
  GemmArgs g = {};
  g.M = r; g.N = b; g.K1 = n; g.K2 = 0;
  g.nch1 = g.nch = cdiv(n, kKC);
  g.A1 = static_cast<const uint16_t*>(A->Vt); g.lda1 = n;
  g.B1 = Xb; g.ldb1 = n;
  g.C = Tb; g.ldc = r; g.out_mode = OUT_BF16;
  g.vec_a1 = aligned16(g.A1, n) && n % 8 == 0;
  g.vec_b1 = aligned16(Xb, n) && n % 8 == 0;
  run_gemm(g, A_DENSE, part, s);
}

// T transposed: Tt[l * ldt + c] = (X V)[c][l] (r x b, row stride ldt >= b;
// columns past b are not written), the GEMM with X as the M operand.
void launch_tt_gemm(const hss_matrix* A, int b, const void* X, uint16_t* Tt, int ldt, float* part, hipStream_t s) {
  const int n = A->n, r = A->r;
  const uint16_t* Xb = static_cast<const uint16_t*>(X);
  GemmArgs g = {};
  g.M = b; g.N = r; g.K1 = n; g.K2 = 0;
  g.nch1 = g.nch = cdiv(n, kKC);
  g.A1 = Xb; g.lda1 = n;
  g.B1 = static_cast<const uint16_t*>(A->Vt); g.ldb1 = n;
  g.C = Tt; g.ldc = ldt; g.out_mode = OUT_BF16;
  g.vec_a1 = aligned16(Xb, n) && n % 8 == 0;
  g.vec_b1 = aligned16(g.B1, n) && n % 8 == 0;
  run_gemm(g, A_DENSE, part, s);
}

// A general bf16 GEMM on the matrix cores: C[n * ldc + m] = sum_k A[m][k]
// B[n][k] for m < M, n < N, k < K (A: M rows, B: N rows, both K-contiguous
// with strides lda, ldb), fp32 accumulation, stored as bf16 (RNE) or fp32.
// `part` holds at least gemm_bf16_part_bytes(M, N, K, ldc) bytes.
void launch_gemm_bf16(int M, int N, int K, const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, void* C,
                      int64_t ldc, bool out_bf16, float* part, hipStream_t s) {
  GemmArgs g = {};
  g.M = M; g.N = N; g.K1 = K; g.K2 = 0;
  g.nch1 = g.nch = cdiv(K, kKC);
  g.A1 = A; g.lda1 = lda;
  g.B1 = B; g.ldb1 = ldb;
  g.C = C; g.ldc = ldc; g.out_mode = out_bf16 ? OUT_BF16 : OUT_F32;
  g.vec_a1 = aligned16(A, lda) && K % 8 == 0;
  g.vec_b1 = aligned16(B, ldb) && K % 8 == 0;
  run_gemm(g, A_DENSE, part, s);
}

size_t gemm_bf16_part_bytes(int M, int N, int K, int64_t ldc) { return gemm_part_bytes(M, N, K, 0) / M * ldc; }

// Partials are laid out with the output's row stride ldt (>= b).
size_t tt_gemm_part_bytes(const hss_matrix* A, int b, int ldt) {
  return A->r > 0 ? gemm_part_bytes(b, A->r, A->n, 0) / b * ldt : 0;
}

hss_status launch_mfma(const hss_matrix* A, int b, const void* X, void* Y, void* ws, hipStream_t s) {
  const MfmaPlan p = plan_mfma(A, b);
  char* base = static_cast<char*>(ws);
  uint16_t* Tb = reinterpret_cast<uint16_t*>(base + p.tb_off);
  uint16_t* Sd = reinterpret_cast<uint16_t*>(base + p.dense_off);
  float* part = reinterpret_cast<float*>(base + p.part_off);
  const int m = A->m, n = A->n, r = A->r;
  const uint16_t* Xb = static_cast<const uint16_t*>(X);
  const bool csr = A->fmt == HSS_FMT_CSR;
  const bool s_empty = csr_empty(A);  // segment 1 has no work

  if (csr && !s_empty) {
    const dim3 grid((unsigned)cdiv(m, 4));
    const uint16_t* vals = static_cast<const uint16_t*>(A->values);
    if (A->flags & HSS_COL16)
      hipLaunchKernelGGL(k_csr_densify<uint16_t>, grid, dim3(256), 0, s, A->row_ptr,
                         reinterpret_cast<const uint16_t*>(A->col_idx), vals, m, n, Sd);
    else
      hipLaunchKernelGGL(k_csr_densify<int32_t>, grid, dim3(256), 0, s, A->row_ptr, A->col_idx, vals, m, n, Sd);
  }
  // T^T (b x r) = X . Vt^T
  if (r > 0) launch_t_gemm(A, b, X, Tb, part, s);
  // Y (b x m) = [X | T^T] . [S | U]^T
  GemmArgs g = {};
  g.M = m; g.N = b; g.K1 = s_empty ? 0 : n; g.K2 = r;
  g.nch1 = cdiv(g.K1, kKC);
  g.nch = g.nch1 + (r > 0 ? cdiv(r, kKC) : 0);
  g.B1 = Xb; g.ldb1 = n;
  g.vec_b1 = aligned16(Xb, n) && n % 8 == 0;
  int amode = A_DENSE;
  if (!csr) {
    amode = A_NM24;
    g.nmv = static_cast<const uint16_t*>(A->nm_values);
    g.meta = A->nm_meta;
  } else {
    g.A1 = Sd; g.lda1 = n;
    g.vec_a1 = aligned16(Sd, n) && n % 8 == 0;
  }
  if (r > 0) {
    g.A2 = static_cast<const uint16_t*>(A->U); g.lda2 = r;
    g.B2 = Tb; g.ldb2 = r;
    g.vec_a2 = aligned16(g.A2, r) && r % 8 == 0;
    g.vec_b2 = aligned16(Tb, r) && r % 8 == 0;
  }
  g.C = Y; g.ldc = m; g.out_mode = OUT_BF16;
  run_gemm(g, amode, part, s);
  return hipGetLastError() == hipSuccess ? HSS_OK : HSS_ERR_HIP;
}

}  // namespace hss
