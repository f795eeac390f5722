// Stage 1 of HSS: magnitude top-k of W into CSR or 2:4, plus the +0 residual.
//
// [HSS] page "LLMの階層的スパース+低ランク圧縮", section "2段階階層的スパース+低ランク
// 圧縮": S keeps the weights of largest absolute magnitude (the worked example
// keeps the top 5 % of a 1024 x 1024 matrix, stored as indices + values);
// the remaining entries form the dense residual.
// [HASSLE] page aibr.jp/archives/82335, section "3.中核となる技術的要素": N:M
// structured sparsity (2 of every 4) as the GPU-friendly form.
//
// CSR pipeline (all on the device, no host round trip; k is known up front,
// so the caller sizes col_idx/values before the call):
//   init     zero the control words and the histogram
//   hist/pick, once per 8-bit digit of key = |w| bits, most significant first:
//            per-block LDS histograms of the digit among keys whose higher
//            digits equal the prefix chosen so far, merged with integer
//            atomics; one small block then walks the histogram from the top
//            to find the digit holding the k-th largest key.  After the last
//            digit: threshold key T, c_gt = #{key > T}, need = k - c_gt.
//   rowcount one wave per row: gt_i = #{key > T}, eq_i = #{key == T}
//   scan     one block: exclusive scan of eq_i gives each row's rank among the
//            ties; row i takes take_i = clamp(need - eqprefix_i, 0, eq_i) ties
//            (lowest linear index first); scan of gt_i + take_i -> row_ptr
//   scatter  one wave per row: per-lane keep flags, wave prefix sums of tie
//            and keep counts -> ascending col_idx / bit-copied values, and the
//            residual with kept positions set to +0.
#include "hss_internal.h"

namespace hss {

// Control-word layout of the split workspace (uint32 words).
enum : int {
  W_ERR = 0,     // nonzero: a non-finite weight was seen
  W_REM = 1,     // keys still to place at or below the current prefix
  W_PREFIX = 2,  // high digits of the threshold chosen so far
  W_T = 3,       // threshold key
  W_CGT = 4,     // #{key > T}
  W_NEED = 5,    // ties at T to keep
  W_HIST = 64,   // 256 bins
  W_ROWS = 320   // gt[m] then eq/take[m]
};

size_t split_ws_bytes(int fmt, int m) {
  if (fmt == HSS_FMT_2OF4) return 256;
  return sizeof(uint32_t) * ((size_t)W_ROWS + 2 * (size_t)m);
}

template <int DT> struct VecLoad;  // 16-byte vectors of keys
template <> struct VecLoad<HSS_F32> {
  static constexpr int N = 4;
  __device__ __forceinline__ static void unpack(const u32x4& v, uint32_t (&o)[4]) {
    o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
  }
};
template <> struct VecLoad<HSS_BF16> {
  static constexpr int N = 8;
  __device__ __forceinline__ static void unpack(const u32x4& v, uint32_t (&o)[8]) {
    o[0] = v.x & 0xffffu; o[1] = v.x >> 16; o[2] = v.y & 0xffffu; o[3] = v.y >> 16;
    o[4] = v.z & 0xffffu; o[5] = v.z >> 16; o[6] = v.w & 0xffffu; o[7] = v.w >> 16;
  }
};

__global__ void k_split_init(uint32_t* ws, int64_t k) {
  const int t = threadIdx.x;
  if (t == 0) {
    ws[W_ERR] = 0;
    ws[W_REM] = (uint32_t)k;
    ws[W_PREFIX] = 0;
    ws[W_T] = (k == 0) ? 0xffffffffu : 0u;  // k == 0: no key exceeds T, none equal
    ws[W_CGT] = 0;
    ws[W_NEED] = 0;
  }
  for (int i = t; i < 256; i += blockDim.x) ws[W_HIST + i] = 0;
}

// Histogram of digit (key >> shift) & 255 over keys whose bits above
// shift+8 equal the prefix.  VEC: use 16-byte loads (W 16-byte aligned).
// Trained (and synthetic heavy-tailed) weights put almost every key of the
// top digit -- essentially the exponent -- into one or two bins, so a single
// LDS histogram would serialise whole waves on one address: lane l counts
// into copy l % 32 instead (copies 257 words apart, so the copies of a bin
// sit in different banks), and the copies are summed at the end.
static constexpr int kHistCopies = 32, kHistStride = 257;

template <int DT, bool VEC>
__global__ __launch_bounds__(256) void k_split_hist(const typename Elem<DT>::bits_t* __restrict__ W,
                                                    int64_t count, uint32_t* __restrict__ ws,
                                                    int shift, int first) {
  using E = Elem<DT>;
  __shared__ uint32_t h[kHistCopies * kHistStride];
  // k == 0 (uniform across the grid): nothing to count, but the first pass
  // still reads every key for the non-finite check
  const bool counting = ws[W_REM] != 0;
  if (!counting && !first) return;
  const uint32_t prefix = ws[W_PREFIX];
  const int hs = shift + 8;
  for (int i = threadIdx.x; i < kHistCopies * kHistStride; i += 256) h[i] = 0;
  __syncthreads();
  uint32_t* hc = h + (lane_id() & (kHistCopies - 1)) * kHistStride;
  bool bad = false;
  auto visit = [&](uint32_t bits) {
    const uint32_t key = bits & E::key_mask;
    bad |= first && key >= E::key_inf;
    const uint32_t hi = hs >= 32 ? 0u : (key >> hs);
    if (counting && hi == prefix) atomicAdd(&hc[(key >> shift) & 255u], 1u);
  };
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  if (VEC) {
    constexpr int NV = VecLoad<DT>::N;
    constexpr int U = 4;  // vectors in flight per thread
    const int64_t nvec = count / NV;
    const u32x4* W4 = reinterpret_cast<const u32x4*>(W);
    for (int64_t v0 = tid; v0 < nvec; v0 += U * stride) {
      u32x4 raw[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t v = v0 + u * stride;
        raw[u] = __builtin_nontemporal_load(W4 + (v < nvec ? v : v0));
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (v0 + u * stride < nvec) {
          uint32_t e[NV];
          VecLoad<DT>::unpack(raw[u], e);
#pragma unroll
          for (int q = 0; q < NV; ++q) visit(e[q]);
        }
      }
    }
    for (int64_t i = nvec * NV + tid; i < count; i += stride) visit(W[i]);
  } else {
    for (int64_t i = tid; i < count; i += stride) visit(W[i]);
  }
  if (bad) atomicOr(&ws[W_ERR], 1u);
  __syncthreads();
  uint32_t c = 0;
  for (int k = 0; k < kHistCopies; ++k) c += h[k * kHistStride + threadIdx.x];
  if (c) atomicAdd(&ws[W_HIST + threadIdx.x], c);
}

// Fix the digit of the k-th largest key: the largest digit d whose suffix
// count S(d) = sum of bins >= d reaches the remaining rank (digit 0 if none
// does).  Thread t holds bin 255 - t; an inclusive scan over t gives S(255 - t)
// and the first thread whose scan reaches the rank (or the last thread) owns
// the digit; keys above it: S(d + 1).  One block of 256 threads.
__global__ __launch_bounds__(256) void k_split_pick(uint32_t* __restrict__ ws, int last) {
  __shared__ uint32_t wsum[4];
  const int t = threadIdx.x, lane = lane_id(), w = t >> 6;
  const uint32_t rem = ws[W_REM];
  if (rem == 0) return;  // k == 0
  const uint32_t v = ws[W_HIST + 255 - t];
  ws[W_HIST + 255 - t] = 0;  // ready for the next digit
  const uint32_t ex = wave_excl_scan_u32(v);
  if (lane == HSS_WAVE - 1) wsum[w] = ex + v;
  __syncthreads();
  uint32_t base = 0;
  for (int k = 0; k < w; ++k) base += wsum[k];
  const uint32_t incl = base + ex + v;
  const bool reach = incl >= rem || t == 255;
  const bool prev = t > 0 && (incl - v >= rem);  // an earlier thread reached it already
  if (reach && !prev) {
    const int d = 255 - t;
    const uint32_t above = incl - v;
    const uint32_t prefix = (ws[W_PREFIX] << 8) | (uint32_t)d;
    ws[W_PREFIX] = prefix;
    ws[W_CGT] += above;
    ws[W_REM] = rem - above;
    if (last) {
      ws[W_T] = prefix;
      ws[W_NEED] = rem - above;
    }
  }
}

// Per row: gt_i = #{key > T}, eq_i = #{key == T}.  One wave per row.
template <int DT, bool VEC>
__global__ __launch_bounds__(256) void k_split_rowcount(const typename Elem<DT>::bits_t* __restrict__ W,
                                                        int m, int n, uint32_t* __restrict__ ws) {
  using E = Elem<DT>;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= m) return;
  const int lane = lane_id();
  const uint32_t T = ws[W_T];
  uint32_t gt = 0, eq = 0;
  const typename E::bits_t* Wr = W + (int64_t)row * n;
  auto visit = [&](uint32_t bits) {
    const uint32_t key = bits & E::key_mask;
    gt += key > T;
    eq += key == T;
  };
  if (VEC) {
    constexpr int NV = VecLoad<DT>::N;
    constexpr int U = 4;  // vectors in flight per lane
    const int nvec = n / NV;
    const u32x4* W4 = reinterpret_cast<const u32x4*>(Wr);
    for (int v0 = lane; v0 < nvec; v0 += U * HSS_WAVE) {
      u32x4 raw[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int v = v0 + u * HSS_WAVE;
        raw[u] = __builtin_nontemporal_load(W4 + (v < nvec ? v : v0));
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (v0 + u * HSS_WAVE < nvec) {
          uint32_t e[NV];
          VecLoad<DT>::unpack(raw[u], e);
#pragma unroll
          for (int q = 0; q < NV; ++q) visit(e[q]);
        }
      }
    }
  } else {
    for (int j = lane; j < n; j += HSS_WAVE) visit(Wr[j]);
  }
  gt = wave_sum_u32(gt);
  eq = wave_sum_u32(eq);
  if (lane == 0) {
    ws[W_ROWS + row] = gt;
    ws[W_ROWS + m + row] = eq;
  }
}

// Block-wide exclusive scan of one value per thread (1024 threads).
__device__ uint32_t block_excl_scan_1024(uint32_t v, uint32_t* sh, uint32_t* total) {
  const int t = threadIdx.x;
  const int lane = lane_id(), w = t >> 6;
  const uint32_t ex = wave_excl_scan_u32(v);
  if (lane == HSS_WAVE - 1) sh[w] = ex + v;
  __syncthreads();
  if (w == 0) {
    const uint32_t s = lane < 16 ? sh[lane] : 0u;
    const uint32_t se = wave_excl_scan_u32(s);
    if (lane < 16) sh[16 + lane] = se;
    if (lane == 15) sh[32] = se + s;
  }
  __syncthreads();
  const uint32_t r = sh[16 + w] + ex;
  *total = sh[32];
  __syncthreads();
  return r;
}

// Tie split and row pointers.  One block of 1024 threads; thread t owns a
// contiguous run of rows.  Rewrites gt[i] <- gt_i + take_i, eq[i] <- take_i.
__global__ __launch_bounds__(1024) void k_split_scan(uint32_t* __restrict__ ws, int m,
                                                     int32_t* __restrict__ row_ptr) {
  __shared__ uint32_t sh[64];
  const int t = threadIdx.x;
  const int per = (m + 1023) / 1024;
  const int r0 = min(m, t * per), r1 = min(m, r0 + per);
  uint32_t* gt = ws + W_ROWS;
  uint32_t* eq = ws + W_ROWS + m;
  const int64_t need = ws[W_NEED];
  uint32_t total;
  // Pass 1: rank of each row's first tie among all ties (row-major order).
  uint32_t s = 0;
  for (int i = r0; i < r1; ++i) s += eq[i];
  uint32_t pre = block_excl_scan_1024(s, sh, &total);
  uint32_t cnt_local = 0;
  for (int i = r0; i < r1; ++i) {
    const uint32_t e = eq[i];
    int64_t take = need - (int64_t)pre;
    take = take < 0 ? 0 : (take > (int64_t)e ? (int64_t)e : take);
    pre += e;
    eq[i] = (uint32_t)take;
    gt[i] += (uint32_t)take;
    cnt_local += gt[i];
  }
  // Pass 2: row pointers.
  uint32_t base = block_excl_scan_1024(cnt_local, sh, &total);
  for (int i = r0; i < r1; ++i) {
    row_ptr[i] = (int32_t)base;
    base += gt[i];
  }
  if (t == 0) row_ptr[m] = (int32_t)total;
}

// Compaction: one wave per row.  Lane l of a step holds NV consecutive
// columns; within a row, tie ranks and output slots follow column order.
template <int DT, bool VEC>
__global__ __launch_bounds__(256) void k_split_scatter(
    const typename Elem<DT>::bits_t* __restrict__ W, int m, int n, const uint32_t* __restrict__ ws,
    const int32_t* __restrict__ row_ptr, int32_t* __restrict__ col_idx,
    typename Elem<DT>::bits_t* __restrict__ values, typename Elem<DT>::bits_t* __restrict__ residual) {
  using E = Elem<DT>;
  using bits_t = typename E::bits_t;
  constexpr int NV = VEC ? VecLoad<DT>::N : 1;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= m) return;
  const int lane = lane_id();
  const uint32_t T = ws[W_T];
  const uint32_t take = ws[W_ROWS + m + row];
  const int32_t out0 = row_ptr[row];
  const bits_t* Wr = W + (int64_t)row * n;
  bits_t* Rr = residual ? residual + (int64_t)row * n : nullptr;
  uint32_t eq_seen = 0, kept = 0;
  for (int j0 = 0; j0 < n; j0 += NV * HSS_WAVE) {
    const int jl = j0 + lane * NV;
    uint32_t e[NV];
    if constexpr (VEC) {
      if (jl < n) {
        VecLoad<DT>::unpack(__builtin_nontemporal_load(reinterpret_cast<const u32x4*>(Wr + jl)), e);
      } else {
#pragma unroll
        for (int q = 0; q < NV; ++q) e[q] = 0;
      }
    } else {
      e[0] = jl < n ? (uint32_t)Wr[jl] : 0u;
    }
    uint32_t gtm = 0, eqm = 0;  // per-lane bit masks over the NV elements
#pragma unroll
    for (int q = 0; q < NV; ++q) {
      const uint32_t key = e[q] & E::key_mask;
      const bool valid = jl + q < n;
      gtm |= (uint32_t)(valid && key > T) << q;
      eqm |= (uint32_t)(valid && key == T) << q;
    }
    const uint32_t neq = __popc(eqm);
    const uint32_t eq_before = eq_seen + wave_excl_scan_u32(neq);
    // keep flags: all gt, plus ties whose row rank is below take
    uint32_t keepm = gtm;
    uint32_t r = eq_before;
#pragma unroll
    for (int q = 0; q < NV; ++q) {
      if (eqm >> q & 1u) {
        if (r < take) keepm |= 1u << q;
        ++r;
      }
    }
    const uint32_t nkeep = __popc(keepm);
    uint32_t pos = (uint32_t)out0 + kept + wave_excl_scan_u32(nkeep);
#pragma unroll
    for (int q = 0; q < NV; ++q) {
      if (keepm >> q & 1u) {
        col_idx[pos] = jl + q;
        values[pos] = (bits_t)e[q];
        ++pos;
      }
    }
    if (Rr) {
      if constexpr (VEC) {
        if (jl < n) {
          uint32_t o[NV];
#pragma unroll
          for (int q = 0; q < NV; ++q) o[q] = (keepm >> q & 1u) ? 0u : e[q];
          u32x4 v;
          if constexpr (DT == HSS_F32) {
            v.x = o[0]; v.y = o[1]; v.z = o[2]; v.w = o[3];
          } else {
            v.x = o[0] | (o[1] << 16); v.y = o[2] | (o[3] << 16);
            v.z = o[4] | (o[5] << 16); v.w = o[6] | (o[7] << 16);
          }
          __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(Rr + jl));
        }
      } else if (jl < n) {
        Rr[jl] = (keepm & 1u) ? (bits_t)0 : (bits_t)e[0];
      }
    }
    eq_seen += wave_sum_u32(neq);
    kept += wave_sum_u32(nkeep);
  }
}

// 2:4: one thread per 32 columns (one metadata word) of one row.
template <int DT>
__global__ __launch_bounds__(256) void k_split_24(const typename Elem<DT>::bits_t* __restrict__ W,
                                                  int m, int n,
                                                  typename Elem<DT>::bits_t* __restrict__ nmv,
                                                  uint32_t* __restrict__ meta,
                                                  typename Elem<DT>::bits_t* __restrict__ residual,
                                                  uint32_t* __restrict__ ws) {
  using E = Elem<DT>;
  using bits_t = typename E::bits_t;
  const int words = (n + 31) >> 5;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)m * words) return;
  const int row = (int)(gid / words);
  const int w = (int)(gid - (int64_t)row * words);
  const int c0 = w * 32;
  const int ng = min(8, (n - c0) >> 2);
  const bits_t* Wr = W + (int64_t)row * n + c0;
  bits_t* Vr = nmv + (int64_t)row * (n >> 1) + (c0 >> 1);
  bits_t* Rr = residual ? residual + (int64_t)row * n + c0 : nullptr;
  uint32_t word = 0;
  bool bad = false;
  for (int g = 0; g < ng; ++g) {
    uint32_t b[4], key[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      b[q] = Wr[4 * g + q];
      key[q] = b[q] & E::key_mask;
      bad |= key[q] >= E::key_inf;
    }
    // rank of q = entries ordered before it by (key desc, column asc); keep rank < 2
    uint32_t keepm = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      int rank = 0;
#pragma unroll
      for (int p = 0; p < 4; ++p)
        rank += (p != q) && (key[p] > key[q] || (key[p] == key[q] && p < q));
      keepm |= (uint32_t)(rank < 2) << q;
    }
    const int i0 = __ffs(keepm) - 1;
    const int i1 = 31 - __clz(keepm);
    word |= (uint32_t)(i0 | (i1 << 2)) << (4 * g);
    Vr[2 * g] = (bits_t)b[i0];
    Vr[2 * g + 1] = (bits_t)b[i1];
    if (Rr) {
#pragma unroll
      for (int q = 0; q < 4; ++q) Rr[4 * g + q] = (keepm >> q & 1u) ? (bits_t)0 : (bits_t)b[q];
    }
  }
  meta[(int64_t)row * words + w] = word;
  if (bad) atomicOr(&ws[W_ERR], 1u);
}

// The same selection with 16-byte loads and stores: one thread per 32
// columns of one row, the 64 (bf16) or 128 (fp32) bytes of W read as whole
// vectors, the 16 kept values and the residual written as whole vectors.
// Needs n % 32 == 0 and W, nm_values and residual 16-byte aligned.
template <int DT>
__global__ __launch_bounds__(256) void k_split_24v(const typename Elem<DT>::bits_t* __restrict__ W,
                                                   int m, int n,
                                                   typename Elem<DT>::bits_t* __restrict__ nmv,
                                                   uint32_t* __restrict__ meta,
                                                   typename Elem<DT>::bits_t* __restrict__ residual,
                                                   uint32_t* __restrict__ ws) {
  using E = Elem<DT>;
  using bits_t = typename E::bits_t;
  constexpr int PW = 4 / (int)sizeof(bits_t);  // values per 32-bit word
  constexpr int NW = 32 / PW;                   // words per 32 columns
  const int words = n >> 5;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)m * words) return;
  const int row = (int)(gid / words);
  const int w = (int)(gid - (int64_t)row * words);
  const int c0 = w * 32;
  uint32_t win[NW];
  const u32x4* src = reinterpret_cast<const u32x4*>(W + (int64_t)row * n + c0);
#pragma unroll
  for (int v = 0; v < NW / 4; ++v) {
    const u32x4 q = src[v];
    win[4 * v] = q.x; win[4 * v + 1] = q.y; win[4 * v + 2] = q.z; win[4 * v + 3] = q.w;
  }
  auto val = [&](int k) -> uint32_t {
    if constexpr (PW == 2) return (win[k >> 1] >> (16 * (k & 1))) & 0xffffu;
    else return win[k];
  };
  uint32_t kept[16], res[32];
  uint32_t word = 0;
  bool bad = false;
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    uint32_t b[4], key[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      b[q] = val(4 * g + q);
      key[q] = b[q] & E::key_mask;
      bad |= key[q] >= E::key_inf;
    }
    uint32_t keepm = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      int rank = 0;
#pragma unroll
      for (int p = 0; p < 4; ++p)
        rank += (p != q) && (key[p] > key[q] || (key[p] == key[q] && p < q));
      keepm |= (uint32_t)(rank < 2) << q;
    }
    const int i0 = __ffs(keepm) - 1;
    const int i1 = 31 - __clz(keepm);
    word |= (uint32_t)(i0 | (i1 << 2)) << (4 * g);
    kept[2 * g] = b[i0];
    kept[2 * g + 1] = b[i1];
#pragma unroll
    for (int q = 0; q < 4; ++q) res[4 * g + q] = (keepm >> q & 1u) ? 0u : b[q];
  }
  auto pack = [&](const uint32_t* v, int j) -> uint32_t {  // 32-bit word j of a value list
    if constexpr (PW == 2) return v[2 * j] | (v[2 * j + 1] << 16);
    else return v[j];
  };
  u32x4* dv = reinterpret_cast<u32x4*>(nmv + (int64_t)row * (n >> 1) + (c0 >> 1));
#pragma unroll
  for (int v = 0; v < NW / 8; ++v)
    dv[v] = u32x4{pack(kept, 4 * v), pack(kept, 4 * v + 1), pack(kept, 4 * v + 2), pack(kept, 4 * v + 3)};
  if (residual) {
    u32x4* dr = reinterpret_cast<u32x4*>(residual + (int64_t)row * n + c0);
#pragma unroll
    for (int v = 0; v < NW / 4; ++v)
      dr[v] = u32x4{pack(res, 4 * v), pack(res, 4 * v + 1), pack(res, 4 * v + 2), pack(res, 4 * v + 3)};
  }
  meta[(int64_t)row * words + w] = word;
  if (bad) atomicOr(&ws[W_ERR], 1u);
}

__global__ void k_zero_err(uint32_t* ws) { ws[W_ERR] = 0; }

static inline unsigned grid_for(int64_t work, int per_block, unsigned cap) {
  int64_t g = (work + per_block - 1) / per_block;
  if (g < 1) g = 1;
  return (unsigned)(g > cap ? cap : g);
}

template <int DT>
static hss_status split_csr_t(int m, int n, const void* Wv, int64_t k, int32_t* row_ptr,
                              int32_t* col_idx, void* values, void* residual, void* wsv,
                              hipStream_t s) {
  using bits_t = typename Elem<DT>::bits_t;
  const bits_t* W = static_cast<const bits_t*>(Wv);
  uint32_t* ws = static_cast<uint32_t*>(wsv);
  const int64_t count = (int64_t)m * n;
  const bool vec_all = ((uintptr_t)W % 16) == 0;
  const bool vec_rows = vec_all && ((size_t)n * sizeof(bits_t)) % 16 == 0 &&
                        (residual == nullptr || ((uintptr_t)residual % 16) == 0);
  hipLaunchKernelGGL(k_split_init, dim3(1), dim3(256), 0, s, ws, k);
  // Digits of the key, most significant first: f32 keys have 31 bits
  // (shifts 24, 16, 8, 0), bf16 keys 15 bits (shifts 8, 0).
  const int top = Elem<DT>::key_bits > 16 ? 24 : 8;
  // ~16 vectors per thread: enough work to amortise the 32-copy histogram per block
  const unsigned hgrid = grid_for(count, 256 * 16 * VecLoad<DT>::N, 512);
  for (int shift = top; shift >= 0; shift -= 8) {
    if (vec_all)
      hipLaunchKernelGGL((k_split_hist<DT, true>), dim3(hgrid), dim3(256), 0, s, W, count, ws, shift,
                         shift == top);
    else
      hipLaunchKernelGGL((k_split_hist<DT, false>), dim3(hgrid), dim3(256), 0, s, W, count, ws, shift,
                         shift == top);
    hipLaunchKernelGGL(k_split_pick, dim3(1), dim3(256), 0, s, ws, shift == 0);
  }
  const unsigned rgrid = (unsigned)((m + 3) / 4);
  if (vec_rows)
    hipLaunchKernelGGL((k_split_rowcount<DT, true>), dim3(rgrid), dim3(256), 0, s, W, m, n, ws);
  else
    hipLaunchKernelGGL((k_split_rowcount<DT, false>), dim3(rgrid), dim3(256), 0, s, W, m, n, ws);
  hipLaunchKernelGGL(k_split_scan, dim3(1), dim3(1024), 0, s, ws, m, row_ptr);
  if (vec_rows)
    hipLaunchKernelGGL((k_split_scatter<DT, true>), dim3(rgrid), dim3(256), 0, s, W, m, n, ws, row_ptr,
                       col_idx, static_cast<bits_t*>(values), static_cast<bits_t*>(residual));
  else
    hipLaunchKernelGGL((k_split_scatter<DT, false>), dim3(rgrid), dim3(256), 0, s, W, m, n, ws, row_ptr,
                       col_idx, static_cast<bits_t*>(values), static_cast<bits_t*>(residual));
  return hipGetLastError() == hipSuccess ? HSS_OK : HSS_ERR_HIP;
}

// 16-bit copy of CSR columns (every column < 65536 by the caller's check).
__global__ __launch_bounds__(256) void k_cols_to_u16(const int32_t* __restrict__ col, int64_t nnz,
                                                     uint16_t* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < nnz; i += stride) out[i] = (uint16_t)col[i];
}

hss_status launch_cols_to_u16(const int32_t* col_idx, int64_t nnz, uint16_t* out, hipStream_t stream) {
  hipLaunchKernelGGL(k_cols_to_u16, dim3(grid_for(nnz, 256 * 4, 4096)), dim3(256), 0, stream, col_idx, nnz, out);
  return hipGetLastError() == hipSuccess ? HSS_OK : HSS_ERR_HIP;
}

hss_status launch_split_csr(int dt, int m, int n, const void* W, int64_t k, int32_t* row_ptr,
                            int32_t* col_idx, void* values, void* residual, void* ws,
                            hipStream_t stream) {
  if (dt == HSS_F32)
    return split_csr_t<HSS_F32>(m, n, W, k, row_ptr, col_idx, values, residual, ws, stream);
  return split_csr_t<HSS_BF16>(m, n, W, k, row_ptr, col_idx, values, residual, ws, stream);
}

hss_status launch_split_24(int dt, int m, int n, const void* W, void* nm_values, uint32_t* nm_meta,
                           void* residual, void* wsv, hipStream_t s) {
  uint32_t* ws = static_cast<uint32_t*>(wsv);
  const int64_t threads = (int64_t)m * ((n + 31) / 32);
  const unsigned grid = (unsigned)((threads + 255) / 256);
  hipLaunchKernelGGL(k_zero_err, dim3(1), dim3(1), 0, s, ws);
  const bool vec = n % 32 == 0 && (uintptr_t)W % 16 == 0 && (uintptr_t)nm_values % 16 == 0 &&
                   (uintptr_t)residual % 16 == 0;
  if (vec) {
    if (dt == HSS_F32)
      hipLaunchKernelGGL((k_split_24v<HSS_F32>), dim3(grid), dim3(256), 0, s,
                         static_cast<const uint32_t*>(W), m, n, static_cast<uint32_t*>(nm_values),
                         nm_meta, static_cast<uint32_t*>(residual), ws);
    else
      hipLaunchKernelGGL((k_split_24v<HSS_BF16>), dim3(grid), dim3(256), 0, s,
                         static_cast<const uint16_t*>(W), m, n, static_cast<uint16_t*>(nm_values),
                         nm_meta, static_cast<uint16_t*>(residual), ws);
  } else if (dt == HSS_F32)
    hipLaunchKernelGGL((k_split_24<HSS_F32>), dim3(grid), dim3(256), 0, s,
                       static_cast<const uint32_t*>(W), m, n, static_cast<uint32_t*>(nm_values),
                       nm_meta, static_cast<uint32_t*>(residual), ws);
  else
    hipLaunchKernelGGL((k_split_24<HSS_BF16>), dim3(grid), dim3(256), 0, s,
                       static_cast<const uint16_t*>(W), m, n, static_cast<uint16_t*>(nm_values),
                       nm_meta, static_cast<uint16_t*>(residual), ws);
  return hipGetLastError() == hipSuccess ? HSS_OK : HSS_ERR_HIP;
}

}  // namespace hss
