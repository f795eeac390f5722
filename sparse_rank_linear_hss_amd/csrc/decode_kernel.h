// Fused small-batch apply (bc <= 8 columns per launch): one kernel computes
//   Y[c][i] = sum_{j in S_i} S_ij X[c][j] + sum_l U[i][l] T[c][l],
//   T[c][l] = sum_j Vt[l][j] X[c][j].
//
// [HSS] page "LLMの階層的スパース+低ランク圧縮", section "実装と運用パターン": the
// compressed forward pass is one sparse product plus two small dense products.
// At decode batch sizes every byte of S, U and V^T is read once and the step
// is bound by HBM bandwidth (SqueezeLLM explainer page aibr.jp/archives/208940,
// section "1.概要と位置づけ": single-batch inference is memory-bandwidth bound),
// so one launch keeps all three streams in flight instead of serialising T
// before the row pass.
//
// Latency, not bandwidth, limits a decode call of a few MB, so the kernel is
// written around dependent round trips to memory:
//   * every load that does not depend on another is issued at kernel start,
//     from a clamped (always valid) address with the value masked afterwards
//     -- a load under a lane-divergent `if` makes the compiler wait for it at
//     the join, which would serialise the prefetches;
//   * the only chains are row_ptr -> (col_idx, values) for CSR rows and
//     (Vt, X) -> T -> readers for the low-rank term.
//
// Cross-block hand-off of T (a launch costs ~2.5 us and a same-address device
// atomic ~10 ns once every block hits it, so no hot counters and no
// cache-wide acquire fences):
//   * T row l is produced at the start of the launch by producer block l (the
//     lowest block ids, dispatched first) or, for one CSR column, by a row
//     block that also produces it (merged producers), and published into 8
//     replicas as 64-bit words (fp32 value, call tag) with coherent
//     (agent-scope) stores -- there is no done counter for T;
//   * every block reads the tagged words with coherent loads after its own
//     sparse work, polls a stale word a bounded number of times, then computes
//     any row still missing itself (same arithmetic, so the same bits).  No
//     wait can hang and a stale value is never used;
//   * the call tag is epoch+1, the epoch being read by every block at its
//     start.  Each block then bumps one of 64 spread arrival counters of the
//     set of the epoch's parity; the last block to arrive (two-level count)
//     stores the next epoch, and block 0 clears the other set for the next
//     call.  All blocks have read the epoch before it can advance.

#pragma once

#include "hss_internal.h"

namespace hss {

// Control region (uint32 words) at the start of the apply workspace: the
// call epoch, then two sets of arrival counters (a top counter and 64 spread
// counters each); a call counts on set (epoch & 1).  Each word sits on its
// own 128-byte line.
static constexpr int kCtlEpoch = 0;
static constexpr int kCtlLine = 32;                  // words per line
static constexpr int kNumSub = 64;  // a power of two (arrive_check divides by it with a shift)
static constexpr int kCtlSetWords = (1 + kNumSub) * kCtlLine;
static constexpr size_t kCtlBytes = 32768;          // >= (1 + 2 * 65) lines
__device__ __forceinline__ int ctl_top(uint32_t epoch) { return kCtlLine + (int)(epoch & 1u) * kCtlSetWords; }
__device__ __forceinline__ int ctl_sub(uint32_t epoch, int k) { return ctl_top(epoch) + kCtlLine * (1 + k); }
// Copies of the tagged T words; block b reads copy b % kTReplicas, so each
// line is polled by 1/kTReplicas of the blocks.
static constexpr int kTReplicas = 8;

struct DecodeArgs {
  int m, n, r, bc;
  const int32_t* row_ptr;
  const int32_t* col_idx;  // 32-bit columns, or
  const uint16_t* col16;   // 16-bit columns (FMT == kFmtCsr16)
  const void* vals;
  const void* nmv;
  const uint32_t* meta;
  const void* U;
  const void* Vt;
  const void* X;
  void* Y;
  uint64_t* Tt;   // tagged T words: T[c * r + l] = value bits | tag << 32, per replica
  int64_t t_stride;  // words between replicas
  uint32_t* ctl;  // control region
  int64_t nnz;    // CSR entries
  int x_lds;      // X staged in LDS
  int x_pad;      // staged X padded (16 bytes after every 64), for the 2:4 fast path
  int vec;        // X, Vt rows 16-byte aligned: vector dot products
  int vec_csr;    // CSR chunks: col_idx 16-byte, values 4*elem aligned, nnz >= 4
  int nm_fast;    // bf16 2:4 with n % 32 == 0 and aligned rows: vector words
  int spin;       // polls of a stale T word before computing it locally
  int t_off, miss_off, x_off;  // dynamic LDS layout (bytes)
  int mtab_off;                // bf16 U pieces: the 256-entry mask table (4 KiB)
  // Block structure of the low-rank term (a flat matrix: ru = r, v_ld = n,
  // h_m0 = m, h_toff = 0, h_n0 = n, h_l1 = h_l2 = h_l3 = r).  U rows hold ru
  // values (row stride ru); rows i >= h_m0 take them against T[h_toff ..
  // h_toff + ru).  T row l dots V^T row l (row stride v_ld) with X columns
  // [0, h_n0), or [h_n0, n) when h_l1 <= l < h_l2 or l >= h_l3.
  int ru, v_ld, h_m0, h_toff, h_n0, h_l1, h_l2, h_l3;
};

// First X column and column count of T row l.
__device__ __forceinline__ void t_cols(const DecodeArgs& a, int l, int& c0, int& len) {
  const bool hi = (l >= a.h_l1 && l < a.h_l2) || l >= a.h_l3;
  c0 = hi ? a.h_n0 : 0;
  len = hi ? a.n - a.h_n0 : a.h_n0;
}

// Several matrices that share X in one launch (at most kMaxGroup): the grid is
// the producer blocks of every matrix, then the row blocks of every matrix.
// One launch, so one epoch and one arrival count; each matrix has its own T
// words.
static constexpr int kMaxGroup = HSS_MAX_GROUP;
struct GroupArgs {
  DecodeArgs a[kMaxGroup];
  int G;
  int prod_start[kMaxGroup + 1];  // producer blocks of matrix g: [prod_start[g], prod_start[g + 1])
  int prod_rows;                   // T rows per producer block: 1, or one per wave (wave producers)
  int row_start[kMaxGroup + 1];   // row blocks of matrix g (after all producers)
};

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Kernel format: HSS_FMT_CSR (32-bit columns), HSS_FMT_2OF4, or CSR with
// 16-bit columns (n <= 65536: 4 instead of 6 bytes per bf16 entry).
static constexpr int kFmtCsr16 = 2;
template <int FMT> constexpr bool is_csr = FMT != HSS_FMT_2OF4;

// Columns of entries ec .. ec + 3 (ec a multiple of 4), as a 16-byte (32-bit
// columns) or 8-byte (16-bit columns) vector load.
template <int FMT>
__device__ __forceinline__ u32x4 col_chunk(const DecodeArgs& a, int64_t ec) {
  if constexpr (FMT == kFmtCsr16) {
    const u32x2 c = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(a.col16 + ec));
    return u32x4{c.x & 0xffffu, c.x >> 16, c.y & 0xffffu, c.y >> 16};
  } else {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.col_idx + ec));
  }
}

template <int FMT>
__device__ __forceinline__ int col_at(const DecodeArgs& a, int64_t p) {
  if constexpr (FMT == kFmtCsr16) return a.col16[p];
  else return a.col_idx[p];
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

template <int DT>
__device__ __forceinline__ float fval(uint32_t bits) {
  return Elem<DT>::to_f(bits);
}

// acc += dot of two 16-byte vectors (8 bf16 or 4 fp32 products).
template <int DT>
__device__ __forceinline__ float dot16(const u32x4& a, const u32x4& b, float acc) {
  if constexpr (DT == HSS_BF16) {
    acc = dot2_bf16(a.x, b.x, acc);
    acc = dot2_bf16(a.y, b.y, acc);
    acc = dot2_bf16(a.z, b.z, acc);
    acc = dot2_bf16(a.w, b.w, acc);
  } else {
    acc = fmaf(__uint_as_float(a.x), __uint_as_float(b.x), acc);
    acc = fmaf(__uint_as_float(a.y), __uint_as_float(b.y), acc);
    acc = fmaf(__uint_as_float(a.z), __uint_as_float(b.z), acc);
    acc = fmaf(__uint_as_float(a.w), __uint_as_float(b.w), acc);
  }
  return acc;
}

// A call's T words carry tag epoch + 1.  The epoch runs 0 .. 2^32 - 2 and
// then wraps to 1 (keeping the parity alternating, which picks the counter
// set), so no tag is ever 0, the tag of a zero-filled word.
__device__ __forceinline__ uint32_t tag_of(uint32_t epoch) { return epoch + 1u; }
__device__ __forceinline__ uint32_t next_epoch(uint32_t tag) { return tag == 0xffffffffu ? 1u : tag; }

// Sum of the NW per-wave partials red[w][c] in a fixed order (NW = 4, 8 or 16).
template <int BC, int NW>
__device__ __forceinline__ float red_sum(float (*red)[BC], int c) {
  float s = (red[0][c] + red[1][c]) + (red[2][c] + red[3][c]);
  if constexpr (NW >= 8) s += (red[4][c] + red[5][c]) + (red[6][c] + red[7][c]);
  if constexpr (NW == 16) {
    s += ((red[8][c] + red[9][c]) + (red[10][c] + red[11][c])) +
         ((red[12][c] + red[13][c]) + (red[14][c] + red[15][c]));
  }
  return s;
}

// Block-wide T[c][l] = v[0 .. n) . xsrc[c * xld + (0 .. n)] for c < bc (all
// NT threads; v is V^T row l over the row's X columns, xsrc the first of
// them in column 0 of X, xld the X row stride).  Thread
// t covers 16-byte vectors q = t + NT*k; TV of them (per operand) are loaded
// before any is used.  Slots past the end load vector 0 (one address for the
// whole wave, a single request) and are skipped at use; clamping them to the
// last vector instead would send every block to the same L2 line.  Leaves
// the NT/64 wave sums in red[w][c] (the caller adds them with red_sum) after a
// barrier.
template <int DT, int BC, int NT>
__device__ __forceinline__ void t_row(const typename Elem<DT>::bits_t* __restrict__ v,
                                      const typename Elem<DT>::bits_t* __restrict__ xsrc, int n, int xld,
                                      int bc, int vec, float (*red)[BC]) {
  using bits_t = typename Elem<DT>::bits_t;
  constexpr int TV = BC <= 2 ? 4 : (BC <= 4 ? 2 : 1);
  const int t = threadIdx.x;
  float acc[BC];
#pragma unroll
  for (int c = 0; c < BC; ++c) acc[c] = 0.f;
  int jt = 0;
  if (vec) {
    constexpr int NV = 16 / sizeof(bits_t);
    const int nv = n / NV;
    const u32x4* v4 = reinterpret_cast<const u32x4*>(v);
    for (int base = 0; base < nv; base += NT * TV) {
      u32x4 vv[TV], xv[TV][BC];
      // every load unconditional (past the end: vector 0; past bc: column
      // bc - 1), so they are all in flight together -- a load under a branch
      // is waited for inside it
#pragma unroll
      for (int k = 0; k < TV; ++k) {
        const int q = base + t + NT * k;
        const int qc = q < nv ? q : 0;
        vv[k] = __builtin_nontemporal_load(v4 + qc);
#pragma unroll
        for (int c = 0; c < BC; ++c)
          xv[k][c] = reinterpret_cast<const u32x4*>(xsrc + (int64_t)min(c, bc - 1) * xld)[qc];
      }
#pragma unroll
      for (int k = 0; k < TV; ++k) {
        if (base + t + NT * k < nv) {
#pragma unroll
          for (int c = 0; c < BC; ++c)
            if (c < bc) acc[c] = dot16<DT>(vv[k], xv[k][c], acc[c]);
        }
      }
    }
    jt = nv * NV;
  }
  for (int j = jt + t; j < n; j += NT) {
    const float vj = fval<DT>(v[j]);
#pragma unroll
    for (int c = 0; c < BC; ++c)
      if (c < bc) acc[c] = fmaf(vj, fval<DT>(xsrc[(int64_t)c * xld + j]), acc[c]);
  }
  const int w = t >> 6;
#pragma unroll
  for (int c = 0; c < BC; ++c) {
    const float s = wave_sum(acc[c]);
    if (lane_id() == 0) red[w][c] = s;
  }
  __syncthreads();
}

// T row of one producer wave (one column, vector path): the same value, bit
// for bit, as t_row<DT, 1, NT> computes with a whole block, because lane L
// keeps the partial sums of the NT / 64 threads L, L + 64, ... of t_row, each
// over the same vectors in the same order, and adds their wave sums as
// red_sum does.  vv holds Vt row's vectors q = 64 s + L + NT k (k < KV, s <
// NT / 64; loaded by t_wave_issue), xl the row's X in LDS; n <= NT * KV *
// (16-byte vector elements).
static constexpr int kWaveProdKV = 2;
template <int DT, int NT>
__device__ __forceinline__ void t_wave_issue(const typename Elem<DT>::bits_t* __restrict__ v, int n,
                                             u32x4 (&vv)[kWaveProdKV][NT / 64]) {
  constexpr int NV = 16 / sizeof(typename Elem<DT>::bits_t);
  const int nv = n / NV, lane = lane_id();
  const u32x4* v4 = reinterpret_cast<const u32x4*>(v);
#pragma unroll
  for (int k = 0; k < kWaveProdKV; ++k) {
#pragma unroll
    for (int s = 0; s < NT / 64; ++s) {
      const int q = 64 * s + lane + NT * k;
      vv[k][s] = __builtin_nontemporal_load(v4 + (q < nv ? q : 0));  // past the end: vector 0, skipped
    }
  }
}

template <int DT, int NT>
__device__ __forceinline__ float t_wave_sum(const u32x4 (&vv)[kWaveProdKV][NT / 64],
                                            const typename Elem<DT>::bits_t* xl, int n) {
  constexpr int NS = NT / 64;
  static_assert(NS == 4, "red_sum order of four waves");
  constexpr int NV = 16 / sizeof(typename Elem<DT>::bits_t);
  const int nv = n / NV, lane = lane_id();
  const u32x4* x4 = reinterpret_cast<const u32x4*>(xl);
  float acc[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) acc[s] = 0.f;
#pragma unroll
  for (int k = 0; k < kWaveProdKV; ++k) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int q = 64 * s + lane + NT * k;
      if (q < nv) acc[s] = dot16<DT>(vv[k][s], x4[q], acc[s]);
    }
  }
  float ws[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) ws[s] = wave_sum(acc[s]);
  return (ws[0] + ws[1]) + (ws[2] + ws[3]);
}

// ---------------------------------------------------------------------------
// CSR rows.  Lane L of pass p holds entries [a0 + 4L + 256p, +4) of a row,
// a0 = row start rounded down to a multiple of 4 (16-byte aligned columns);
// entries outside [start, end) are masked.  Pass-0 chunks of all the wave's
// rows are loaded right after the row bounds return.  The array's last
// partial chunk (nnz % 4 entries) cannot be read as a vector; lanes 0..3
// load its entries one by one at kernel start (clamped, so always valid) and
// the chunk reads them back with readlane -- no load sits in the consume path.
// CP = 2 also loads the pass-1 chunks up front (rows of up to 509 entries
// then need no dependent load); passes beyond are loaded in the consume loop.
// ---------------------------------------------------------------------------
template <int DT, int RPW, int CP = 1>
struct CsrChunks {
  static constexpr int VB = 4 * sizeof(typename Elem<DT>::bits_t);  // value bytes per chunk
  typedef uint32_t vchunk_t __attribute__((ext_vector_type(VB / 4)));
  int st[RPW], en[RPW], e0[RPW];
  u32x4 cq[RPW];
  vchunk_t vq[RPW];
  u32x4 cq1[CP > 1 ? RPW : 1];   // pass 1 (CP == 2)
  vchunk_t vq1[CP > 1 ? RPW : 1];
  uint32_t tcol = 0, tval = 0;  // lane k < 4: entry (nnz & ~3) + k of the array tail
};

template <int DT, int FMT, int RPW, int CP = 1>
__device__ __forceinline__ void csr_tail_issue(const DecodeArgs& a, CsrChunks<DT, RPW, CP>& ch) {
  using bits_t = typename Elem<DT>::bits_t;
  const int64_t e = (a.nnz & ~(int64_t)3) + (lane_id() & 3);
  const int64_t ec = e < a.nnz - 1 ? e : a.nnz - 1;
  if constexpr (FMT == kFmtCsr16)
    ch.tcol = (uint32_t)__builtin_nontemporal_load(a.col16 + ec);
  else
    ch.tcol = (uint32_t)__builtin_nontemporal_load(a.col_idx + ec);
  ch.tval = (uint32_t)__builtin_nontemporal_load(static_cast<const bits_t*>(a.vals) + ec);
}

template <int DT, int FMT, int RPW, int CP = 1>
__device__ __forceinline__ void csr_issue(const DecodeArgs& a, const int (&rb)[RPW + 1],
                                          CsrChunks<DT, RPW, CP>& ch) {
  using bits_t = typename Elem<DT>::bits_t;
  using vchunk_t = typename CsrChunks<DT, RPW, CP>::vchunk_t;
  const int lane = lane_id();
  const bits_t* __restrict__ vals = static_cast<const bits_t*>(a.vals);
  // highest aligned full chunk; entry indices fit 32 bits (arrays hold
  // fewer than 2^31 elements), so the clamps are 32-bit
  const uint32_t last = (uint32_t)((a.nnz - 4) & ~(int64_t)3);
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    ch.st[i] = uniform(rb[i]);
    ch.en[i] = uniform(rb[i + 1]);
    ch.e0[i] = (ch.st[i] & ~3) + 4 * lane;
    if (a.vec_csr) {
      const uint32_t ec = min((uint32_t)ch.e0[i], last);
      ch.cq[i] = col_chunk<FMT>(a, ec);
      ch.vq[i] = __builtin_nontemporal_load(reinterpret_cast<const vchunk_t*>(vals + ec));
    }
  }
  if constexpr (CP > 1) {
    if (a.vec_csr) {
#pragma unroll
      for (int i = 0; i < RPW; ++i) {
        const uint32_t ec = min((uint32_t)ch.e0[i] + 256u, last);
        ch.cq1[i] = col_chunk<FMT>(a, ec);
        ch.vq1[i] = __builtin_nontemporal_load(reinterpret_cast<const vchunk_t*>(vals + ec));
      }
    }
  }
}

// One chunk (entries e..e+3): the four X values are gathered with no branch
// (entries outside [st, en) read column 0) so the LDS reads go out back to
// back; csr_chunk_fma then adds the in-range products, in entry order.
template <int DT, int BC>
struct ChunkX {
  uint32_t vb[4];   // value bits
  bool in[4];       // entry in [st, en)
  float x[4][BC];   // gathered X
};

// The array's last partial chunk as wave-uniform values (read from lanes
// 0..3 once per wave, outside any lane-dependent branch: a readlane under a
// divergent select compiles into an exec-masked branch per entry).
struct CsrTail {
  int col[4];
  uint32_t val[4];
};

__device__ __forceinline__ CsrTail csr_tail_values(uint32_t tcol, uint32_t tval) {
  CsrTail t;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    t.col[k] = __builtin_amdgcn_readlane((int)tcol, k);
    t.val[k] = (uint32_t)__builtin_amdgcn_readlane((int)tval, k);
  }
  return t;
}

template <int DT, int BC, typename VC>
__device__ __forceinline__ void csr_chunk_gather(const DecodeArgs& a, int e, int st, int en, const u32x4& cc,
                                                 const VC& vv, const CsrTail& tl,
                                                 const typename Elem<DT>::bits_t* __restrict__ xsrc,
                                                 ChunkX<DT, BC>& g) {
  using bits_t = typename Elem<DT>::bits_t;
  const bool whole = e + 4 <= a.nnz;  // else: the array's tail
  const int cols[4] = {(int)cc.x, (int)cc.y, (int)cc.z, (int)cc.w};
  uint32_t vb4[4];
  if constexpr (sizeof(bits_t) == 2) {
    vb4[0] = vv.x & 0xffffu; vb4[1] = vv.x >> 16; vb4[2] = vv.y & 0xffffu; vb4[3] = vv.y >> 16;
  } else {
    vb4[0] = vv.x; vb4[1] = vv.y; vb4[2] = vv.z; vb4[3] = vv.w;
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int ek = e + k;
    g.in[k] = ek >= st && ek < en;
    const int ck = whole ? cols[k] : tl.col[k];
    g.vb[k] = whole ? vb4[k] : tl.val[k];
    const int cx = g.in[k] ? ck : 0;
#pragma unroll
    for (int c = 0; c < BC; ++c)
      g.x[k][c] = fval<DT>(xsrc[(c == 0 ? 0 : (int64_t)min(c, a.bc - 1) * a.n) + cx]);
  }
}

template <int DT, int BC>
__device__ __forceinline__ void csr_chunk_fma(const ChunkX<DT, BC>& g, float (&acc)[BC]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float vk = fval<DT>(g.vb[k]);
#pragma unroll
    for (int c = 0; c < BC; ++c) {
      const float f = fmaf(vk, g.x[k][c], acc[c]);
      acc[c] = g.in[k] ? f : acc[c];
    }
  }
}

// bf16 chunk (entries e .. e + 3) of a row whose entries all lie in whole
// chunks of the arrays (en <= nnz rounded down to 4: every row but those in
// the arrays' last partial chunk).  The four X values are gathered at the
// chunk's columns as they are -- every column is a valid index, also for
// entries outside [st, en) -- the entries outside [st, en) are zeroed in the
// values and in the gathered X (so that no product of them reaches the sum,
// whatever their values), and the two pairs go to v_dot2_f32_bf16: about
// half the instructions of csr_chunk_gather + csr_chunk_fma, which a launch
// of many rows spends a good part of its time issuing.
template <int BC, typename VC>
__device__ __forceinline__ void csr_chunk_dot2(const DecodeArgs& a, int e, int st, int en, const u32x4& cc,
                                               const VC& vv, const uint16_t* __restrict__ xsrc, float (&acc)[BC]) {
  const int lo = min(max(st - e, 0), 4), hi = min(max(en - e, 0), 4);
  const int m4 = (0xf << lo) & (0xf >> (4 - hi));  // bit k: entry e + k is the row's
  const uint32_t k01 = (m4 & 1 ? 0x0000ffffu : 0u) | (m4 & 2 ? 0xffff0000u : 0u);
  const uint32_t k23 = (m4 & 4 ? 0x0000ffffu : 0u) | (m4 & 8 ? 0xffff0000u : 0u);
  const uint32_t v01 = vv.x & k01, v23 = vv.y & k23;
  uint32_t x01[BC], x23[BC];
#pragma unroll
  for (int c = 0; c < BC; ++c) {
    const uint16_t* __restrict__ xc = xsrc + (c == 0 ? 0 : (int64_t)min(c, a.bc - 1) * a.n);
    const uint32_t x0 = xc[cc.x], x1 = xc[cc.y], x2 = xc[cc.z], x3 = xc[cc.w];
    x01[c] = (x0 | (x1 << 16)) & k01;
    x23[c] = (x2 | (x3 << 16)) & k23;
  }
#pragma unroll
  for (int c = 0; c < BC; ++c) acc[c] = dot2_bf16(v23, x23[c], dot2_bf16(v01, x01[c], acc[c]));
}

template <int DT, int FMT, int BC, int RPW, int CP = 1>
__device__ __forceinline__ void csr_consume(const DecodeArgs& a, CsrChunks<DT, RPW, CP>& ch,
                                            const typename Elem<DT>::bits_t* __restrict__ xsrc,
                                            float (&ssum)[RPW][BC]) {
  using bits_t = typename Elem<DT>::bits_t;
  using vchunk_t = typename CsrChunks<DT, RPW, CP>::vchunk_t;
  const int lane = lane_id();
  const bits_t* __restrict__ vals = static_cast<const bits_t*>(a.vals);
  const int64_t last = ((a.nnz - 4) & ~(int64_t)3);
  float accs[RPW][BC];
  const CsrTail tl = csr_tail_values(ch.tcol, ch.tval);
  const int64_t nnz4 = a.nnz & ~(int64_t)3;  // rows ending at or before this take csr_chunk_dot2 (bf16)
  if (DT == HSS_BF16 && a.vec_csr) {
    const uint16_t* __restrict__ x16 = reinterpret_cast<const uint16_t*>(xsrc);
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
#pragma unroll
      for (int c = 0; c < BC; ++c) accs[i][c] = 0.f;
      if (ch.en[i] <= nnz4) {  // wave-uniform
        csr_chunk_dot2<BC>(a, ch.e0[i], ch.st[i], ch.en[i], ch.cq[i], ch.vq[i], x16, accs[i]);
        if constexpr (CP > 1)
          csr_chunk_dot2<BC>(a, ch.e0[i] + 256, ch.st[i], ch.en[i], ch.cq1[i], ch.vq1[i], x16, accs[i]);
      } else {
        ChunkX<DT, BC> g;
        csr_chunk_gather<DT, BC>(a, ch.e0[i], ch.st[i], ch.en[i], ch.cq[i], ch.vq[i], tl, xsrc, g);
        csr_chunk_fma<DT, BC>(g, accs[i]);
        if constexpr (CP > 1) {
          csr_chunk_gather<DT, BC>(a, ch.e0[i] + 256, ch.st[i], ch.en[i], ch.cq1[i], ch.vq1[i], tl, xsrc, g);
          csr_chunk_fma<DT, BC>(g, accs[i]);
        }
      }
    }
  } else if (a.vec_csr) {
    // first chunks of all rows: every gather first, then the products
    ChunkX<DT, BC> g[RPW];
#pragma unroll
    for (int i = 0; i < RPW; ++i)
      csr_chunk_gather<DT, BC>(a, ch.e0[i], ch.st[i], ch.en[i], ch.cq[i], ch.vq[i], tl, xsrc, g[i]);
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
#pragma unroll
      for (int c = 0; c < BC; ++c) accs[i][c] = 0.f;
      csr_chunk_fma<DT, BC>(g[i], accs[i]);
    }
    if constexpr (CP > 1) {  // the prefetched pass-1 chunks, in the same order as the loop below
#pragma unroll
      for (int i = 0; i < RPW; ++i)
        csr_chunk_gather<DT, BC>(a, ch.e0[i] + 256, ch.st[i], ch.en[i], ch.cq1[i], ch.vq1[i], tl, xsrc, g[i]);
#pragma unroll
      for (int i = 0; i < RPW; ++i) csr_chunk_fma<DT, BC>(g[i], accs[i]);
    }
  }
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    float acc[BC];
#pragma unroll
    for (int c = 0; c < BC; ++c) acc[c] = 0.f;
    const int st = ch.st[i], en = ch.en[i];
    if (a.vec_csr) {
#pragma unroll
      for (int c = 0; c < BC; ++c) acc[c] = accs[i][c];
      for (int base = (st & ~3) + 256 * CP; base < en; base += 256) {  // rows longer than 256 CP - 3
        const int e = base + 4 * lane;
        const int64_t ec = e < last ? e : last;
        const u32x4 cc = col_chunk<FMT>(a, ec);
        const vchunk_t vv = __builtin_nontemporal_load(reinterpret_cast<const vchunk_t*>(vals + ec));
        if (DT == HSS_BF16 && en <= nnz4) {
          csr_chunk_dot2<BC>(a, e, st, en, cc, vv, reinterpret_cast<const uint16_t*>(xsrc), acc);
        } else {
          ChunkX<DT, BC> gl;
          csr_chunk_gather<DT, BC>(a, e, st, en, cc, vv, tl, xsrc, gl);
          csr_chunk_fma<DT, BC>(gl, acc);
        }
      }
    } else {
      for (int p = st + lane; p < en; p += 64) {
        const float v = fval<DT>(vals[p]);
        const int col = col_at<FMT>(a, p);
#pragma unroll
        for (int c = 0; c < BC; ++c)
          if (c < a.bc) acc[c] = fmaf(v, fval<DT>(xsrc[(int64_t)c * a.n + col]), acc[c]);
      }
    }
#pragma unroll
    for (int c = 0; c < BC; ++c) ssum[i][c] = acc[c];  // this lane's share; the row's sum is taken with U's
  }
}

// ---------------------------------------------------------------------------
// 2:4 rows.  Lane L owns metadata words L, L+64, ... (32 columns each); the
// first kWPL words of every row (metadata + 16 values) are loaded at kernel
// start.  Fast path (bf16, n % 32 == 0): the 4-bit group index becomes a
// byte-permute selector that packs the two kept X values next to each other,
// and one bf16 dot2 per group accumulates both products in fp32.
// ---------------------------------------------------------------------------
static constexpr int kWPL = 2;

template <int RPW>
struct NmWords {
  uint32_t mw[RPW][kWPL];
  u32x4 vv[RPW][kWPL][2];
};

template <int DT, int RPW>
__device__ __forceinline__ void nm_issue(const DecodeArgs& a, int row0, NmWords<RPW>& nw) {
  using bits_t = typename Elem<DT>::bits_t;
  if (!a.nm_fast) return;
  const int lane = lane_id();
  const int words = a.n >> 5;
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    const int rowc = min(row0 + i, a.m - 1);
    const uint32_t* __restrict__ Mr = a.meta + (int64_t)rowc * words;
    const bits_t* __restrict__ Vr = static_cast<const bits_t*>(a.nmv) + (int64_t)rowc * (a.n >> 1);
#pragma unroll
    for (int k = 0; k < kWPL; ++k) {
      const int wdc = min(lane + 64 * k, words - 1);
      nw.mw[i][k] = __builtin_nontemporal_load(Mr + wdc);
      const u32x4* vp = reinterpret_cast<const u32x4*>(Vr + wdc * 16);
      nw.vv[i][k][0] = __builtin_nontemporal_load(vp);
      nw.vv[i][k][1] = __builtin_nontemporal_load(vp + 1);
    }
  }
}

// X chunk of one 2:4 word (32 columns) of batch column c: four 16-byte
// vectors, from the padded LDS copy (pad: 16 bytes after every 64, so the
// lanes' 64-byte-strided reads fall on distinct banks) or from global X.
__device__ __forceinline__ void nm_xload(const uint16_t* __restrict__ xsrc, int n, int c, int c0, int pad,
                                         u32x4 (&xq)[4]) {
  const int64_t v = ((int64_t)c * n + c0) >> 3;  // a multiple of 4
  const u32x4* xp = reinterpret_cast<const u32x4*>(xsrc) + (pad ? v + (v >> 2) : v);
#pragma unroll
  for (int h = 0; h < 4; ++h) xq[h] = xp[h];
}

// acc += the word's 16 products with one column's X chunk (8 groups of 4
// columns, 2 kept values each), groups in ascending order; nothing is added
// unless `valid`.
__device__ __forceinline__ void nm_word_dot(uint32_t mw, const u32x4 (&vv)[2], const u32x4 (&xq)[4],
                                            bool valid, float& acc) {
  const uint32_t vw[8] = {vv[0].x, vv[0].y, vv[0].z, vv[0].w, vv[1].x, vv[1].y, vv[1].z, vv[1].w};
  uint32_t sel[8];
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    // bytes 2*i, 2*i+1 of the 8-byte group {x3 x2 | x1 x0} hold x[i]
    const uint32_t i0 = (mw >> (4 * g)) & 3u;
    const uint32_t i1 = (mw >> (4 * g + 2)) & 3u;
    sel[g] = (i0 | (i1 << 16)) * 0x0202u + 0x01000100u;
  }
  const uint32_t xw[16] = {xq[0].x, xq[0].y, xq[0].z, xq[0].w, xq[1].x, xq[1].y, xq[1].z, xq[1].w,
                           xq[2].x, xq[2].y, xq[2].z, xq[2].w, xq[3].x, xq[3].y, xq[3].z, xq[3].w};
  float f = acc;
#pragma unroll
  for (int g = 0; g < 8; ++g) f = dot2_bf16(vw[g], __builtin_amdgcn_perm(xw[2 * g + 1], xw[2 * g], sel[g]), f);
  acc = valid ? f : acc;
}

// Fast path: lane L owns words L + 64k of every row of the wave, so the X
// chunk of a word (per batch column) is read once and used for all RPW rows.
template <int DT, int BC, int RPW>
__device__ __forceinline__ void nm_consume(const DecodeArgs& a, int row0, const NmWords<RPW>& nw,
                                           const typename Elem<DT>::bits_t* __restrict__ xsrc,
                                           float (&ssum)[RPW][BC]) {
  using bits_t = typename Elem<DT>::bits_t;
  const int lane = lane_id();
  const int m = a.m, n = a.n, bc = a.bc;
  const int words = (n + 31) >> 5;
  float acc[RPW][BC];
#pragma unroll
  for (int i = 0; i < RPW; ++i)
#pragma unroll
    for (int c = 0; c < BC; ++c) acc[i][c] = 0.f;
  if constexpr (DT == HSS_BF16) {
    if (a.nm_fast) {
      const uint16_t* __restrict__ x16 = reinterpret_cast<const uint16_t*>(xsrc);
#pragma unroll
      for (int k = 0; k < kWPL; ++k) {
        const int wd = lane + 64 * k;
        const bool wv = wd < words;
#pragma unroll
        for (int c = 0; c < BC; ++c) {
          u32x4 xq[4];
          nm_xload(x16, n, min(c, bc - 1), (wv ? wd : 0) * 32, a.x_pad, xq);
#pragma unroll
          for (int i = 0; i < RPW; ++i) nm_word_dot(nw.mw[i][k], nw.vv[i][k], xq, wv, acc[i][c]);
        }
      }
      for (int base = 64 * kWPL; base < words; base += 64) {  // words beyond the prefetched ones
        const int wd = base + lane;
        const bool wv = wd < words;
        const int wdc = wv ? wd : words - 1;
        uint32_t mw[RPW];
        u32x4 vv[RPW][2];
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
          const int64_t rowc = min(row0 + i, m - 1);
          mw[i] = __builtin_nontemporal_load(a.meta + rowc * words + wdc);
          const u32x4* vp = reinterpret_cast<const u32x4*>(static_cast<const bits_t*>(a.nmv) +
                                                           rowc * (n >> 1) + wdc * 16);
          vv[i][0] = __builtin_nontemporal_load(vp);
          vv[i][1] = __builtin_nontemporal_load(vp + 1);
        }
#pragma unroll
        for (int c = 0; c < BC; ++c) {
          u32x4 xq[4];
          nm_xload(x16, n, min(c, bc - 1), wdc * 32, a.x_pad, xq);
#pragma unroll
          for (int i = 0; i < RPW; ++i) nm_word_dot(mw[i], vv[i], xq, wv, acc[i][c]);
        }
      }
    }
  }
  if (!(DT == HSS_BF16 && a.nm_fast)) {
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      const int row = row0 + i;
      if (row < m) {
        const uint32_t* __restrict__ Mr = a.meta + (int64_t)row * words;
        const bits_t* __restrict__ Vr = static_cast<const bits_t*>(a.nmv) + (int64_t)row * (n >> 1);
        for (int wd = lane; wd < words; wd += 64) {
          const uint32_t mw = Mr[wd];
          const int c0 = wd * 32;
          const int ng = min(8, (n - c0) >> 2);
          for (int g = 0; g < ng; ++g) {
            const uint32_t nib = (mw >> (4 * g)) & 15u;
            const int j0 = c0 + 4 * g + (int)(nib & 3u);
            const int j1 = c0 + 4 * g + (int)(nib >> 2);
            const float v0 = fval<DT>(Vr[(c0 >> 1) + 2 * g]);
            const float v1 = fval<DT>(Vr[(c0 >> 1) + 2 * g + 1]);
#pragma unroll
            for (int c = 0; c < BC; ++c) {
              if (c < bc) {
                acc[i][c] = fmaf(v0, fval<DT>(xsrc[(int64_t)c * n + j0]), acc[i][c]);
                acc[i][c] = fmaf(v1, fval<DT>(xsrc[(int64_t)c * n + j1]), acc[i][c]);
              }
            }
          }
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < RPW; ++i)
#pragma unroll
    for (int c = 0; c < BC; ++c) ssum[i][c] = acc[i][c];  // this lane's share; the row's sum is taken with U's
}

// ---------------------------------------------------------------------------
// U entries of this wave's rows.
// UQ > 0 (bf16, U 16-byte aligned, any r): row i's elements i*r .. i*r+r-1
// are read as the aligned 16-byte pieces (8 elements each) that cover them:
// lane L holds piece p0 + L + 64q (q < UQ), p0 = the piece holding the row's
// first element.  A piece may straddle the row's ends; its elements outside
// [0, r) are masked in the epilogue (their neighbours' rows are read from
// cache, never used).  UQ = 1 covers r <= 506 entirely, UQ = 2 r <= 1018; the
// epilogue reads any rest element by element.  Pieces past the row's last
// load the row's first piece again (one address per wave).
// UQ == 0 (fp32, or U not 16-byte aligned): lane L holds l = L + 64q (q < 8).
// Loads are never under a branch: a load under a branch is copied into its
// merged value right away, which makes the wave wait for it there.
// ---------------------------------------------------------------------------
static constexpr int kUPL = 8;

template <int UQ> struct UBuf { u32x4 p[UQ > 0 ? UQ : 1]; uint32_t e[UQ > 0 ? 1 : kUPL]; };

template <int DT, int RPW, int UQ>
__device__ __forceinline__ void u_issue(const DecodeArgs& a, int row0, UBuf<UQ> (&ub)[RPW]) {
  using bits_t = typename Elem<DT>::bits_t;
  const bits_t* __restrict__ U = static_cast<const bits_t*>(a.U);
  const int lane = lane_id();
  const int m = a.m, r = a.ru;
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    const int rowc = min(row0 + i, m - 1);  // U has fewer than 2^31 elements: 32-bit offsets
    if constexpr (UQ > 0) {
      const int e0 = rowc * r;
      const int p0 = e0 >> 3, plast = (e0 + r - 1) >> 3;
#pragma unroll
      for (int q = 0; q < UQ; ++q) {
        const int p = p0 + lane + 64 * q;
        ub[i].p[q] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(U) + (p <= plast ? p : p0));
      }
    } else {
#pragma unroll
      for (int q = 0; q < kUPL; ++q) {
        const int l = lane + 64 * q;
        ub[i].e[q] = __builtin_nontemporal_load(U + (int64_t)rowc * r + min(l, r - 1));  // masked at use
      }
    }
  }
}

// T in LDS: column c's value l at Tp[c * t_ld(r) + l], with kTPad zeros on
// each side of every column, so a piece reads its 8 T values from one base
// (its first l, clamped to r) without clamping each index.
static constexpr int kTPad = 8;
__device__ __host__ __forceinline__ int t_ld(int r) { return r + 2 * kTPad; }

// bf16 T (bf16 matrices whose U rows are read as 16-byte pieces): T is
// rounded to bf16 once, as the matrix-core routes round it, and each column
// holds two copies of its padded values, E (element j = T[j - kTPad]) and,
// t_ld2(r) elements later, O (element j = E[j + 1]), so that every pair
// T[l], T[l + 1] is one aligned 32-bit word, of E when l + kTPad is even and
// of O when it is odd.  A piece's 8 products are then 4 v_dot2_f32_bf16 of
// U words and T words, with the elements outside the row zeroed in both by
// a mask from a 256-entry table (one 16-byte read), where the fp32 T took
// 8 conversions, 8 FMAs and 8 range selects.  Both copies are zero outside
// [0, r) (the column's region is cleared before T is written).
__device__ __host__ __forceinline__ int t_ld2(int r) { return (t_ld(r) + 1) & ~1; }
// Halfword mask of a 16-byte piece whose elements k with bit k of m8 set
// are kept: entry m8 of the table, built once per block.
__device__ __forceinline__ u32x4 piece_mask(int m8) {
  uint32_t w[4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
    w[q] = ((m8 >> (2 * q)) & 1 ? 0x0000ffffu : 0u) | ((m8 >> (2 * q + 1)) & 1 ? 0xffff0000u : 0u);
  return u32x4{w[0], w[1], w[2], w[3]};
}

template <int DT, int BC, int RPW, int UQ>
__device__ __forceinline__ void u_epilogue(const DecodeArgs& a, int row0, const UBuf<UQ> (&ub)[RPW],
                                           const float* __restrict__ Tp0, const unsigned char* __restrict__ smem,
                                           float (&acc)[RPW][BC]) {
  using bits_t = typename Elem<DT>::bits_t;
  const bits_t* __restrict__ U = static_cast<const bits_t*>(a.U);
  const int lane = lane_id();
  const int m = a.m, r = a.ru, bc = a.bc;
  const int tld = t_ld(a.r);
  if constexpr (DT == HSS_BF16 && UQ > 0) {
    const uint16_t* __restrict__ T16 = reinterpret_cast<const uint16_t*>(smem + a.t_off);
    const u32x4* __restrict__ mtab = reinterpret_cast<const u32x4*>(smem + a.mtab_off);
    const int ld2 = t_ld2(a.r);
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      const int row = row0 + i;
#pragma unroll
      for (int c = 0; c < BC; ++c) acc[i][c] = 0.f;
      if (row >= m) continue;
      const int toff = row >= a.h_m0 ? a.h_toff : 0;  // T[h_toff ..] for the second row half of a block term
      const int64_t e0 = (int64_t)row * r;
      const int sh = (int)(e0 & 7);  // the row starts at element sh of its first piece
#pragma unroll
      for (int q = 0; q < UQ; ++q) {
        const int lb = 8 * (lane + 64 * q) - sh;  // l of the piece's first element (>= -7)
        const int base = min(lb, r);               // reads stay inside the column and its pads
        // elements k with 0 <= lb + k < r are kept
        const int lo = min(max(-lb, 0), 8), hi = min(max(r - lb, 0), 8);
        const u32x4 mk = mtab[(0xff << lo) & (0xffu >> (8 - hi)) & 0xff];
        const u32x4 uw = {ub[i].p[q].x & mk.x, ub[i].p[q].y & mk.y, ub[i].p[q].z & mk.z, ub[i].p[q].w & mk.w};
        const int s0 = base + toff + kTPad;  // E element of the piece's first T value
        const int off = (s0 & 1) ? ld2 + s0 - 1 : s0;
#pragma unroll
        for (int c = 0; c < BC; ++c) {
          const uint32_t* __restrict__ tw =
              reinterpret_cast<const uint32_t*>(T16 + (c == 0 ? 0 : min(c, bc - 1) * 2 * ld2) + off);
          float f = acc[i][c];
          f = dot2_bf16(uw.x, tw[0] & mk.x, f);
          f = dot2_bf16(uw.y, tw[1] & mk.y, f);
          f = dot2_bf16(uw.z, tw[2] & mk.z, f);
          f = dot2_bf16(uw.w, tw[3] & mk.w, f);
          acc[i][c] = f;
        }
      }
      for (int l = 512 * UQ - sh + lane; l < r; l += 64) {  // beyond the pieces in registers
        const float u = fval<DT>(U[e0 + l]);
#pragma unroll
        for (int c = 0; c < BC; ++c)
          if (c < bc) acc[i][c] = fmaf(u, bf16lo(T16[c * 2 * ld2 + l + toff + kTPad]), acc[i][c]);
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    const int row = row0 + i;
#pragma unroll
    for (int c = 0; c < BC; ++c) acc[i][c] = 0.f;
    if (row >= m) continue;
    // this row's T values: T[h_toff ..] in the second row half of a block-
    // structured term (pieces still read at most 8 past r or 7 before 0:
    // other T values or the column's zero pads)
    const float* __restrict__ Tp = Tp0 + (row >= a.h_m0 ? a.h_toff : 0);
    if constexpr (UQ > 0) {
      const int64_t e0 = (int64_t)row * r;
      const int sh = (int)(e0 & 7);  // the row starts at element sh of its first piece
#pragma unroll
      for (int q = 0; q < UQ; ++q) {
        const int lb = 8 * (lane + 64 * q) - sh;  // l of the piece's first element (>= -7)
        const int base = min(lb, r);               // reads stay inside the column and its pads
        // T reads first (no branch), then the masked products
        float tq[8][BC];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
#pragma unroll
          for (int c = 0; c < BC; ++c) tq[k][c] = Tp[(c == 0 ? 0 : min(c, bc - 1) * tld) + base + k];
        }
        const uint32_t w[4] = {ub[i].p[q].x, ub[i].p[q].y, ub[i].p[q].z, ub[i].p[q].w};
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const bool in = (unsigned)(lb + k) < (unsigned)r;
          const float u = (k & 1) ? bf16hi(w[k >> 1]) : bf16lo(w[k >> 1]);
#pragma unroll
          for (int c = 0; c < BC; ++c) {
            const float f = fmaf(u, tq[k][c], acc[i][c]);
            acc[i][c] = in ? f : acc[i][c];
          }
        }
      }
      for (int l = 512 * UQ - sh + lane; l < r; l += 64) {  // beyond the pieces in registers
        const float u = fval<DT>(U[e0 + l]);
#pragma unroll
        for (int c = 0; c < BC; ++c)
          if (c < bc) acc[i][c] = fmaf(u, Tp[c * tld + l], acc[i][c]);
      }
    } else {
      float tq[kUPL][BC];
#pragma unroll
      for (int q = 0; q < kUPL; ++q) {
        const int lc = min(lane + 64 * q, r - 1);
#pragma unroll
        for (int c = 0; c < BC; ++c) tq[q][c] = Tp[min(c, bc - 1) * tld + lc];
      }
#pragma unroll
      for (int q = 0; q < kUPL; ++q) {
        const bool in = lane + 64 * q < r;
        const float u = fval<DT>(ub[i].e[q]);
#pragma unroll
        for (int c = 0; c < BC; ++c) {
          const float f = fmaf(u, tq[q][c], acc[i][c]);
          acc[i][c] = in ? f : acc[i][c];
        }
      }
      for (int l = lane + 64 * kUPL; l < r; l += 64) {
        const float u = fval<DT>(U[(int64_t)row * r + l]);
#pragma unroll
        for (int c = 0; c < BC; ++c)
          if (c < bc) acc[i][c] = fmaf(u, Tp[c * tld + l], acc[i][c]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Arrival count, in three stages so that no atomic round trip sits on a
// block's critical path.  Thread 0 of every block:
//   arrive_issue  once its epoch load has returned, bumps one of the 64
//                 spread counters of set (epoch & 1).  An empty asm that reads
//                 the epoch register and yields an opaque zero offset orders
//                 the add after that load and keeps the compiler from
//                 rewriting the single-lane add as a wave scan that waits for
//                 the result at once;
//   arrive_check  later, reads that result; the last arrival on a spread
//                 counter bumps the set's top counter;
//   finish_epoch  at the block's end, the last arrival overall (every block
//                 has read the epoch) advances the epoch for the next call,
//                 which starts after this kernel -- one store.
// The other set was used by the previous call, which has completed: block 0
// clears it (clear_next_set) early in this call, away from any critical
// path, for the next call to count on.  (Clearing this call's own counters
// at its end put 66 device-scope stores between its last block and the end
// of the kernel.)
// ---------------------------------------------------------------------------
// The call epoch, read coherently at device scope (from L2): caches above L2
// are not guaranteed to be clean between launches.
__device__ __forceinline__ uint32_t load_epoch(const DecodeArgs& a) {
  return __hip_atomic_load(a.ctl + kCtlEpoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t arrive_issue(const DecodeArgs& a, int sub, uint32_t epoch) {
  uint32_t off = 0;
  asm volatile("" : "+v"(off) : "v"(epoch));
  return __hip_atomic_fetch_add(a.ctl + ctl_sub(epoch, sub) + off, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ bool arrive_check(const DecodeArgs& a, int G, int nsub, int sub, uint32_t epoch,
                                             uint32_t arrived, uint32_t& top) {
  // blocks on counter sub: ceil((G - sub) / nsub), nsub being G (< 64: one each) or 64
  const uint32_t quota = nsub == kNumSub ? (uint32_t)(G - sub + kNumSub - 1) >> 6 : 1u;
  const bool sub_last = arrived == quota - 1;
  if (sub_last) {
    uint32_t off = 0;
    asm volatile("" : "+v"(off));  // opaque: keeps the add a plain single-lane atomic
    top = __hip_atomic_fetch_add(a.ctl + ctl_top(epoch) + off, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  return sub_last;
}

__device__ __forceinline__ void finish_epoch(const DecodeArgs& a, int nsub, bool sub_last, uint32_t top,
                                             uint32_t tag) {
  if (sub_last && top == (uint32_t)nsub - 1)
    __hip_atomic_store(a.ctl + kCtlEpoch, next_epoch(tag), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Block 0, threads 0 .. 64: clear the counter set of the next call (the one
// the previous call counted on).
__device__ __forceinline__ void clear_next_set(const DecodeArgs& a, uint32_t epoch) {
  const int t = threadIdx.x;
  if (blockIdx.x == 0 && t <= kNumSub)
    __hip_atomic_store(a.ctl + ctl_top(epoch + 1u) + kCtlLine * t, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Grid: blocks [0, r) are T producers (row l of T each; the lowest block ids
// are dispatched first), the rest own 4*RPW output rows each.  (Producers of
// 2, 4 or 8 T rows each, so that fewer producer blocks hold residency slots,
// measured slower on the decoder layer -- 61-67 vs 59 us per token: the T
// rows, which every row block waits for, are then published later.)
//
// FAST instances are launched only when r > 0, X is staged through registers
// into LDS in one pass, and the sparse operand takes its vector path; with
// those flags fixed at compile time every load of the prologue is issued
// unconditionally, so the compiler can count outstanding loads exactly and
// never waits for the (dependent, slowest) sparse loads before it must.
//
// MERGED instances (CSR, one column, FAST; MTR > 0) have no producer blocks:
// kMergedThreads-thread blocks, at most one per CU, own 8*RPW rows each, and block `local` of a matrix with nb blocks also produces T rows
// local + nb*i (i < MTR, while below r).  The epoch, X and those Vt rows are
// loaded first; each wave adds its share of the rows' dot products as soon as
// they return, and the last wave to do so (an LDS counter) publishes them.
// The block's CSR chunks are requested only then, so they do not queue ahead
// of the Vt rows that every block waits for.  X is staged once per block of 8
// waves instead of once per 4, and the T reads after the barrier find the
// CU's load queue nearly empty.  (Measured on the 4096^2 layer: 512 threads
// beat 1024, whose 4096 waves take ~1 us to launch, delaying the last T rows.)
static constexpr int kXR = 4;      // staged X vectors per thread held in registers
static constexpr size_t kMaxLdsAll = 112 * 1024;  // dynamic LDS a decode block may request
static constexpr int kXRFast = 2;  // FAST: this many in the prologue, unconditionally; any more after it
static constexpr int kMergedThreads = 512;  // MERGED block size

template <int DT, int FMT, int BC, int RPW, int UQ, bool FAST, int MTR, int CP>
__global__ __launch_bounds__(MTR > 0 ? kMergedThreads : 256) void k_decode(GroupArgs ga) {
  using bits_t = typename Elem<DT>::bits_t;
  constexpr bool MERGED = MTR > 0;  // producers merged into the row blocks, MTR T rows each at most
  static_assert(!MERGED || (FAST && BC == 1 && is_csr<FMT>), "merged producers: one CSR column, FAST only");
  constexpr int NT = MERGED ? kMergedThreads : 256;  // threads per block
  constexpr int NW = NT / 64;              // waves per block
  // this block's matrix and its index among that matrix's producer or row blocks
  const int bid = blockIdx.x;
  const bool producer = bid < ga.prod_start[ga.G];
  int gi = 0;
  if (producer) {
    while (gi + 1 < ga.G && bid >= ga.prod_start[gi + 1]) ++gi;
  } else {
    while (gi + 1 < ga.G && bid >= ga.row_start[gi + 1]) ++gi;
  }
  const int local = bid - (producer ? ga.prod_start[gi] : ga.row_start[gi]);
  DecodeArgs a = ga.a[gi];
  if constexpr (FAST) {
    a.x_lds = 1;
    a.vec = 1;
    a.vec_csr = is_csr<FMT>;
    a.nm_fast = FMT == HSS_FMT_2OF4;
    a.x_pad = FMT == HSS_FMT_2OF4;
    __builtin_assume(a.r > 0);
    __builtin_assume(a.bc * a.n > 0);
  }
  const int nb = ga.row_start[gi + 1] - ga.row_start[gi];  // row blocks of this matrix
  if constexpr (MERGED) {
    a.bc = 1;
    __builtin_assume(a.r <= MTR * nb);
  }
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ float red[NW][BC];
  __shared__ uint32_t epoch_sh;
  __shared__ uint32_t tdone_sh;  // MERGED: waves that have added their shares of the T rows
  __shared__ float tred[MERGED ? MTR : 1][NW][1];  // MERGED: per-wave shares of each T row

  const int t = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);  // wave index, uniform
  const int m = a.m, n = a.n, r = a.r, bc = a.bc;
  const int G = (int)gridDim.x;
  const bits_t* __restrict__ X = static_cast<const bits_t*>(a.X);
  const bits_t* __restrict__ Vt = static_cast<const bits_t*>(a.Vt);
  float* Tp = reinterpret_cast<float*>(smem + a.t_off) + kTPad;  // T column 0, element 0
  uint32_t* miss = reinterpret_cast<uint32_t*>(smem + a.miss_off);
  bits_t* xs = reinterpret_cast<bits_t*>(smem + a.x_off);
  const bits_t* xsrc = a.x_lds ? xs : X;
  const int nsub = G < kNumSub ? G : kNumSub;
  // counter of this block: blockIdx mod nsub, nsub being G (< 64) or 64
  const int sub = G < kNumSub ? (int)blockIdx.x : (int)(blockIdx.x & (kNumSub - 1));

  // ---- T producer: Vt row l and X loaded together, published tagged into
  //      every replica ----
  if constexpr (!MERGED) {
    if constexpr (FAST && BC == 1 && NT == 256) {
      // Wave producers: wave w owns T row local * NW + w.  Every wave loads
      // its Vt row (rows past r: row r - 1, published by no one) while the
      // block stages X in LDS once, so a producer holds a residency slot of
      // one wave per T row instead of four, and a launch of a few thousand
      // blocks fits on the CUs at once.
      if (producer && ga.prod_rows > 1) {
        const uint32_t e = load_epoch(a);
        const int l = local * NW + w;  // wave-uniform
        const int lc = l < r ? l : r - 1;
        int tc0, tlen;
        t_cols(a, lc, tc0, tlen);
        u32x4 vv[kWaveProdKV][NT / 64];
        t_wave_issue<DT, NT>(Vt + (int64_t)lc * a.v_ld, tlen, vv);
        // X (n / NV <= 2 * NT vectors) into LDS, unpadded
        const u32x4* X4 = reinterpret_cast<const u32x4*>(X);
        u32x4* dst = reinterpret_cast<u32x4*>(smem + a.x_off);
        const int xv = n / (16 / (int)sizeof(bits_t));
        u32x4 xq[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const int q = t + NT * k;
          xq[k] = X4[q < xv ? q : 0];
        }
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const int q = t + NT * k;
          if (q < xv) dst[q] = xq[k];
        }
        __syncthreads();
        const float tval =
            t_wave_sum<DT, NT>(vv, reinterpret_cast<const bits_t*>(smem + a.x_off) + tc0, tlen);
        uint32_t arrived = 0;
        if (t == 0) arrived = arrive_issue(a, sub, e);
        if (l < r && lane_id() < kTReplicas) {
          const uint64_t word = (uint64_t)__float_as_uint(tval) | ((uint64_t)tag_of(e) << 32);
          __hip_atomic_store(a.Tt + (int64_t)lane_id() * a.t_stride + l, word, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
        }
        clear_next_set(a, e);
        if (t == 0) {
          uint32_t top = 0;
          const bool sub_last = arrive_check(a, G, nsub, sub, e, arrived, top);
          finish_epoch(a, nsub, sub_last, top, tag_of(e));
        }
        return;
      }
    }
    if (producer) {
      const int l = local;
      const uint32_t e = load_epoch(a);
      int tc0, tlen;
      t_cols(a, l, tc0, tlen);
      t_row<DT, BC, NT>(Vt + (int64_t)l * a.v_ld, X + tc0, tlen, n, bc, a.vec, red);
      uint32_t arrived = 0;
      if (t == 0) arrived = arrive_issue(a, sub, e);
      // lane rep of wave 0 publishes the row into replica rep
      if (t < kTReplicas) {
#pragma unroll
        for (int c = 0; c < BC; ++c) {
          if (c < bc) {
            const uint64_t word = (uint64_t)__float_as_uint(red_sum<BC, NW>(red, c)) | ((uint64_t)tag_of(e) << 32);
            __hip_atomic_store(a.Tt + (int64_t)t * a.t_stride + (int64_t)c * r + l, word, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
          }
        }
      }
      clear_next_set(a, e);
      if (t == 0) {
        uint32_t top = 0;
        const bool sub_last = arrive_check(a, G, nsub, sub, e, arrived, top);
        finish_epoch(a, nsub, sub_last, top, tag_of(e));
      }
      return;
    }
  }

  // ---- row blocks ----
  const int row0 = (local * NW + w) * RPW;  // wave-uniform
  if (MERGED && t == 0) tdone_sh = 0;

  // row bounds: uniform addresses, scalar loads (own counter, so waiting for
  // them does not wait for the vector loads below)
  int rb[RPW + 1];
  if constexpr (is_csr<FMT>) {
#pragma unroll
    for (int i = 0; i <= RPW; ++i) rb[i] = a.row_ptr[min(row0 + i, m)];
  }

  constexpr int NV = 16 / sizeof(bits_t);
  const bool xreg = a.x_lds && a.vec;
  const int xvecs = xreg ? bc * n / NV : 0;
  constexpr int XR = MERGED ? 1 : (FAST ? kXRFast : kXR);
  if constexpr (FAST) __builtin_assume(xvecs > 0);
  if constexpr (MERGED) __builtin_assume(xvecs <= NT * XR);
  u32x4 xr[XR];
  // Lanes past the end read vector 0: one address for the whole wave (a
  // single request, served from L1), where clamping to the last vector would
  // pile every block onto one L2 line.  FAST loads its XR vectors with no
  // branch at all (a branch around them makes the compiler hold several
  // times the registers there).
  auto x_issue = [&]() {
    if (FAST || xvecs > 0) {
#pragma unroll
      for (int k = 0; k < XR; ++k) {
        if (FAST || NT * k < xvecs) {  // block-uniform
          const int q = t + NT * k;
          xr[k] = reinterpret_cast<const u32x4*>(X)[q < xvecs ? q : 0];
        }
      }
    }
  };

  // MERGED: the epoch, X and this block's Vt rows go out first, so its T rows
  // can be published as soon as they return (loads return in issue order).
  // Slots past r load row l % r (a valid row, not the same one for every
  // block) and publish nothing.  Thread t takes vector t of each row and the
  // X vector it meets (t itself, or t + n/2 / NV for a row of the second
  // column half of a block-structured term), as t_row does.
  uint32_t epoch = 0;
  u32x4 vt[MERGED ? MTR : 1], xt[MERGED ? MTR : 1];
  int tvecs[MERGED ? MTR : 1];
  if constexpr (MERGED) {
    epoch = load_epoch(a);
    x_issue();
#pragma unroll
    for (int i = 0; i < MTR; ++i) {
      const int l = local + nb * i;
      const int lc = l < r ? l : l % r;
      int tc0, tlen;
      t_cols(a, lc, tc0, tlen);
      tvecs[i] = tlen / NV;
      const int q = t < tvecs[i] ? t : 0;
      vt[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(Vt + (int64_t)lc * a.v_ld) + q);
      xt[i] = reinterpret_cast<const u32x4*>(X + tc0)[q];
    }
  }

  // vector loads that depend on nothing: epoch, U rows, 2:4 words
  // every block reads the epoch and arrives, also those of a matrix with no
  // low-rank term in a grouped launch: the arrival quotas count every block
  if constexpr (!MERGED) epoch = load_epoch(a);
  UBuf<UQ> ub[RPW];
  if (r > 0) u_issue<DT, RPW, UQ>(a, row0, ub);
  NmWords<RPW> nw;
  if constexpr (FMT == HSS_FMT_2OF4) nm_issue<DT, RPW>(a, row0, nw);
  CsrChunks<DT, RPW, CP> ch;
  if constexpr (is_csr<FMT>) {
    if (a.vec_csr) csr_tail_issue<DT, FMT, RPW, CP>(a, ch);
  }

  // CSR chunks: the one dependent load (MERGED: after the T row is out)
  if constexpr (is_csr<FMT> && !MERGED) csr_issue<DT, FMT, RPW, CP>(a, rb, ch);

  // X for LDS, issued last otherwise: writing it to LDS waits for every load
  // above, all of which the sparse part needs right after the barrier anyway.
  if constexpr (!MERGED) x_issue();

  if constexpr (MERGED) {
    // this wave's shares of the block's T rows (X vector t times Vt vector
    // t; the same arithmetic as t_row, so a row computed again locally has
    // the same bits), then the last wave publishes the fixed-order sums.
    // The barrier only orders the counter's reset before its increments; it
    // does not wait for the loads in flight.
    __syncthreads();
    float p[MTR];
#pragma unroll
    for (int i = 0; i < MTR; ++i) p[i] = wave_sum(t < tvecs[i] ? dot16<DT>(vt[i], xt[i], 0.f) : 0.f);
    uint32_t done = 0;
    if (lane_id() == 0) {
#pragma unroll
      for (int i = 0; i < MTR; ++i) tred[i][w][0] = p[i];
      asm volatile("" ::: "memory");  // the shares are written before the count (LDS keeps a wave's order)
      done = __hip_atomic_fetch_add(&tdone_sh, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    done = (uint32_t)__builtin_amdgcn_readlane((int)done, 0);
    if (done == (uint32_t)NW - 1) {
      asm volatile("" ::: "memory");
      // lane 8i + k writes replica k of row i
      const int i = lane_id() / kTReplicas, rep = lane_id() % kTReplicas;
      const int l = local + nb * i;
      if (i < MTR && l < r) {
        const uint64_t word = (uint64_t)__float_as_uint(red_sum<1, NW>(tred[i], 0)) | ((uint64_t)tag_of(epoch) << 32);
        __hip_atomic_store(a.Tt + (int64_t)rep * a.t_stride + l, word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    csr_issue<DT, FMT, RPW, CP>(a, rb, ch);
  }

  if (t == 0) epoch_sh = epoch;
  {
    u32x4* dst = reinterpret_cast<u32x4*>(xs);
#pragma unroll
    for (int k = 0; k < XR; ++k) {
      const int q = t + NT * k;
      if (q < xvecs) dst[a.x_pad ? q + (q >> 2) : q] = xr[k];
    }
  }
  for (int q = t; q < (r + 31) / 32; q += NT) miss[q] = 0;
  constexpr bool T16 = DT == HSS_BF16 && UQ > 0;  // bf16 T in two copies (u_epilogue)
  if constexpr (T16) {
    // both copies of every column zero (the pads stay so), and the mask table
    uint32_t* tz = reinterpret_cast<uint32_t*>(smem + a.t_off);
    for (int q = t; q < bc * t_ld2(r); q += NT) tz[q] = 0u;
    if (t < 256) reinterpret_cast<u32x4*>(smem + a.mtab_off)[t] = piece_mask(t);
  } else {
    for (int q = t; q < 2 * kTPad * bc; q += NT) {  // the zero pads around every T column
      const int c = q / (2 * kTPad), j = q % (2 * kTPad);
      Tp[c * t_ld(r) + (j < kTPad ? j - kTPad : r + j - kTPad)] = 0.f;
    }
  }
  // T value l of column c into LDS
  auto t_put = [&](int c, int l, float v) {
    if constexpr (T16) {
      uint16_t* col = reinterpret_cast<uint16_t*>(smem + a.t_off) + c * 2 * t_ld2(r);
      const uint16_t h = f32_to_bf16(v);
      col[l + kTPad] = h;                  // E
      col[t_ld2(r) + l + kTPad - 1] = h;   // O (O[j] = E[j + 1])
    } else {
      Tp[c * t_ld(r) + l] = v;
    }
  };
  if (xvecs > 0) {
    // the rest of X, four vectors per thread in flight per step (unconditional
    // loads, past the end of X: vector 0)
    u32x4* dst = reinterpret_cast<u32x4*>(xs);
    const u32x4* X4 = reinterpret_cast<const u32x4*>(X);
    for (int q0 = t + NT * XR; q0 < xvecs; q0 += 4 * NT) {
      u32x4 v[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int q = q0 + NT * k;
        v[k] = X4[q < xvecs ? q : 0];
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int q = q0 + NT * k;
        if (q < xvecs) dst[a.x_pad ? q + (q >> 2) : q] = v[k];
      }
    }
  } else if (a.x_lds) {
    for (int q = t; q < bc * n; q += NT) xs[q] = X[q];
  }
  // Arrival right before the barrier: every load above has returned (X went
  // last), so nothing later waits for this atomic by accident.
  uint32_t arrived = 0;
  if (t == 0) arrived = arrive_issue(a, sub, epoch);
  __syncthreads();
  const uint32_t tag = tag_of(epoch_sh);
  clear_next_set(a, epoch_sh);

  // T words, first pass.  FAST: issued now and read after the sparse part,
  // which then has no memory wait that could catch them (its operands all
  // arrived before the barrier).  The loads take no branch -- a load under a
  // branch is copied into its merged value at once, which waits for it --
  // so slots past the end re-read a word this block reads anyway.  A word
  // still stale here is re-read below.
  constexpr int kTW = MERGED ? 1 : (FAST ? 2 : 4);
  const uint64_t* __restrict__ Tr = a.Tt + (int64_t)(blockIdx.x % kTReplicas) * a.t_stride;
  // The T rows this block reads: all r of them, or, for a block-structured
  // term whose rows all lie in one row half, that half's ru rows (the
  // epilogue reads no others).  Slot e is column e / tn, row tlo + e % tn.
  int tlo = 0, tn = r;
  if (a.h_m0 < m) {
    const int first = local * NW * RPW, last = first + NW * RPW - 1;
    if (first >= a.h_m0) {
      tlo = a.h_toff;
      tn = a.ru;
    } else if (last < a.h_m0) {
      tn = a.ru;
    }
  }
  const int ttotal = bc * tn;
  auto t_word = [&](int e) { return BC == 1 ? tlo + e : (e / tn) * r + tlo + e % tn; };
  // slots past the end re-read a word this block reads anyway (e - ttotal,
  // or word 0 when that is past the end too): a conditional subtract, not an
  // integer division
  auto t_slot = [&](int e) {
    const int w = e - ttotal;
    return e < ttotal ? e : (w < ttotal ? w : 0);
  };
  uint64_t tv[kTW];
  if constexpr (FAST) {
#pragma unroll
    for (int k = 0; k < kTW; ++k) {
      const int e = t + NT * k;
      tv[k] = __hip_atomic_load(Tr + t_word(t_slot(e)), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }

  // sparse part
  float ssum[RPW][BC];
  if constexpr (is_csr<FMT>)
    csr_consume<DT, FMT, BC, RPW, CP>(a, ch, xsrc, ssum);
  else
    nm_consume<DT, BC, RPW>(a, row0, nw, xsrc, ssum);

  bool sub_last = false;
  uint32_t top = 0;
  if (t == 0) sub_last = arrive_check(a, G, nsub, sub, epoch_sh, arrived, top);

  // T -> LDS: this block's replica (other passes read after the sparse part,
  // when the producers, dispatched first, have normally published), tag
  // check, bounded polling of stale words, then local computation of any row
  // still missing.
  if (r > 0) {
    for (int base = 0; base < ttotal; base += kTW * NT) {
      if (!FAST || base > 0) {
#pragma unroll
        for (int k = 0; k < kTW; ++k) {
          const int e = base + t + NT * k;
          tv[k] = __hip_atomic_load(Tr + t_word(t_slot(e)), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
#pragma unroll
      for (int k = 0; k < kTW; ++k) {
        const int e = base + t + NT * k;
        if (e < ttotal) {
          uint64_t v = tv[k];
          for (int s = 0; (uint32_t)(v >> 32) != tag && s < a.spin; ++s) {
            __builtin_amdgcn_s_sleep(1);
            v = __hip_atomic_load(Tr + t_word(e), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
          const int ce = BC == 1 ? 0 : e / tn;
          const int l = tlo + (BC == 1 ? e : e - ce * tn);
          if ((uint32_t)(v >> 32) == tag && a.spin >= 0) {
            t_put(ce, l, __uint_as_float((uint32_t)v));
          } else {
            atomicOr(&miss[l >> 5], 1u << (l & 31));
          }
        }
      }
    }
    __syncthreads();
    for (int wi = 0; wi < (r + 31) / 32; ++wi) {
      uint32_t bits = (uint32_t)__builtin_amdgcn_readfirstlane((int)miss[wi]);  // block-uniform
      while (bits) {
        const int l = wi * 32 + __ffs(bits) - 1;
        bits &= bits - 1;
        int tc0, tlen;
        t_cols(a, l, tc0, tlen);
        t_row<DT, BC, NT>(Vt + (int64_t)l * a.v_ld, (a.x_pad ? X : xsrc) + tc0, tlen, n, bc, a.vec, red);
        if (t < bc) t_put(t, l, red_sum<BC, NW>(red, t));
        __syncthreads();
      }
    }
  }

  // low-rank epilogue, store
  float lacc[RPW][BC];
  if (r > 0) u_epilogue<DT, BC, RPW, UQ>(a, row0, ub, Tp, smem, lacc);
  bits_t* __restrict__ Y = static_cast<bits_t*>(a.Y);
  const int lane = lane_id();
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    const int row = row0 + i;
#pragma unroll
    for (int c = 0; c < BC; ++c) {
      const float s = wave_sum((r > 0 ? lacc[i][c] : 0.f) + ssum[i][c]);  // one reduction per row and column
      if (row < m && c < bc && lane == c) {
        if constexpr (DT == HSS_F32)
          Y[(int64_t)c * m + row] = __float_as_uint(s);
        else
          Y[(int64_t)c * m + row] = f32_to_bf16(s);
      }
    }
  }
  if (t == 0) finish_epoch(a, nsub, sub_last, top, tag);
}

// ---------------------------------------------------------------------------
// Launch one instance; more than 64 KiB of dynamic LDS (wide batches: X for
// 8 columns) must be allowed per kernel first, once.
template <int DT, int FMT, int BC, int RPW, int UQ, bool FAST, int MTR = 0, int CP = 1>
static void launch_k(const GroupArgs& ga, unsigned grid, size_t lds, hipStream_t s) {
  static bool big_lds = false;
  if (lds > 64 * 1024 && !big_lds) {
    hipFuncSetAttribute(reinterpret_cast<const void*>(&k_decode<DT, FMT, BC, RPW, UQ, FAST, MTR, CP>),
                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMaxLdsAll);
    big_lds = true;
  }
  hipLaunchKernelGGL((k_decode<DT, FMT, BC, RPW, UQ, FAST, MTR, CP>), dim3(grid),
                     dim3(MTR > 0 ? kMergedThreads : 256), lds, s, ga);
}

template <int DT, int FMT, int RPW, int UQ>
static void launch_merged_tr(const GroupArgs& ga, unsigned grid, int mtr, size_t lds, hipStream_t s) {
  if (mtr == 1) launch_k<DT, FMT, 1, RPW, UQ, true, 1>(ga, grid, lds, s);
  else if (mtr == 2) launch_k<DT, FMT, 1, RPW, UQ, true, 2>(ga, grid, lds, s);
  else launch_k<DT, FMT, 1, RPW, UQ, true, 4>(ga, grid, lds, s);
}

// cp: CSR chunks per row loaded up front (2 only for one bf16 CSR column on
// the FAST path).
template <int DT, int FMT, int BC, int UQ>
static void launch_v(const GroupArgs& ga, unsigned grid, bool fast, int mtr, int rpw, int cp, size_t lds,
                     hipStream_t s) {
  if constexpr (DT == HSS_BF16) {
    if constexpr (BC == 1 && is_csr<FMT> && UQ > 0) {
      if (mtr > 0) {
        if (rpw == 1)
          launch_merged_tr<DT, FMT, 1, UQ>(ga, grid, mtr, lds, s);
        else if (rpw == 4)
          launch_merged_tr<DT, FMT, 4, UQ>(ga, grid, mtr, lds, s);
        else
          launch_merged_tr<DT, FMT, 2, UQ>(ga, grid, mtr, lds, s);
        return;
      }
    }
    if (fast) {
      if constexpr (BC == 1 && is_csr<FMT>) {
        if (cp == 2) {
          if (rpw == 1)
            launch_k<DT, FMT, BC, 1, UQ, true, 0, 2>(ga, grid, lds, s);
          else if (rpw == 4)
            launch_k<DT, FMT, BC, 4, UQ, true, 0, 2>(ga, grid, lds, s);
          else
            launch_k<DT, FMT, BC, 2, UQ, true, 0, 2>(ga, grid, lds, s);
          return;
        }
      }
      if (rpw == 1)
        launch_k<DT, FMT, BC, 1, UQ, true>(ga, grid, lds, s);
      else if (rpw == 4)
        launch_k<DT, FMT, BC, 4, UQ, true>(ga, grid, lds, s);
      else
        launch_k<DT, FMT, BC, 2, UQ, true>(ga, grid, lds, s);
      return;
    }
  }
  if (rpw == 1)
    launch_k<DT, FMT, BC, 1, UQ, false>(ga, grid, lds, s);
  else  // 2 (four rows per wave are launched FAST only)
    launch_k<DT, FMT, BC, 2, UQ, false>(ga, grid, lds, s);
}

template <int DT, int FMT, int BC>
static void launch_bc(const GroupArgs& ga, unsigned grid, int uq, bool fast, int mtr, int rpw, int cp, size_t lds,
                      hipStream_t s) {
  if constexpr (DT == HSS_BF16) {
    if (uq == 1) return launch_v<DT, FMT, BC, 1>(ga, grid, fast, mtr, rpw, cp, lds, s);
    if (uq == 2) return launch_v<DT, FMT, BC, 2>(ga, grid, fast, mtr, rpw, cp, lds, s);
  }
  launch_v<DT, FMT, BC, 0>(ga, grid, fast, 0, rpw, cp, lds, s);
}

template <int DT, int FMT>
static void launch_fmt(const GroupArgs& ga, unsigned grid, int bc, int uq, bool fast, int mtr, int rpw,
                       size_t lds, hipStream_t s) {
  if (bc == 1) launch_bc<DT, FMT, 1>(ga, grid, uq, fast, mtr, rpw, 1, lds, s);
  else if (bc == 2) launch_bc<DT, FMT, 2>(ga, grid, uq, fast, 0, rpw, 1, lds, s);
  else if (bc <= 4) launch_bc<DT, FMT, 4>(ga, grid, uq, fast, 0, rpw, 1, lds, s);
  else launch_bc<DT, FMT, 8>(ga, grid, uq, fast, 0, rpw, 1, lds, s);
}

// Instances of launch_fmt, compiled in separate files (decode_inst_*.hip)
// so that the build runs them in parallel.
void decode_launch_bf16_csr_b1(const GroupArgs& ga, unsigned grid, int uq, bool fast, int mtr, int rpw, int cp,
                               size_t lds, hipStream_t s);
void decode_launch_bf16_csr_bn(const GroupArgs& ga, unsigned grid, int bc, int uq, bool fast, int rpw,
                               size_t lds, hipStream_t s);
void decode_launch_bf16_csr16_b1(const GroupArgs& ga, unsigned grid, int uq, bool fast, int mtr, int rpw, int cp,
                                 size_t lds, hipStream_t s);
void decode_launch_bf16_csr16_bn(const GroupArgs& ga, unsigned grid, int bc, int uq, bool fast, int rpw,
                                 size_t lds, hipStream_t s);
void decode_launch_bf16_nm(const GroupArgs& ga, unsigned grid, int bc, int uq, bool fast, int rpw, size_t lds,
                           hipStream_t s);
void decode_launch_f32(const GroupArgs& ga, unsigned grid, int fmt, int bc, int rpw, size_t lds, hipStream_t s);

}  // namespace hss
