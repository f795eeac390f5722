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
//   * T row l is produced by "home" block l mod G at the start of the launch
//     and published as 64-bit words (fp32 value, call tag) with coherent
//     (agent-scope) stores -- there is no done counter;
//   * every block reads the tagged words with coherent loads after its own
//     sparse work, polls a stale word a bounded number of times, then computes
//     any row still missing itself (same arithmetic, so the same bits).  No
//     wait can hang and a stale value is never used;
//   * the call tag is epoch+1, the epoch being read by every block at its
//     start.  Each block then bumps one of 64 spread arrival counters; the
//     last block to arrive (two-level count) advances the epoch and clears the
//     counters.  All blocks have read the epoch before it can advance.
#include <stdlib.h>

#include "hss_internal.h"

namespace hss {

// Control region (uint32 words) at the start of the apply workspace.  Each
// counter sits on its own 128-byte line.
static constexpr int kCtlEpoch = 0;
static constexpr int kCtlTop = 32;
static constexpr int kCtlSub0 = 64;
static constexpr int kCtlSubStride = 32;
static constexpr int kNumSub = 64;
static constexpr size_t kCtlBytes = 16384;
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
};

// Several matrices that share X in one launch (at most kMaxGroup): the grid is
// the producer blocks of every matrix, then the row blocks of every matrix.
// One launch, so one epoch and one arrival count; each matrix has its own T
// words.
static constexpr int kMaxGroup = HSS_MAX_GROUP;
struct GroupArgs {
  DecodeArgs a[kMaxGroup];
  int G;
  int prod_start[kMaxGroup + 1];  // producer blocks of matrix g: [prod_start[g], prod_start[g + 1])
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

__device__ __forceinline__ uint32_t tag_of(uint32_t epoch) { return epoch + 1u; }

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

// Block-wide T[c][l] = Vt[l,:] . X[c,:] for c < bc (all NT threads).  Thread
// t covers 16-byte vectors q = t + NT*k; TV of them (per operand) are loaded
// before any is used.  Slots past the end load vector 0 (one address for the
// whole wave, a single request) and are skipped at use; clamping them to the
// last vector instead would send every block to the same L2 line.  Leaves
// the NT/64 wave sums in red[w][c] (the caller adds them with red_sum) after a
// barrier.
template <int DT, int BC, int NT>
__device__ __forceinline__ void t_row(const typename Elem<DT>::bits_t* __restrict__ v,
                                      const typename Elem<DT>::bits_t* __restrict__ xsrc, int n,
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
          xv[k][c] = reinterpret_cast<const u32x4*>(xsrc + (int64_t)min(c, bc - 1) * n)[qc];
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
      if (c < bc) acc[c] = fmaf(vj, fval<DT>(xsrc[(int64_t)c * n + j]), acc[c]);
  }
  const int w = t >> 6;
#pragma unroll
  for (int c = 0; c < BC; ++c) {
    const float s = wave_sum(acc[c]);
    if (lane_id() == 0) red[w][c] = s;
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// CSR rows.  Lane L of pass p holds entries [a0 + 4L + 256p, +4) of a row,
// a0 = row start rounded down to a multiple of 4 (16-byte aligned columns);
// entries outside [start, end) are masked.  Pass-0 chunks of all the wave's
// rows are loaded right after the row bounds return.  The array's last
// partial chunk (nnz % 4 entries) cannot be read as a vector; lanes 0..3
// load its entries one by one at kernel start (clamped, so always valid) and
// the chunk reads them back with readlane -- no load sits in the consume path.
// ---------------------------------------------------------------------------
template <int DT, int RPW>
struct CsrChunks {
  static constexpr int VB = 4 * sizeof(typename Elem<DT>::bits_t);  // value bytes per chunk
  typedef uint32_t vchunk_t __attribute__((ext_vector_type(VB / 4)));
  int st[RPW], en[RPW], e0[RPW];
  u32x4 cq[RPW];
  vchunk_t vq[RPW];
  uint32_t tcol, tval;  // lane k < 4: entry (nnz & ~3) + k of the array tail
};

template <int DT, int FMT, int RPW>
__device__ __forceinline__ void csr_tail_issue(const DecodeArgs& a, CsrChunks<DT, RPW>& ch) {
  using bits_t = typename Elem<DT>::bits_t;
  const int64_t e = (a.nnz & ~(int64_t)3) + (lane_id() & 3);
  const int64_t ec = e < a.nnz - 1 ? e : a.nnz - 1;
  if constexpr (FMT == kFmtCsr16)
    ch.tcol = (uint32_t)__builtin_nontemporal_load(a.col16 + ec);
  else
    ch.tcol = (uint32_t)__builtin_nontemporal_load(a.col_idx + ec);
  ch.tval = (uint32_t)__builtin_nontemporal_load(static_cast<const bits_t*>(a.vals) + ec);
}

template <int DT, int FMT, int RPW>
__device__ __forceinline__ void csr_issue(const DecodeArgs& a, const int (&rb)[RPW + 1],
                                          CsrChunks<DT, RPW>& ch) {
  using bits_t = typename Elem<DT>::bits_t;
  using vchunk_t = typename CsrChunks<DT, RPW>::vchunk_t;
  const int lane = lane_id();
  const bits_t* __restrict__ vals = static_cast<const bits_t*>(a.vals);
  const int64_t last = ((a.nnz - 4) & ~(int64_t)3);  // highest aligned full chunk
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    ch.st[i] = uniform(rb[i]);
    ch.en[i] = uniform(rb[i + 1]);
    ch.e0[i] = (ch.st[i] & ~3) + 4 * lane;
    if (a.vec_csr) {
      const int64_t ec = ch.e0[i] < last ? ch.e0[i] : last;
      ch.cq[i] = col_chunk<FMT>(a, ec);
      ch.vq[i] = __builtin_nontemporal_load(reinterpret_cast<const vchunk_t*>(vals + ec));
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

template <int DT, int BC, typename VC>
__device__ __forceinline__ void csr_chunk_gather(const DecodeArgs& a, int e, int st, int en, const u32x4& cc,
                                                 const VC& vv, uint32_t tcol, uint32_t tval,
                                                 const typename Elem<DT>::bits_t* __restrict__ xsrc,
                                                 ChunkX<DT, BC>& g) {
  using bits_t = typename Elem<DT>::bits_t;
  const bool whole = e + 4 <= a.nnz;  // else: the array's tail, from lanes 0..3
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
    const int ck = whole ? cols[k] : __builtin_amdgcn_readlane((int)tcol, k);
    g.vb[k] = whole ? vb4[k] : (uint32_t)__builtin_amdgcn_readlane((int)tval, k);
    const int cx = g.in[k] ? ck : 0;
#pragma unroll
    for (int c = 0; c < BC; ++c)
      g.x[k][c] = fval<DT>(xsrc[(int64_t)min(c, a.bc - 1) * a.n + cx]);
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

template <int DT, int FMT, int BC, int RPW>
__device__ __forceinline__ void csr_consume(const DecodeArgs& a, CsrChunks<DT, RPW>& ch,
                                            const typename Elem<DT>::bits_t* __restrict__ xsrc,
                                            float (&ssum)[RPW][BC]) {
  using bits_t = typename Elem<DT>::bits_t;
  using vchunk_t = typename CsrChunks<DT, RPW>::vchunk_t;
  const int lane = lane_id();
  const bits_t* __restrict__ vals = static_cast<const bits_t*>(a.vals);
  const int64_t last = ((a.nnz - 4) & ~(int64_t)3);
  float accs[RPW][BC];
  if (a.vec_csr) {
    // first chunks of all rows: every gather first, then the products
    ChunkX<DT, BC> g[RPW];
#pragma unroll
    for (int i = 0; i < RPW; ++i)
      csr_chunk_gather<DT, BC>(a, ch.e0[i], ch.st[i], ch.en[i], ch.cq[i], ch.vq[i], ch.tcol, ch.tval, xsrc, g[i]);
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
#pragma unroll
      for (int c = 0; c < BC; ++c) accs[i][c] = 0.f;
      csr_chunk_fma<DT, BC>(g[i], accs[i]);
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
      for (int base = (st & ~3) + 256; base < en; base += 256) {  // rows longer than 256 - 3
        const int e = base + 4 * lane;
        const int64_t ec = e < last ? e : last;
        const u32x4 cc = col_chunk<FMT>(a, ec);
        const vchunk_t vv = __builtin_nontemporal_load(reinterpret_cast<const vchunk_t*>(vals + ec));
        ChunkX<DT, BC> gl;
        csr_chunk_gather<DT, BC>(a, e, st, en, cc, vv, ch.tcol, ch.tval, xsrc, gl);
        csr_chunk_fma<DT, BC>(gl, acc);
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
    for (int c = 0; c < BC; ++c) ssum[i][c] = wave_sum(acc[c]);
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
    for (int c = 0; c < BC; ++c) ssum[i][c] = wave_sum(acc[i][c]);
}

// ---------------------------------------------------------------------------
// U entries of this wave's rows.  VECU (bf16, r % 4 == 0): lane L holds
// l = 4L + 256q .. +3 (q < 2 covers r <= 512) as 8-byte vectors; otherwise
// lane L holds l = L + 64q (q < 8).  Larger r continues in the epilogue.
// Out-of-range slots load a clamped valid address (one per wave) and are
// skipped at use: a load under a branch would be copied into its merged
// value right away, making the wave wait for it there.
// ---------------------------------------------------------------------------
static constexpr int kUPL = 8;

template <int DT, int RPW, bool VECU>
__device__ __forceinline__ void u_issue(const DecodeArgs& a, int row0, uint32_t (&ub)[RPW][kUPL]) {
  using bits_t = typename Elem<DT>::bits_t;
  const bits_t* __restrict__ U = static_cast<const bits_t*>(a.U);
  const int lane = lane_id();
  const int m = a.m, r = a.r;
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    const int row = row0 + i;
    const int64_t rowc = min(row, m - 1);
    if constexpr (VECU) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int l = 4 * lane + 256 * q;
        const int lc = min(l, r - 4);  // past the row: one address per wave
        const u32x2 u2 = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(U + rowc * r + lc));
        ub[i][2 * q] = u2.x;  // masked at use (the epilogue skips l >= r, row >= m)
        ub[i][2 * q + 1] = u2.y;
      }
    } else {
#pragma unroll
      for (int q = 0; q < kUPL; ++q) {
        const int l = lane + 64 * q;
        ub[i][q] = __builtin_nontemporal_load(U + rowc * r + min(l, r - 1));  // masked at use
      }
    }
  }
}

template <int DT, int BC, int RPW, bool VECU>
__device__ __forceinline__ void u_epilogue(const DecodeArgs& a, int row0, const uint32_t (&ub)[RPW][kUPL],
                                           const float* __restrict__ Ts, float (&acc)[RPW][BC]) {
  using bits_t = typename Elem<DT>::bits_t;
  const bits_t* __restrict__ U = static_cast<const bits_t*>(a.U);
  const int lane = lane_id();
  const int m = a.m, r = a.r, bc = a.bc;
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    const int row = row0 + i;
#pragma unroll
    for (int c = 0; c < BC; ++c) acc[i][c] = 0.f;
    if (row >= m) continue;
    if constexpr (VECU) {
      // T reads first (clamped index, no branch), then the masked products
      float4 tv[2][BC];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int lc = min(4 * lane + 256 * q, r - 4);
#pragma unroll
        for (int c = 0; c < BC; ++c) tv[q][c] = *reinterpret_cast<const float4*>(Ts + min(c, bc - 1) * r + lc);
      }
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const bool in = 4 * lane + 256 * q < r;
        const float u0 = bf16lo(ub[i][2 * q]), u1 = bf16hi(ub[i][2 * q]);
        const float u2 = bf16lo(ub[i][2 * q + 1]), u3 = bf16hi(ub[i][2 * q + 1]);
#pragma unroll
        for (int c = 0; c < BC; ++c) {
          float f = fmaf(u0, tv[q][c].x, acc[i][c]);
          f = fmaf(u1, tv[q][c].y, f);
          f = fmaf(u2, tv[q][c].z, f);
          f = fmaf(u3, tv[q][c].w, f);
          acc[i][c] = in ? f : acc[i][c];
        }
      }
      for (int l = 4 * lane + 512; l < r; l += 256) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float u = fval<DT>(U[(int64_t)row * r + l + k]);
#pragma unroll
          for (int c = 0; c < BC; ++c)
            if (c < bc) acc[i][c] = fmaf(u, Ts[c * r + l + k], acc[i][c]);
        }
      }
    } else {
      float tq[kUPL][BC];
#pragma unroll
      for (int q = 0; q < kUPL; ++q) {
        const int lc = min(lane + 64 * q, r - 1);
#pragma unroll
        for (int c = 0; c < BC; ++c) tq[q][c] = Ts[min(c, bc - 1) * r + lc];
      }
#pragma unroll
      for (int q = 0; q < kUPL; ++q) {
        const bool in = lane + 64 * q < r;
        const float u = fval<DT>(ub[i][q]);
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
          if (c < bc) acc[i][c] = fmaf(u, Ts[c * r + l], acc[i][c]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Arrival count, in three stages so that no atomic round trip sits on a
// block's critical path.  Thread 0 of every block:
//   arrive_issue  once its epoch load has returned, bumps one of the 64
//                 spread counters.  An empty asm that reads the epoch register
//                 and yields an opaque zero offset orders the add after that
//                 load and keeps the compiler from rewriting the single-lane
//                 add as a wave scan that waits for the result at once;
//   arrive_check  later, reads that result; the last arrival on a spread
//                 counter bumps the top counter;
//   finish_epoch  at the block's end, the last arrival overall (every block
//                 has read the epoch) clears the counters and advances the
//                 epoch for the next call, which starts after this kernel.
// ---------------------------------------------------------------------------
// The call epoch, read coherently at device scope (from L2): caches above L2
// are not guaranteed to be clean between launches.
__device__ __forceinline__ uint32_t load_epoch(const DecodeArgs& a) {
  return __hip_atomic_load(a.ctl + kCtlEpoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t arrive_issue(const DecodeArgs& a, int sub, uint32_t epoch) {
  uint32_t off = 0;
  asm volatile("" : "+v"(off) : "v"(epoch));
  return __hip_atomic_fetch_add(a.ctl + kCtlSub0 + kCtlSubStride * sub + off, 1u, __ATOMIC_RELAXED,
                                __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ bool arrive_check(const DecodeArgs& a, int G, int nsub, int sub, uint32_t arrived,
                                             uint32_t& top) {
  const bool sub_last = arrived == (uint32_t)((G - sub + nsub - 1) / nsub) - 1;
  if (sub_last) {
    uint32_t off = 0;
    asm volatile("" : "+v"(off));  // opaque: keeps the add a plain single-lane atomic
    top = __hip_atomic_fetch_add(a.ctl + kCtlTop + off, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  return sub_last;
}

__device__ __forceinline__ void finish_epoch(const DecodeArgs& a, int nsub, bool sub_last, uint32_t top,
                                             uint32_t tag) {
  if (sub_last && top == (uint32_t)nsub - 1) {
    for (int k = 0; k < nsub; ++k)
      __hip_atomic_store(a.ctl + kCtlSub0 + kCtlSubStride * k, 0u, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(a.ctl + kCtlTop, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(a.ctl + kCtlEpoch, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Grid: blocks [0, r) are T producers (row l of T each; the lowest block ids
// are dispatched first), the rest own 4*RPW output rows each.
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
static constexpr int kXRFast = 2;  // FAST: exactly this many, no branches (bc * n <= 4096 bf16)
static constexpr int kMergedThreads = 512;  // MERGED block size

template <int DT, int FMT, int BC, int RPW, bool VECU, bool FAST, int MTR>
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
    __builtin_assume(a.bc * a.n > 0 && a.bc * a.n <= 256 * kXRFast * (16 / (int)sizeof(bits_t)));
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
  float* Ts = reinterpret_cast<float*>(smem + a.t_off);
  uint32_t* miss = reinterpret_cast<uint32_t*>(smem + a.miss_off);
  bits_t* xs = reinterpret_cast<bits_t*>(smem + a.x_off);
  const bits_t* xsrc = a.x_lds ? xs : X;
  const int nsub = G < kNumSub ? G : kNumSub;
  const int sub = (int)blockIdx.x % nsub;

  // ---- T producer: Vt row l and X loaded together, published tagged into
  //      every replica ----
  if (producer) {
    const int l = local;
    const uint32_t e = load_epoch(a);
    t_row<DT, BC, NT>(Vt + (int64_t)l * n, X, n, bc, a.vec, red);
    if (t == 0) {
      const uint32_t arrived = arrive_issue(a, sub, e);
#pragma unroll
      for (int c = 0; c < BC; ++c) {
        if (c < bc) {
          const uint64_t word =
              (uint64_t)__float_as_uint(red_sum<BC, NW>(red, c)) | ((uint64_t)tag_of(e) << 32);
          for (int rep = 0; rep < kTReplicas; ++rep)
            __hip_atomic_store(a.Tt + (int64_t)rep * a.t_stride + (int64_t)c * r + l, word,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      uint32_t top = 0;
      const bool sub_last = arrive_check(a, G, nsub, sub, arrived, top);
      finish_epoch(a, nsub, sub_last, top, tag_of(e));
    }
    return;
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
  if constexpr (FAST) __builtin_assume(xvecs > 0 && xvecs <= NT * XR);
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
  // block) and publish nothing.
  uint32_t epoch = 0;
  u32x4 vt[MERGED ? MTR : 1];
  if constexpr (MERGED) {
    epoch = load_epoch(a);
    x_issue();
#pragma unroll
    for (int i = 0; i < MTR; ++i) {
      const int l = local + nb * i;
      const int lc = l < r ? l : l % r;
      vt[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(Vt + (int64_t)lc * n) + (t < xvecs ? t : 0));
    }
  }

  // vector loads that depend on nothing: epoch, U rows, 2:4 words
  if (!MERGED && r > 0) epoch = load_epoch(a);
  uint32_t ub[RPW][kUPL];
  if (r > 0) u_issue<DT, RPW, VECU>(a, row0, ub);
  NmWords<RPW> nw;
  if constexpr (FMT == HSS_FMT_2OF4) nm_issue<DT, RPW>(a, row0, nw);
  CsrChunks<DT, RPW> ch;
  if constexpr (is_csr<FMT>) {
    if (a.vec_csr) csr_tail_issue<DT, FMT, RPW>(a, ch);
  }

  // CSR chunks: the one dependent load (MERGED: after the T row is out)
  if constexpr (is_csr<FMT> && !MERGED) csr_issue<DT, FMT, RPW>(a, rb, ch);

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
    for (int i = 0; i < MTR; ++i) p[i] = wave_sum(t < xvecs ? dot16<DT>(vt[i], xr[0], 0.f) : 0.f);
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
    csr_issue<DT, FMT, RPW>(a, rb, ch);
  }

  if (r > 0 && t == 0) epoch_sh = epoch;
  {
    u32x4* dst = reinterpret_cast<u32x4*>(xs);
#pragma unroll
    for (int k = 0; k < XR; ++k) {
      const int q = t + NT * k;
      if (q < xvecs) dst[a.x_pad ? q + (q >> 2) : q] = xr[k];
    }
  }
  for (int q = t; q < (r + 31) / 32; q += NT) miss[q] = 0;
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
  if (r > 0 && t == 0) arrived = arrive_issue(a, sub, epoch);
  __syncthreads();
  const uint32_t tag = tag_of(epoch_sh);

  // T words, first pass.  FAST: issued now and read after the sparse part,
  // which then has no memory wait that could catch them (its operands all
  // arrived before the barrier).  The loads take no branch -- a load under a
  // branch is copied into its merged value at once, which waits for it --
  // so slots past the end re-read a word this block reads anyway.  A word
  // still stale here is re-read below.
  constexpr int kTW = MERGED ? 1 : (FAST ? 2 : 4);
  const uint64_t* __restrict__ Tr = a.Tt + (int64_t)(blockIdx.x % kTReplicas) * a.t_stride;
  const int ttotal = bc * r;
  uint64_t tv[kTW];
  if constexpr (FAST) {
#pragma unroll
    for (int k = 0; k < kTW; ++k) {
      const int e = t + NT * k;
      tv[k] = __hip_atomic_load(Tr + (e < ttotal ? e : e % ttotal), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }

  // sparse part
  float ssum[RPW][BC];
  if constexpr (is_csr<FMT>)
    csr_consume<DT, FMT, BC, RPW>(a, ch, xsrc, ssum);
  else
    nm_consume<DT, BC, RPW>(a, row0, nw, xsrc, ssum);

  bool sub_last = false;
  uint32_t top = 0;
  if (r > 0 && t == 0) sub_last = arrive_check(a, G, nsub, sub, arrived, top);

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
          tv[k] = __hip_atomic_load(Tr + (e < ttotal ? e : e % ttotal), __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT);
        }
      }
#pragma unroll
      for (int k = 0; k < kTW; ++k) {
        const int e = base + t + NT * k;
        if (e < ttotal) {
          uint64_t v = tv[k];
          for (int s = 0; (uint32_t)(v >> 32) != tag && s < a.spin; ++s) {
            __builtin_amdgcn_s_sleep(1);
            v = __hip_atomic_load(Tr + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
          if ((uint32_t)(v >> 32) == tag) {
            Ts[e] = __uint_as_float((uint32_t)v);
          } else {
            const int l = e % r;
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
        t_row<DT, BC, NT>(Vt + (int64_t)l * n, a.x_pad ? X : xsrc, n, bc, a.vec, red);
        if (t < bc) Ts[(int64_t)t * r + l] = red_sum<BC, NW>(red, t);
        __syncthreads();
      }
    }
  }

  // low-rank epilogue, store
  float lacc[RPW][BC];
  if (r > 0) u_epilogue<DT, BC, RPW, VECU>(a, row0, ub, Ts, lacc);
  bits_t* __restrict__ Y = static_cast<bits_t*>(a.Y);
  const int lane = lane_id();
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    const int row = row0 + i;
#pragma unroll
    for (int c = 0; c < BC; ++c) {
      const float s = (r > 0 ? wave_sum(lacc[i][c]) : 0.f) + ssum[i][c];
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

// Compute units of the current device, cached per device.
static int cu_count() {
  static int cache[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cache[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess) cache[dev] = v;
  }
  return cache[dev];
}

// HSS_DECODE_MERGED=0 keeps separate producer blocks (a diagnostic switch).
static bool merged_enabled() {
  const char* s = getenv("HSS_DECODE_MERGED");
  return !(s && s[0] == '0');
}

// ---------------------------------------------------------------------------
// Launch one instance; more than 64 KiB of dynamic LDS (wide batches: X for
// 8 columns) must be allowed per kernel first, once.
template <int DT, int FMT, int BC, int RPW, bool VECU, bool FAST, int MTR = 0>
static void launch_k(const GroupArgs& ga, unsigned grid, size_t lds, hipStream_t s) {
  static bool big_lds = false;
  if (lds > 64 * 1024 && !big_lds) {
    hipFuncSetAttribute(reinterpret_cast<const void*>(&k_decode<DT, FMT, BC, RPW, VECU, FAST, MTR>),
                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMaxLdsAll);
    big_lds = true;
  }
  hipLaunchKernelGGL((k_decode<DT, FMT, BC, RPW, VECU, FAST, MTR>), dim3(grid), dim3(MTR > 0 ? kMergedThreads : 256),
                     lds, s, ga);
}

template <int DT, int FMT, int RPW, bool VECU>
static void launch_merged_tr(const GroupArgs& ga, unsigned grid, int mtr, size_t lds, hipStream_t s) {
  if (mtr == 1) launch_k<DT, FMT, 1, RPW, VECU, true, 1>(ga, grid, lds, s);
  else if (mtr == 2) launch_k<DT, FMT, 1, RPW, VECU, true, 2>(ga, grid, lds, s);
  else launch_k<DT, FMT, 1, RPW, VECU, true, 4>(ga, grid, lds, s);
}

template <int DT, int FMT, int BC, bool VECU>
static void launch_v(const GroupArgs& ga, unsigned grid, bool fast, int mtr, int rpw, size_t lds,
                     hipStream_t s) {
  if constexpr (DT == HSS_BF16) {
    if constexpr (BC == 1 && is_csr<FMT>) {
      if (mtr > 0) {
        if (rpw == 1)
          launch_merged_tr<DT, FMT, 1, VECU>(ga, grid, mtr, lds, s);
        else if (rpw == 4)
          launch_merged_tr<DT, FMT, 4, VECU>(ga, grid, mtr, lds, s);
        else
          launch_merged_tr<DT, FMT, 2, VECU>(ga, grid, mtr, lds, s);
        return;
      }
    }
    if (fast) {
      if (rpw == 1)
        launch_k<DT, FMT, BC, 1, VECU, true>(ga, grid, lds, s);
      else if (rpw == 4)
        launch_k<DT, FMT, BC, 4, VECU, true>(ga, grid, lds, s);
      else
        launch_k<DT, FMT, BC, 2, VECU, true>(ga, grid, lds, s);
      return;
    }
  }
  if (rpw == 1)
    launch_k<DT, FMT, BC, 1, VECU, false>(ga, grid, lds, s);
  else  // 2 (four rows per wave are launched FAST only)
    launch_k<DT, FMT, BC, 2, VECU, false>(ga, grid, lds, s);
}

template <int DT, int FMT, int BC>
static void launch_bc(const GroupArgs& ga, unsigned grid, bool vecu, bool fast, int mtr, int rpw, size_t lds,
                      hipStream_t s) {
  if constexpr (DT == HSS_BF16) {
    if (vecu) return launch_v<DT, FMT, BC, true>(ga, grid, fast, mtr, rpw, lds, s);
  }
  launch_v<DT, FMT, BC, false>(ga, grid, fast, mtr, rpw, lds, s);
}

template <int DT, int FMT>
static void launch_fmt(const GroupArgs& ga, unsigned grid, int bc, bool vecu, bool fast, int mtr, int rpw,
                       size_t lds, hipStream_t s) {
  if (bc == 1) launch_bc<DT, FMT, 1>(ga, grid, vecu, fast, mtr, rpw, lds, s);
  else if (bc == 2) launch_bc<DT, FMT, 2>(ga, grid, vecu, fast, 0, rpw, lds, s);
  else if (bc <= 4) launch_bc<DT, FMT, 4>(ga, grid, vecu, fast, 0, rpw, lds, s);
  else launch_bc<DT, FMT, 8>(ga, grid, vecu, fast, 0, rpw, lds, s);
}

// Dynamic LDS budget per block.  CSR gathers X at random columns, so X goes
// to LDS even for 8 columns (64 KiB at n = 4096); 2:4 reads X in contiguous
// 64-byte chunks that caches serve well, and a large LDS request would halve
// the blocks per CU, so it keeps the smaller budget (measured: 8 columns of
// the 11008 x 4096 2:4 layer 45 us with X from cache, 72 us through LDS).
static constexpr size_t kMaxLdsCsr = 100 * 1024;
static constexpr size_t kMaxLdsNm = 60 * 1024;
static size_t max_lds(const hss_matrix* A) { return A->fmt == HSS_FMT_CSR ? kMaxLdsCsr : kMaxLdsNm; }
static bool col16_of(const hss_matrix* A) { return A->fmt == HSS_FMT_CSR && (A->flags & HSS_COL16); }

static size_t align16(size_t x) { return (x + 15) / 16 * 16; }

size_t decode_ctl_bytes() { return kCtlBytes; }

// Words between T replicas for a matrix of rank r: room for 8 columns, padded
// to whole 4 KiB pages plus one 128-byte line so copies start on different
// lines and pages.
static int64_t t_stride_words(int r) {
  const int64_t words = 8 * (int64_t)(r > 0 ? r : 1);
  return (words + 511) / 512 * 512 + 16;
}

size_t decode_t_bytes(const hss_matrix* A) {
  return sizeof(uint64_t) * (size_t)t_stride_words(A->r) * kTReplicas;
}

// Largest column count per launch (1, 2, 4 or 8) whose T fits the LDS budget;
// 0 if even one column does not fit.
int decode_max_cols(const hss_matrix* A) {
  for (int bc = 8; bc >= 1; bc /= 2) {
    const size_t tb = align16(sizeof(float) * (size_t)bc * A->r) +
                      align16(4 * (size_t)((A->r + 31) / 32));
    if (tb <= max_lds(A)) return bc;
  }
  return 0;
}

static int spin_limit() {
  const char* s = getenv("HSS_DECODE_SPIN");
  return s ? atoi(s) : 4096;
}

// Arguments of one matrix of a decode pass, and the per-matrix launch
// properties the group has to agree on.
struct MatrixLaunch {
  DecodeArgs a;
  size_t lds;
  bool vecu, fast;
  int rpw;
};

static MatrixLaunch matrix_launch(const hss_matrix* A, int bc, const void* X, void* Y, uint32_t* ctl, uint64_t* Tt) {
  MatrixLaunch L;
  DecodeArgs& a = L.a;
  a.m = A->m; a.n = A->n; a.r = A->r; a.bc = bc;
  a.row_ptr = A->row_ptr; a.vals = A->values;
  a.col_idx = col16_of(A) ? nullptr : A->col_idx;
  a.col16 = col16_of(A) ? reinterpret_cast<const uint16_t*>(A->col_idx) : nullptr;
  a.nmv = A->nm_values; a.meta = A->nm_meta;
  a.U = A->U; a.Vt = A->Vt; a.X = X; a.Y = Y;
  a.ctl = ctl;
  a.Tt = Tt;
  a.t_stride = t_stride_words(A->r);
  a.nnz = A->nnz;
  a.spin = spin_limit();

  const size_t es = A->dtype == HSS_F32 ? 4 : 2;
  const size_t tbytes = align16(sizeof(float) * (size_t)bc * A->r);
  const size_t mbytes = align16(4 * (size_t)((A->r + 31) / 32));
  const bool nm_fast = A->fmt == HSS_FMT_2OF4 && A->dtype == HSS_BF16 && ((uintptr_t)X % 16 == 0) &&
                       A->n % 32 == 0 && (uintptr_t)A->nm_values % 16 == 0 && (uintptr_t)A->nm_meta % 4 == 0 &&
                       (A->r == 0 || (uintptr_t)A->Vt % 16 == 0);
  // the 2:4 fast path reads 64-byte X chunks at a 64-byte lane stride: pad them
  const size_t xbytes = align16((size_t)bc * A->n * es * (nm_fast ? 5 : 4) / 4);
  a.t_off = 0;
  a.miss_off = (int)tbytes;
  a.x_off = (int)(tbytes + mbytes);
  a.x_lds = tbytes + mbytes + xbytes <= max_lds(A);
  a.x_pad = nm_fast && a.x_lds;
  // Vector dot products: X rows and Vt rows start 16-byte aligned.
  a.vec = ((uintptr_t)X % 16 == 0) && ((size_t)A->n * es) % 16 == 0 &&
          (A->r == 0 || (uintptr_t)A->Vt % 16 == 0);
  a.vec_csr = A->fmt == HSS_FMT_CSR && A->nnz >= 4 && (uintptr_t)A->col_idx % (col16_of(A) ? 8 : 16) == 0 &&
              (uintptr_t)A->values % (4 * es) == 0;
  a.nm_fast = A->fmt == HSS_FMT_2OF4 && A->dtype == HSS_BF16 && a.vec && A->n % 32 == 0 &&
              (uintptr_t)A->nm_values % 16 == 0 && (uintptr_t)A->nm_meta % 4 == 0;
  // bf16 U rows as 8-byte vectors; T rows in LDS (c * r floats) stay 16-byte aligned.
  L.vecu = A->dtype == HSS_BF16 && A->r > 0 && A->r % 4 == 0 && (uintptr_t)A->U % 8 == 0;
  L.lds = tbytes + mbytes + (a.x_lds ? xbytes : 0);
  L.fast = A->dtype == HSS_BF16 && A->r > 0 && a.x_lds && a.vec &&
           (size_t)bc * A->n / 8 <= 256 * (size_t)kXRFast &&
           (A->fmt == HSS_FMT_CSR ? a.vec_csr : a.nm_fast);
  // Rows per wave: more rows per block means fewer copies of X staged through
  // L2 into LDS and fewer blocks queueing loads on each CU (measured best:
  // 2 for 4096 rows, 4 for 11008 rows); small matrices keep one row per wave
  // for parallelism.  Four rows per wave exist only as FAST instances.
  L.rpw = A->m >= 8192 ? 4 : (A->m >= 2048 ? 2 : 1);
  return L;
}

// Merged producers for one CSR column (bf16, FAST): the fewest rows per wave
// (1, 2 or 4) whose blocks, 8*RPW rows each, number at most the CUs (each
// block waits for T rows that other blocks produce, so all must be resident;
// measured: with 2-3 merged blocks per CU the 3-matrix q/k/v launch of the
// decoder layer is slower than with separate producers), with at most 4 T
// rows per block (r <= 4 * blocks of each matrix).  Returns the T rows per
// block (1, 2 or 4; 0: not merged) and sets rpw.
static int merged_plan(const hss_matrix* const* A, int G, int bc, bool fast_bf16, int fmt, int& rpw) {
  if (bc != 1 || !fast_bf16 || fmt == HSS_FMT_2OF4 || !merged_enabled()) return 0;
  const int cus = cu_count();
  constexpr int mw = kMergedThreads / 64;
  for (int rp = 1; rp <= 4; rp *= 2) {
    int blocks = 0, tr = 0;
    for (int g = 0; g < G; ++g) {
      const int nb = (A[g]->m + mw * rp - 1) / (mw * rp);
      blocks += nb;
      const int t = (A[g]->r + nb - 1) / nb;
      tr = tr > t ? tr : t;
    }
    if (tr <= 4 && blocks <= cus) {
      rpw = rp;
      return tr <= 1 ? 1 : (tr <= 2 ? 2 : 4);
    }
  }
  return 0;
}

// One fused decode pass over bc columns (1 <= bc <= decode_max_cols of every
// matrix) for G matrices sharing X (same n, dtype and format); Y[g] is
// matrix g's output.  The T words of matrix g follow those of matrix g - 1.
void launch_decode_group(const hss_matrix* const* A, int G, int bc, const void* X, void* const* Y, void* ws,
                         hipStream_t s) {
  GroupArgs ga = {};
  ga.G = G;
  uint32_t* ctl = static_cast<uint32_t*>(ws);
  char* tw = static_cast<char*>(ws) + kCtlBytes;
  size_t lds = 0;
  bool vecu = true, fast = true;
  int rpw = 4;
  MatrixLaunch L[kMaxGroup];
  for (int g = 0; g < G; ++g) {
    L[g] = matrix_launch(A[g], bc, X, Y[g], ctl, reinterpret_cast<uint64_t*>(tw));
    tw += decode_t_bytes(A[g]);
    lds = lds > L[g].lds ? lds : L[g].lds;
    vecu = vecu && L[g].vecu;
    fast = fast && L[g].fast;
    rpw = rpw < L[g].rpw ? rpw : L[g].rpw;
  }
  if (!fast && rpw > 2) rpw = 2;
  const int dt = A[0]->dtype, fmt = col16_of(A[0]) ? kFmtCsr16 : A[0]->fmt;
  const int mtr = merged_plan(A, G, bc, fast && dt == HSS_BF16, fmt, rpw);
  const bool merged = mtr > 0;
  ga.prod_start[0] = 0;
  for (int g = 0; g < G; ++g) {
    ga.a[g] = L[g].a;
    ga.prod_start[g + 1] = ga.prod_start[g] + (merged ? 0 : A[g]->r);
  }
  ga.row_start[0] = ga.prod_start[G];
  const int rows_per_block = (merged ? kMergedThreads / 64 : 4) * rpw;
  for (int g = 0; g < G; ++g) ga.row_start[g + 1] = ga.row_start[g] + (A[g]->m + rows_per_block - 1) / rows_per_block;
  for (int g = G; g < kMaxGroup; ++g) { ga.prod_start[g + 1] = ga.prod_start[G]; ga.row_start[g + 1] = ga.row_start[G]; }
  const unsigned grid = (unsigned)ga.row_start[G];
  if (dt == HSS_F32) {
    if (fmt == HSS_FMT_CSR) launch_fmt<HSS_F32, HSS_FMT_CSR>(ga, grid, bc, false, false, 0, rpw, lds, s);
    else if (fmt == kFmtCsr16) launch_fmt<HSS_F32, kFmtCsr16>(ga, grid, bc, false, false, 0, rpw, lds, s);
    else launch_fmt<HSS_F32, HSS_FMT_2OF4>(ga, grid, bc, false, false, 0, rpw, lds, s);
  } else {
    if (fmt == HSS_FMT_CSR) launch_fmt<HSS_BF16, HSS_FMT_CSR>(ga, grid, bc, vecu, fast, mtr, rpw, lds, s);
    else if (fmt == kFmtCsr16) launch_fmt<HSS_BF16, kFmtCsr16>(ga, grid, bc, vecu, fast, mtr, rpw, lds, s);
    else launch_fmt<HSS_BF16, HSS_FMT_2OF4>(ga, grid, bc, vecu, fast, mtr, rpw, lds, s);
  }
}

void launch_decode(const hss_matrix* A, int bc, const void* X, void* Y, void* ws, hipStream_t s) {
  launch_decode_group(&A, 1, bc, X, &Y, ws, s);
}

// ---------------------------------------------------------------------------
// Dense-and-sparse apply (HSS_DQ4 matrices):
//   Y[c][i] = sum_{j in S_i} S_ij X[c][j] + sum_j D(i, j) X[c][j],
//   D(i, j) = levels[i][code(i, j)],
// [SQZ] page aibr.jp/archives/208940, section "3.中核となる技術的要素": the
// dense part, quantised with non-uniform levels, and the outliers in CSR are
// multiplied side by side.  The codes (4 bits per weight) are the dominant
// stream; every byte holds the codes of two adjacent columns, so one lookup
// in a 256-entry table of level pairs (rebuilt per row from the row's 16
// levels, in the wave's own LDS) gives both weights, and one dot2 (bf16) or
// two FMAs (fp32) with the matching X pair from LDS accumulates them.
//
// Block: 4 waves, RPW rows per wave.  Lane L owns 16-byte code chunks
// L + 64 k of each row (32 columns each); the first kDqPre chunks of every
// row are requested at kernel start with the CSR chunks, the rest inside the
// loop.  X (bc columns) is staged in LDS for both parts.
// ---------------------------------------------------------------------------
static constexpr int kDqPre = 2;

struct DqArgs {
  DecodeArgs a;          // m, n, bc, X, Y and the CSR outliers (r = 0)
  const uint8_t* codes;  // m x n/2 bytes
  const void* levels;    // m x 16, storage type
  int vec_codes;         // rows of codes 16-byte aligned (n % 32 == 0, aligned base)
  int tab_off;           // dynamic LDS byte offset of the 4 per-wave tables
};

template <int DT> struct DqEntry;  // one table entry: levels of (low, high) nibble
template <> struct DqEntry<HSS_BF16> { using t = uint32_t; };
template <> struct DqEntry<HSS_F32> { using t = u32x2; };

// acc += (lo, hi) . (x[2p], x[2p + 1]) for one code byte.
template <int DT>
__device__ __forceinline__ float dq_pair(const typename DqEntry<DT>::t& e, uint32_t x0, uint32_t x1, float acc) {
  if constexpr (DT == HSS_BF16) {
    return dot2_bf16(e, x0, acc);  // x0 holds both bf16 x values
  } else {
    acc = fmaf(__uint_as_float(e.x), __uint_as_float(x0), acc);
    return fmaf(__uint_as_float(e.y), __uint_as_float(x1), acc);
  }
}

// One 16-byte code chunk q (columns 32 q .. 32 q + 31) of one row: 16 table
// lookups, then the products with every column of X.  `valid` bytes of the
// chunk belong to the row (a row's last chunk may be partial).
template <int DT, int BC>
__device__ __forceinline__ void dq_chunk(const u32x4& cw, int q, int valid, const typename DqEntry<DT>::t* tab,
                                         const typename Elem<DT>::bits_t* xs, int n, int bc, float (&acc)[BC]) {
  using E = typename DqEntry<DT>::t;
  const uint32_t w4[4] = {cw.x, cw.y, cw.z, cw.w};
  E e[16];
#pragma unroll
  for (int b = 0; b < 16; ++b) e[b] = tab[(w4[b >> 2] >> (8 * (b & 3))) & 0xffu];
#pragma unroll
  for (int c = 0; c < BC; ++c) {
    if (c >= bc) break;
    const typename Elem<DT>::bits_t* xr = xs + (int64_t)c * n + 32 * q;
    if constexpr (DT == HSS_BF16) {
      const u32x4* xv = reinterpret_cast<const u32x4*>(xr);  // 32 bf16 = 4 x 16 bytes
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const u32x4 x4 = xv[v];
        const uint32_t xw[4] = {x4.x, x4.y, x4.z, x4.w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int b = 4 * v + t;
          const float f = dq_pair<DT>(e[b], xw[t], 0u, acc[c]);
          acc[c] = b < valid ? f : acc[c];
        }
      }
    } else {
      const u32x4* xv = reinterpret_cast<const u32x4*>(xr);  // 32 fp32 = 8 x 16 bytes
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        const u32x4 x4 = xv[v];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int b = 2 * v + t;
          const float f = dq_pair<DT>(e[b], t ? x4.z : x4.x, t ? x4.w : x4.y, acc[c]);
          acc[c] = b < valid ? f : acc[c];
        }
      }
    }
  }
}

template <int DT, int FMT, int BC, int RPW>
__global__ __launch_bounds__(256) void k_decode_dq(DqArgs q) {
  using bits_t = typename Elem<DT>::bits_t;
  using E = typename DqEntry<DT>::t;
  const DecodeArgs& a = q.a;
  extern __shared__ __align__(16) unsigned char smem[];
  bits_t* xs = reinterpret_cast<bits_t*>(smem + a.x_off);
  const int t = threadIdx.x, lane = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  E* tab = reinterpret_cast<E*>(smem + q.tab_off) + w * 256;
  const int m = a.m, n = a.n, bc = a.bc;
  const int row0 = ((int)blockIdx.x * 4 + w) * RPW;
  const int nb = n >> 1;                 // code bytes per row
  const int nch = (nb + 15) >> 4;        // 16-byte chunks per row
  const bits_t* __restrict__ X = static_cast<const bits_t*>(a.X);
  const bits_t* __restrict__ L = static_cast<const bits_t*>(q.levels);

  // CSR outliers: row bounds (scalar), chunk loads
  int rb[RPW + 1];
#pragma unroll
  for (int i = 0; i <= RPW; ++i) rb[i] = a.row_ptr[min(row0 + i, m)];
  CsrChunks<DT, RPW> ch;
  if (a.vec_csr) csr_tail_issue<DT, FMT, RPW>(a, ch);
  // levels (lane k % 16 holds level k % 16 of each row) and the first code chunks
  uint32_t lv[RPW];
  u32x4 cpre[RPW][kDqPre];
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    const int64_t rowc = min(row0 + i, m - 1);
    lv[i] = (uint32_t)L[rowc * 16 + (lane & 15)];
#pragma unroll
    for (int k = 0; k < kDqPre; ++k) {
      const int cq = min(lane + 64 * k, nch - 1);
      if (q.vec_codes)
        cpre[i][k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(q.codes + rowc * nb) + cq);
      else
        cpre[i][k] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  csr_issue<DT, FMT, RPW>(a, rb, ch);

  // X -> LDS, four vectors per thread in flight per step (unconditional
  // loads; past the end of X: vector 0)
  constexpr int NV = 16 / sizeof(bits_t);
  if (a.vec) {
    const int xv = bc * n / NV;
    const u32x4* X4 = reinterpret_cast<const u32x4*>(X);
    for (int v0 = t; v0 < xv; v0 += 4 * 256) {
      u32x4 vv[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int v = v0 + 256 * k;
        vv[k] = X4[v < xv ? v : 0];
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int v = v0 + 256 * k;
        if (v < xv) reinterpret_cast<u32x4*>(xs)[v] = vv[k];
      }
    }
  } else {
    for (int v = t; v < bc * n; v += 256) xs[v] = X[v];
  }
  __syncthreads();

  // sparse part
  float ssum[RPW][BC];
  csr_consume<DT, FMT, BC, RPW>(a, ch, xs, ssum);

  bits_t* __restrict__ Y = static_cast<bits_t*>(a.Y);
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    const int row = row0 + i;
    const int64_t rowc = min(row, m - 1);
    // table of level pairs: entry e = (level[e & 15], level[e >> 4]); lane L
    // writes entries 4L .. 4L + 3 (the same high level, low levels 4(L & 3) + u)
    {
      const uint32_t hi = (uint32_t)__shfl((int)lv[i], lane >> 2, 64);
      uint32_t lo[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) lo[u] = (uint32_t)__shfl((int)lv[i], 4 * (lane & 3) + u, 64);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if constexpr (DT == HSS_BF16)
          tab[4 * lane + u] = (lo[u] & 0xffffu) | (hi << 16);
        else
          tab[4 * lane + u] = u32x2{lo[u], hi};
      }
    }
    float acc[BC];
#pragma unroll
    for (int c = 0; c < BC; ++c) acc[c] = 0.f;
    if (q.vec_codes) {
#pragma unroll
      for (int k = 0; k < kDqPre; ++k) {
        const int cq = lane + 64 * k;
        if (cq < nch) dq_chunk<DT, BC>(cpre[i][k], cq, min(16, nb - 16 * cq), tab, xs, n, bc, acc);
      }
      for (int cq = lane + 64 * kDqPre; cq < nch; cq += 64) {
        const u32x4 cw = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(q.codes + rowc * nb) + cq);
        dq_chunk<DT, BC>(cw, cq, min(16, nb - 16 * cq), tab, xs, n, bc, acc);
      }
    } else {
      // unaligned rows: bytes one at a time
      for (int cq = lane; cq < nch; cq += 64) {
        uint32_t w4[4] = {0u, 0u, 0u, 0u};
        const int valid = min(16, nb - 16 * cq);
        for (int b = 0; b < valid; ++b) w4[b >> 2] |= (uint32_t)q.codes[rowc * nb + 16 * cq + b] << (8 * (b & 3));
        dq_chunk<DT, BC>(u32x4{w4[0], w4[1], w4[2], w4[3]}, cq, valid, tab, xs, n, bc, acc);
      }
    }
#pragma unroll
    for (int c = 0; c < BC; ++c) {
      const float s = wave_sum(acc[c]) + ssum[i][c];
      if (row < m && c < bc && lane == c) {
        if constexpr (DT == HSS_F32)
          Y[(int64_t)c * m + row] = __float_as_uint(s);
        else
          Y[(int64_t)c * m + row] = f32_to_bf16(s);
      }
    }
  }
}

// Largest column count per dense-and-sparse pass whose staged X fits 96 KiB;
// one column when n % 8 != 0 (the 16-byte X reads of later columns would be
// misaligned).
int decode_dq_max_cols(const hss_matrix* A) {
  const size_t es = A->dtype == HSS_F32 ? 4 : 2;
  if (A->n % 8 != 0) return 1;
  for (int bc = 8; bc >= 1; bc /= 2)
    if (align16((size_t)bc * A->n * es) <= 96 * 1024) return bc;
  return 0;
}

template <int DT, int FMT, int BC, int RPW>
static void launch_dq_k(const DqArgs& q, unsigned grid, size_t lds, hipStream_t s) {
  static bool big_lds = false;
  if (lds > 64 * 1024 && !big_lds) {
    hipFuncSetAttribute(reinterpret_cast<const void*>(&k_decode_dq<DT, FMT, BC, RPW>),
                        hipFuncAttributeMaxDynamicSharedMemorySize, 112 * 1024);
    big_lds = true;
  }
  hipLaunchKernelGGL((k_decode_dq<DT, FMT, BC, RPW>), dim3(grid), dim3(256), lds, s, q);
}

template <int DT, int FMT, int BC>
static void launch_dq_rpw(const DqArgs& q, unsigned grid, int rpw, size_t lds, hipStream_t s) {
  if (rpw == 2) launch_dq_k<DT, FMT, BC, 2>(q, grid, lds, s);
  else launch_dq_k<DT, FMT, BC, 1>(q, grid, lds, s);
}

template <int DT, int FMT>
static void launch_dq_bc(const DqArgs& q, unsigned grid, int bc, int rpw, size_t lds, hipStream_t s) {
  if (bc == 1) launch_dq_rpw<DT, FMT, 1>(q, grid, rpw, lds, s);
  else if (bc == 2) launch_dq_rpw<DT, FMT, 2>(q, grid, rpw, lds, s);
  else if (bc <= 4) launch_dq_rpw<DT, FMT, 4>(q, grid, rpw, lds, s);
  else launch_dq_rpw<DT, FMT, 8>(q, grid, rpw, lds, s);
}

// One dense-and-sparse pass over bc (<= decode_dq_max_cols) columns.
void launch_decode_dq(const hss_matrix* A, int bc, const void* X, void* Y, hipStream_t s) {
  DqArgs q = {};
  DecodeArgs& a = q.a;
  const size_t es = A->dtype == HSS_F32 ? 4 : 2;
  a.m = A->m; a.n = A->n; a.r = 0; a.bc = bc;
  a.row_ptr = A->row_ptr; a.vals = A->values;
  a.col_idx = col16_of(A) ? nullptr : A->col_idx;
  a.col16 = col16_of(A) ? reinterpret_cast<const uint16_t*>(A->col_idx) : nullptr;
  a.X = X; a.Y = Y;
  a.nnz = A->nnz;
  a.x_lds = 1;
  a.vec = ((uintptr_t)X % 16 == 0) && ((size_t)A->n * es) % 16 == 0;
  a.vec_csr = A->nnz >= 4 && (uintptr_t)A->col_idx % (col16_of(A) ? 8 : 16) == 0 &&
              (uintptr_t)A->values % (4 * es) == 0;
  a.x_off = 0;
  q.codes = A->dq_codes;
  q.levels = A->dq_levels;
  q.vec_codes = A->n % 32 == 0 && (uintptr_t)A->dq_codes % 16 == 0;
  q.tab_off = (int)align16((size_t)bc * A->n * es);
  const size_t lds = (size_t)q.tab_off + 4 * 256 * (A->dtype == HSS_F32 ? 8 : 4);
  // two rows per wave pay off only with several columns (4096^2: b = 8 20.7
  // vs 22.6 us); one column runs faster with twice the waves (8.9 vs 8.4 us)
  const int rpw = A->m >= 2048 && bc > 1 ? 2 : 1;
  const unsigned grid = (unsigned)((A->m + 4 * rpw - 1) / (4 * rpw));
  const int fmt = col16_of(A) ? kFmtCsr16 : HSS_FMT_CSR;
  if (A->dtype == HSS_F32) {
    if (fmt == kFmtCsr16) launch_dq_bc<HSS_F32, kFmtCsr16>(q, grid, bc, rpw, lds, s);
    else launch_dq_bc<HSS_F32, HSS_FMT_CSR>(q, grid, bc, rpw, lds, s);
  } else {
    if (fmt == kFmtCsr16) launch_dq_bc<HSS_BF16, kFmtCsr16>(q, grid, bc, rpw, lds, s);
    else launch_dq_bc<HSS_BF16, HSS_FMT_CSR>(q, grid, bc, rpw, lds, s);
  }
}

}  // namespace hss
