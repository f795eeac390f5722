// Host side of the fused small-batch apply (kernel in decode_kernel.h): launch
// planning for single and grouped calls, and the dense-and-sparse kernel.
#include "decode_kernel.h"

namespace hss {

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

// HSS_OPT_DECODE_MERGED = 0 keeps separate producer blocks (a diagnostic switch).
static bool merged_enabled() { return option(HSS_OPT_DECODE_MERGED) != 0; }

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
static constexpr size_t kMaskTabBytes = 256 * 16;  // u_epilogue's mask table (bf16 U pieces)

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
    const size_t tb = align16(sizeof(float) * (size_t)bc * t_ld2(A->r)) + kMaskTabBytes +
                      align16(4 * (size_t)((A->r + 31) / 32));
    if (tb <= max_lds(A)) return bc;
  }
  return 0;
}

// Polls of a stale T word before the row is computed locally; -1 when every
// block is to compute every T row itself (HSS_OPT_DECODE_FORCE_LOCAL).
static int spin_limit() {
  return option(HSS_OPT_DECODE_FORCE_LOCAL) ? -1 : option(HSS_OPT_DECODE_SPIN);
}

// Arguments of one matrix of a decode pass, and the per-matrix launch
// properties the group has to agree on.
struct MatrixLaunch {
  DecodeArgs a;
  size_t lds;
  int uq;  // U pieces per lane and row (0: element-wise U reads)
  int cp;  // CSR chunks per row loaded up front
  bool fast;
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
  const bool hier = (A->flags & HSS_HIER2) != 0;
  if (hier) {  // the 2 x 2 block-structured low-rank term in compact form
    a.ru = A->hier_r[0] + A->hier_r[1];
    a.v_ld = hier_vt_ld(A->n);
    a.h_m0 = A->m / 2;
    a.h_toff = a.ru;
    a.h_n0 = A->n / 2;
    a.h_l1 = A->hier_r[0];
    a.h_l2 = A->hier_r[0] + A->hier_r[1];
    a.h_l3 = a.h_l2 + A->hier_r[2];
  } else {
    a.ru = A->r;
    a.v_ld = A->n;
    a.h_m0 = A->m;
    a.h_toff = 0;
    a.h_n0 = A->n;
    a.h_l1 = a.h_l2 = a.h_l3 = A->r;
  }

  const size_t es = A->dtype == HSS_F32 ? 4 : 2;
  // bf16 U rows as aligned 16-byte pieces (any r): one piece per lane covers
  // r <= 506, two r <= 1018 (and give the same bits there as one would).
  L.uq = (A->dtype == HSS_BF16 && a.ru > 0 && (uintptr_t)A->U % 16 == 0) ? (a.ru <= 506 ? 1 : 2) : 0;
  // T: fp32, or bf16 in two copies (the same bytes, see t_ld2), plus the
  // pieces' mask table
  const size_t tbytes = align16(sizeof(float) * (size_t)bc * t_ld2(A->r)) + (L.uq > 0 ? kMaskTabBytes : 0);
  const size_t mbytes = align16(4 * (size_t)((A->r + 31) / 32));
  const bool nm_fast = A->fmt == HSS_FMT_2OF4 && A->dtype == HSS_BF16 && ((uintptr_t)X % 16 == 0) &&
                       A->n % 32 == 0 && (uintptr_t)A->nm_values % 16 == 0 && (uintptr_t)A->nm_meta % 4 == 0 &&
                       (A->r == 0 || (uintptr_t)A->Vt % 16 == 0);
  // the 2:4 fast path reads 64-byte X chunks at a 64-byte lane stride: pad them
  const size_t xbytes = align16((size_t)bc * A->n * es * (nm_fast ? 5 : 4) / 4);
  a.t_off = 0;
  a.mtab_off = (int)(tbytes - (L.uq > 0 ? kMaskTabBytes : 0));
  a.miss_off = (int)tbytes;
  a.x_off = (int)(tbytes + mbytes);
  a.x_lds = tbytes + mbytes + xbytes <= max_lds(A);
  a.x_pad = nm_fast && a.x_lds;
  // Vector dot products: X rows and Vt rows start 16-byte aligned.
  a.vec = ((uintptr_t)X % 16 == 0) && ((size_t)A->n * es) % 16 == 0 &&
          (A->r == 0 || (uintptr_t)A->Vt % 16 == 0) && ((size_t)a.v_ld * es) % 16 == 0 &&
          ((size_t)a.h_n0 * es) % 16 == 0;
  a.vec_csr = A->fmt == HSS_FMT_CSR && A->nnz >= 4 && (uintptr_t)A->col_idx % (col16_of(A) ? 8 : 16) == 0 &&
              (uintptr_t)A->values % (4 * es) == 0;
  a.nm_fast = A->fmt == HSS_FMT_2OF4 && A->dtype == HSS_BF16 && a.vec && A->n % 32 == 0 &&
              (uintptr_t)A->nm_values % 16 == 0 && (uintptr_t)A->nm_meta % 4 == 0;
  L.lds = tbytes + mbytes + (a.x_lds ? xbytes : 0);
  L.fast = A->dtype == HSS_BF16 && A->r > 0 && a.x_lds && a.vec &&
           (A->fmt == HSS_FMT_CSR ? a.vec_csr : a.nm_fast);
  // Rows averaging more than 192 entries (the 4096 x 11008 down projection
  // at 3 %: 330) load their second 256-entry chunk up front as well.
  L.cp = A->fmt == HSS_FMT_CSR && A->nnz > 192 * (int64_t)A->m ? 2 : 1;
  // Rows per wave: more rows per block means fewer copies of X staged through
  // L2 into LDS and fewer blocks queueing loads on each CU (measured best:
  // 4 for one column from 2048 rows -- the decoder layer's q/k/v launch 13.0
  // against 14.0 us with 2 -- and 4 for 11008 rows, 2 for 4096 rows at more
  // columns); small matrices keep one row per wave for parallelism.  Four
  // rows per wave exist only as FAST instances.
  L.rpw = A->m >= 8192 ? 4 : (A->m >= 2048 ? (bc == 1 ? 4 : 2) : 1);
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
  for (int g = 0; g < G; ++g)
    if (A[g]->n / 8 > kMergedThreads) return 0;  // a block's threads hold X one 16-byte vector each
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
  int uq = -1;  // the group's: 0 if any matrix needs element-wise U reads, else the largest
  int cp = 1;
  bool fast = true;
  int rpw = 4;
  MatrixLaunch L[kMaxGroup];
  for (int g = 0; g < G; ++g) {
    L[g] = matrix_launch(A[g], bc, X, Y[g], ctl, reinterpret_cast<uint64_t*>(tw));
    tw += decode_t_bytes(A[g]);
    lds = lds > L[g].lds ? lds : L[g].lds;
    uq = (L[g].uq == 0 || uq == 0) ? 0 : (uq > L[g].uq ? uq : L[g].uq);
    cp = cp > L[g].cp ? cp : L[g].cp;
    fast = fast && L[g].fast;
    rpw = rpw < L[g].rpw ? rpw : L[g].rpw;
  }
  if (option(HSS_OPT_DECODE_RPW) > 0) rpw = option(HSS_OPT_DECODE_RPW);
  if (!fast && rpw > 2) rpw = 2;
  const int dt = A[0]->dtype, fmt = col16_of(A[0]) ? kFmtCsr16 : A[0]->fmt;
  if (uq < 0) uq = 0;
  const int mtr = merged_plan(A, G, bc, fast && dt == HSS_BF16 && uq > 0, fmt, rpw);
  const bool merged = mtr > 0;
  // Wave producers (one bf16 column on the FAST path, X of at most 4096
  // elements): one T row per wave, four per block.  The q/k/v launch of the
  // decoder layer then has 309 producer blocks instead of 1,227, and its
  // producers and row blocks all fit on the CUs at once.
  bool wave_prod = !merged && bc == 1 && fast && dt == HSS_BF16 && option(HSS_OPT_DECODE_WAVE_PRODUCERS) != 0;
  for (int g = 0; g < G; ++g) wave_prod = wave_prod && (size_t)A[g]->n * 2 <= 2 * 256 * 16;
  ga.prod_rows = wave_prod ? 4 : 1;
  ga.prod_start[0] = 0;
  for (int g = 0; g < G; ++g) {
    ga.a[g] = L[g].a;
    ga.prod_start[g + 1] = ga.prod_start[g] + (merged ? 0 : (A[g]->r + ga.prod_rows - 1) / ga.prod_rows);
  }
  ga.row_start[0] = ga.prod_start[G];
  const int rows_per_block = (merged ? kMergedThreads / 64 : 4) * rpw;
  for (int g = 0; g < G; ++g) ga.row_start[g + 1] = ga.row_start[g] + (A[g]->m + rows_per_block - 1) / rows_per_block;
  for (int g = G; g < kMaxGroup; ++g) { ga.prod_start[g + 1] = ga.prod_start[G]; ga.row_start[g + 1] = ga.row_start[G]; }
  const unsigned grid = (unsigned)ga.row_start[G];
  if (dt == HSS_F32) {
    decode_launch_f32(ga, grid, fmt, bc, rpw, lds, s);
  } else {
    if (fmt == HSS_FMT_CSR) {
      if (bc == 1) decode_launch_bf16_csr_b1(ga, grid, uq, fast, mtr, rpw, cp, lds, s);
      else decode_launch_bf16_csr_bn(ga, grid, bc, uq, fast, rpw, lds, s);
    } else if (fmt == kFmtCsr16) {
      if (bc == 1) decode_launch_bf16_csr16_b1(ga, grid, uq, fast, mtr, rpw, cp, lds, s);
      else decode_launch_bf16_csr16_bn(ga, grid, bc, uq, fast, rpw, lds, s);
    } else {
      decode_launch_bf16_nm(ga, grid, bc, uq, fast, rpw, lds, s);
    }
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
      const float s = wave_sum(acc[c] + ssum[i][c]);  // the dense part's and the outliers' lane shares
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
