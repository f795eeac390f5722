// 2:4 layers at 2..64 bf16 columns on gfx950's sparse matrix cores.
//
// [HASSLE] page aibr.jp/archives/82335, section "3.中核となる技術的要素": S
// kept in N:M (here 2:4) form, the structure GPUs accelerate.  [HSS] page
// "LLMの階層的スパース+低ランク圧縮", section "実装と運用パターン": the forward
// pass is the sparse product plus two small dense products through the
// factors.  Here, for b columns:
//
//   T = X V                  (b x r, bf16) k_spmm_prep's T blocks on the
//                                          vector units up to 16 columns,
//                                          k_nm_t on the matrix cores above
//   Y = X S^T + T U^T        (b x m)       k_nm_smfmac, one launch
//
// v_smfmac_f32_32x32x32_bf16 multiplies a 32 x 32 A held 2:4-compressed (16
// stored values and 16 index bits per row pair of lanes) by a dense 32 x 32 B.
// Its 2-bit indices have exactly the library's 2:4 metadata format (a group's
// first stored value at position nib & 3, the second at nib >> 2), so S's
// values and metadata words go to the matrix cores as stored: no expansion.
// Operand layout of the instruction (measured with one-hot and random
// inputs, every case bit-exact):
//   A  lane l: row l % 32; half h = l / 32.  Its 8 values are four groups of
//      two (group q: values 2q, 2q + 1), placed by nibble q of the index
//      word (bits 4q .. 4q + 3).  Group q of half h is the 4-wide K group
//      kappa = 2h + q for q < 2, 2h + q + 2 for q >= 2.
//   B  lane l: column l % 32; its 16 values are K = 16 (l / 32) .. + 15.
//   D  as v_mfma_f32_32x32x16_bf16: lane l value v is row 8 (v / 4) +
//      4 (l / 32) + v % 4, column l % 32.
// A 32-column chunk of S (one metadata word, 16 values per row) is one
// instruction: half h takes the chunk's groups 4h .. 4h + 3 (values 8h ..
// 8h + 7, the word's bits 16h .. 16h + 15).  Inverting kappa, B half hb then
// needs X columns 8 hb .. 8 hb + 7 and 16 + 8 hb .. 16 + 8 hb + 7 of the chunk.
//
// One block owns 64 rows (two 32-row tiles, so each X piece it reads from
// L2 serves both) and one 32-column tile of the batch; its 4 waves take the
// rows' 128-column stages in turn (wave w: stages w, w + 4, ...), two stages
// in flight per lane.  A stage's values are loaded row-contiguous (each load
// instruction covers 8 whole 128-byte row segments) and passed through the
// wave's own LDS area into the operand layout; X comes through a buffer
// resource (rows past b read as zeros).  The low-rank part T U^T runs on the
// dense v_mfma_f32_32x32x16_bf16 into the same accumulators (16 rank
// columns per step, steps dealt round robin to the waves).  The 4 partial
// tiles are added through LDS in wave order, so the result does not depend
// on scheduling.
#include "hss_internal.h"

namespace hss {

void launch_t_vec(const hss_matrix* A, int b, const void* X, int ldt, uint16_t* T, hipStream_t s);
int64_t prep_t_blocks(int r, int b);

typedef __bf16 nm_bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 nm_bf16x16 __attribute__((ext_vector_type(16)));
typedef float nm_f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t nm_u32x8 __attribute__((ext_vector_type(8)));

static constexpr int kNmBlockWaves = 4;         // waves (turns at the stages) per block
static constexpr int kNmStride = 36;            // LDS floats per column of a partial tile
static constexpr int kNmMinCols = 2, kNmMaxCols = 64;
// T on the vector units (k_spmm_prep's T blocks, one per rank row and pass
// of up to 16 columns, the passes side by side) while that takes at most
// kNmTVecMaxBlocks blocks, else on the matrix cores (k_nm_t).  On the
// 11008 x 4096 rank-64 layer the passes win at every batch: b = 2 .. 8
// 4.5 us against 7.0; whole calls at b = 32 / 48 / 64 27.0 / 37.8 / 41.6 us
// against 31.2 / 42.1 / 45.7.
static constexpr int kNmTVecMaxBlocks = 1024;
// 32-row tiles per block: X, read once per block from L2, serves 64 rows.
// Measured on the 11008 x 4096 layer (one tile vs two, us): b = 2 22.0 vs
// 20.2, b = 8 23.6 vs 21.4, b = 32 38.8 vs 31.3, b = 64 57.3 vs 45.6 (three
// tiles need 250 VGPRs: one wave per SIMD; 8 waves per block: 23.0 us at
// b = 8).
static constexpr int kNmRowTiles = 2;

static size_t align256_nm(size_t x) { return (x + 255) & ~(size_t)255; }

struct NmArgs {
  const uint16_t* X;       // b x n
  const uint16_t* vals;    // m x n/2: the two kept values of every group of 4
  const uint32_t* meta;    // m x n/32: 8 nibbles per word
  const uint16_t* U;       // m x r
  const uint16_t* T;       // b x tld (X V, bf16; columns r .. tld - 1 never read as values)
  uint16_t* Y;             // b x m
  int m, n, r, b, tld;
  int uvec;                // U rows 16-byte aligned (r % 8 == 0, U aligned)
  int nbx, nby;            // row blocks, 32-column batch tiles
};

// T's row stride: 16-byte rows.
static int nm_tld(int r) { return (r + 7) & ~7; }

// One stage of a lane: 4 chunks (128 columns) of its block's 32 RT rows.
// v: the rows' values loaded row-contiguous (for row tile t, lane l: row
// 32 t + 8 k + l / 8, bytes 16 (l % 8) .. of the stage's 128-byte row
// segment, k = 0..3), so each load instruction covers 8 whole 128-byte row
// segments; mw: the 4 metadata words of row 32 t + l % 32; x: the stage's
// 256-byte segments of the block's 32 X rows, loaded the same way (lane l:
// row 32 by + l / 16 + 4 j, bytes 16 (l % 16) ..).  (Loading X in the B
// operand's layout -- 16 bytes from each of 32 rows per instruction -- made
// every X load touch 32 cache lines: 17 us per block at b = 32 against 8.)
template <int RT>
struct NmStage {
  u32x4 v[RT][4];
  u32x4 mw[RT];
  u32x4 x[8];
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t nm_rsrc(const uint16_t* p, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p), 0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 nm_bload(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// Rows of a wave's staging area in LDS: 128 bytes + 16 of padding, so the
// operand reads (lane l: row l % 32) fall on distinct banks; X rows: 256 +
// 16 bytes for the same reason.
static constexpr int kNmRowBytes = 144;
static constexpr int kNmXRowBytes = 272;
static_assert(kNmRowBytes * 32 == 32 * kNmStride * 4, "staging area = the wave's reduction tile");

// Block (bx, by): rows 32 RT bx .. (RT tiles of 32), batch columns 32 by ..
// 32 by + 31.  WV waves take its 128-column stages in turn (wave w: stages
// w, w + WV, ...); D stages in flight per lane.
//
// The 1-D grid is dealt round robin to the 8 XCDs, so block id runs on XCD
// id % 8.  Blocks 8 q + j of one run of 8 nby ids (j < 8) are the nby batch
// tiles of row block 8 (q / nby) + j: all tiles of a row block run on one
// XCD at about the same time, and S, streamed by the first, is an L2 hit
// for the others instead of a second read from HBM.
template <int RT, int D, int WV>
__global__ __launch_bounds__(64 * WV) void k_nm_smfmac(NmArgs a) {
  constexpr int kNmWaves = WV, kNmThreads = 64 * WV;
  // Each wave's slice is its staging area during the main loop and its
  // partial tiles afterwards (only that wave touches it in between).
  __shared__ __align__(16) float red[kNmWaves][32 * RT][kNmStride];
  __shared__ __align__(16) char xsh[kNmWaves][32 * kNmXRowBytes];  // each wave's X segments
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int i = lane & 31, h = lane >> 5;
  const int xj = (int)blockIdx.x & 7, xq = (int)blockIdx.x >> 3;
  const int bx = 8 * (xq / a.nby) + xj, by = xq % a.nby;
  if (bx >= a.nbx) return;  // the grid is a whole number of runs
  const int row0 = bx * 32 * RT, c0 = by * 32;
  const int n = a.n, nst = n >> 7;         // 128-column stages (n % 128 == 0)
  const int per = (nst + kNmWaves - 1) / kNmWaves;  // stages per wave
  char* const stg = reinterpret_cast<char*>(&red[w][0][0]);
  int rows[RT];  // this lane's operand row of each tile (rows past m: a copy of row m - 1, never stored)
#pragma unroll
  for (int t = 0; t < RT; ++t) rows[t] = min(row0 + 32 * t + i, a.m - 1);

  nm_f32x16 acc[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) acc[t] = nm_f32x16{};

  // Low-rank part: step s covers rank columns 16 s .. 16 s + 15 (half h: 8 of
  // them).  Its loads go out first, so waiting for them waits for nothing else.
  // Rank columns past r are zeros on both sides.
  const int nus = (a.r + 15) >> 4;
  const __amdgpu_buffer_rsrc_t rtb = nm_rsrc(a.T, (int64_t)a.b * a.tld * 2);
  auto u_load = [&](int s, u32x4 (&ua)[RT], u32x4& ub) {
    const int col = 16 * s + 8 * h;
    const int nv = min(max(a.r - col, 0), 8);  // valid columns of this half step
    const int cc = nv > 0 ? col : 0;
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      const uint16_t* up = a.U + (int64_t)rows[t] * a.r + cc;
      if (a.uvec) {
        ua[t] = *reinterpret_cast<const u32x4*>(up);
      } else {
        uint32_t e[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) e[q] = up[q < nv ? q : 0];
        ua[t] = u32x4{e[0] | e[1] << 16, e[2] | e[3] << 16, e[4] | e[5] << 16, e[6] | e[7] << 16};
      }
    }
    ub = nm_bload(rtb, 2u * ((uint32_t)(c0 + i) * (uint32_t)a.tld + (uint32_t)cc));
    if (nv < 8) {
      uint32_t mk[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) mk[q] = (2 * q < nv ? 0xffffu : 0u) | (2 * q + 1 < nv ? 0xffff0000u : 0u);
      const u32x4 m4 = {mk[0], mk[1], mk[2], mk[3]};
#pragma unroll
      for (int t = 0; t < RT; ++t) ua[t] &= m4;
      ub &= m4;
    }
  };
  auto u_mma = [&](const u32x4 (&ua)[RT], const u32x4& ub) {
#pragma unroll
    for (int t = 0; t < RT; ++t)
      acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(nm_bf16x8, ua[t]),
                                                       __builtin_bit_cast(nm_bf16x8, ub), acc[t], 0, 0, 0);
  };
  u32x4 ua0[RT], ub0;
  if (w < nus) u_load(w, ua0, ub0);  // wave-uniform

  // Sparse part.
  const __amdgpu_buffer_rsrc_t rx = nm_rsrc(a.X, (int64_t)a.b * n * 2);
  const int vr = lane >> 3, vb = 16 * (lane & 7);  // coalesced value loads: row 8 k + vr, byte vb
  const char* __restrict__ vbase[RT][4];
  const uint32_t* __restrict__ mrow[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) {
#pragma unroll
    for (int k = 0; k < 4; ++k)
      vbase[t][k] = reinterpret_cast<const char*>(a.vals) + (int64_t)min(row0 + 32 * t + 8 * k + vr, a.m - 1) * n + vb;
    mrow[t] = a.meta + (int64_t)rows[t] * (n >> 5);
  }
  // X: lane l loads row c0 + l / 16 + 4 j, bytes 16 (l % 16) .. of each
  // stage's 256-byte row segment (rows past b read as zeros)
  const uint32_t xo = 2u * (uint32_t)(c0 + (lane >> 4)) * (uint32_t)n + 16u * (uint32_t)(lane & 15);
  const uint32_t xstep = 8u * (uint32_t)n;  // 4 rows
  char* const xs = &xsh[w][0];

  // Stage k of this wave (clamped into the matrix: loads are unconditional).
  auto issue = [&](NmStage<RT>& st, int k) {
    const int sg = min(w + kNmWaves * k, nst - 1);
#pragma unroll
    for (int t = 0; t < RT; ++t) {
#pragma unroll
      for (int q = 0; q < 4; ++q) st.v[t][q] = *reinterpret_cast<const u32x4*>(vbase[t][q] + 128 * (int64_t)sg);
      st.mw[t] = *reinterpret_cast<const u32x4*>(mrow[t] + 4 * sg);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) st.x[j] = nm_bload(rx, xo + 256u * (uint32_t)sg + xstep * (uint32_t)j);
  };
  auto consume = [&](const NmStage<RT>& st, bool ok) {
    // the stage's rows into the staging area, then each chunk's A operand
    // (row l % 32 of a tile, the chunk's values 8 h .. 8 h + 7) back out
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<u32x4*>(stg + (32 * t + 8 * q + vr) * kNmRowBytes + vb) = st.v[t][q];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      *reinterpret_cast<u32x4*>(xs + ((lane >> 4) + 4 * j) * kNmXRowBytes + 16 * (lane & 15)) = st.x[j];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      // B operand of chunk c: X row c0 + i, bytes 64 c + 16 h and 64 c + 32 + 16 h
      const u32x4 x0 = *reinterpret_cast<const u32x4*>(xs + i * kNmXRowBytes + 64 * c + 16 * h);
      const u32x4 x1 = *reinterpret_cast<const u32x4*>(xs + i * kNmXRowBytes + 64 * c + 32 + 16 * h);
      const nm_u32x8 bx = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const u32x4 z = {0u, 0u, 0u, 0u};
        u32x4 av = *reinterpret_cast<const u32x4*>(stg + (32 * t + i) * kNmRowBytes + 32 * c + 16 * h);
        av = ok ? av : z;  // a stage past the range adds zeros
        const uint32_t mwv[4] = {st.mw[t].x, st.mw[t].y, st.mw[t].z, st.mw[t].w};
        const int idx = (int)(mwv[c] >> (16 * h));
        acc[t] = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(__builtin_bit_cast(nm_bf16x8, av),
                                                           __builtin_bit_cast(nm_bf16x16, bx), acc[t], idx, 0, 0);
      }
    }
  };

  NmStage<RT> st[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    issue(st[d], d);
    __builtin_amdgcn_sched_barrier(0);  // the loop's order, stage by stage
  }
  if (w < nus) u_mma(ua0, ub0);
  for (int k0 = 0; k0 < per; k0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int k = k0 + d;
      consume(st[d], k < per && w + kNmWaves * k < nst);
      issue(st[d], k + D);
      // keep each stage's loads right after its use: grouped at the loop's
      // end they would all be waited for at its start
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // further low-rank steps (r > 16 * waves)
  for (int s = w + kNmWaves; s < nus; s += kNmWaves) {
    u32x4 ua[RT], ub;
    u_load(s, ua, ub);
    u_mma(ua, ub);
  }

  // Partial tiles added in wave order; column c0 + cc to Y[c0 + cc][row0 ..].
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float4 q = {acc[t][4 * g], acc[t][4 * g + 1], acc[t][4 * g + 2], acc[t][4 * g + 3]};
      *reinterpret_cast<float4*>(&red[w][32 * t + i][8 * g + 4 * h]) = q;
    }
  __syncthreads();
  const int rr = threadIdx.x & 31;
#pragma unroll
  for (int t = 0; t < RT; ++t)
    for (int cc = threadIdx.x >> 5; cc < 32; cc += kNmThreads / 32) {
      float sum = red[0][32 * t + cc][rr];
#pragma unroll
      for (int ww = 1; ww < kNmWaves; ++ww) sum += red[ww][32 * t + cc][rr];
      const int c = c0 + cc, row = row0 + 32 * t + rr;
      if (c < a.b && row < a.m) a.Y[(int64_t)c * a.m + row] = f32_to_bf16(sum);
    }
}

// T = X V for this route on the matrix cores, one block per 16 x 16 tile of
// T (rank rows 16 lt .., batch rows 16 ct ..): its 16 waves split the n
// columns into 16 ranges, each a chain of v_mfma_f32_16x16x32_bf16 (A: V^T
// rows, B: X rows, all of a wave's loads in flight at once), and the 16
// partial tiles are added through LDS in wave order and rounded once to bf16.
static constexpr int kNmTWaves = 16;
static constexpr int kNmTSteps = 8;      // 32-column steps per wave per batch of loads

typedef float nm_f32x4 __attribute__((ext_vector_type(4)));

struct NmTArgs {
  const uint16_t* X;    // b x n
  const uint16_t* Vt;   // r x n
  uint16_t* T;          // (X V)[c][l] at T[c * sc + l * sl]
  int n, r, b, sc, sl;
  int kw;               // columns per wave (a multiple of 32)
};

// Operand layout of v_mfma_f32_16x16x32_bf16: A lane l holds row l % 16, K
// 8 (l / 16) .. + 7 of each 32; B lane l column l % 16, the same K; D lane l
// holds rows 4 (l / 16) .. + 3 of column l % 16.
__global__ __launch_bounds__(64 * kNmTWaves) void k_nm_t(NmTArgs a) {
  __shared__ float tred[kNmTWaves][16][17];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int lt = blockIdx.x, ct = blockIdx.y;
  const __amdgpu_buffer_rsrc_t rv = nm_rsrc(a.Vt, (int64_t)a.r * a.n * 2);
  const __amdgpu_buffer_rsrc_t rx = nm_rsrc(a.X, (int64_t)a.b * a.n * 2);
  const uint32_t ko = 8u * (uint32_t)(lane >> 4);
  const uint32_t ao = 2u * ((uint32_t)(16 * lt + (lane & 15)) * (uint32_t)a.n + ko);  // rows past r read zeros
  const uint32_t bo = 2u * ((uint32_t)(16 * ct + (lane & 15)) * (uint32_t)a.n + ko);  // rows past b read zeros
  nm_f32x4 acc = {};
  for (int kb = w * a.kw; kb < (w + 1) * a.kw; kb += 32 * kNmTSteps) {  // wave-uniform
    u32x4 av[kNmTSteps], bv[kNmTSteps];
#pragma unroll
    for (int q = 0; q < kNmTSteps; ++q) {
      const int k = min(kb + 32 * q, a.n - 32);  // clamped; steps past n are dropped below
      av[q] = nm_bload(rv, ao + 2u * (uint32_t)k);
      bv[q] = nm_bload(rx, bo + 2u * (uint32_t)k);
    }
#pragma unroll
    for (int q = 0; q < kNmTSteps; ++q)
      if (kb + 32 * q < a.n && kb + 32 * q < (w + 1) * a.kw)  // wave-uniform
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(nm_bf16x8, av[q]),
                                                      __builtin_bit_cast(nm_bf16x8, bv[q]), acc, 0, 0, 0);
  }
  // acc[v] = D[l = 4 (lane / 16) + v][c = lane % 16]
#pragma unroll
  for (int v = 0; v < 4; ++v) tred[w][lane & 15][4 * (lane >> 4) + v] = acc[v];
  __syncthreads();
  if (threadIdx.x < 256) {
    const int c = threadIdx.x >> 4, l = threadIdx.x & 15;
    float sum = tred[0][c][l];
#pragma unroll
    for (int ww = 1; ww < kNmTWaves; ++ww) sum += tred[ww][c][l];
    const int cg = 16 * ct + c, lg = 16 * lt + l;
    if (cg < a.b && lg < a.r) a.T[(int64_t)cg * a.sc + (int64_t)lg * a.sl] = f32_to_bf16(sum);
  }
}

// T = X V on the matrix cores (k_nm_t) at T[c * sc + l * sl].  Needs n % 32
// == 0 and 16-byte aligned X and V^T rows (t_mfma_supported), bf16, r > 0.
bool t_mfma_supported(const hss_matrix* A, const void* X) {
  return A->dtype == HSS_BF16 && A->r > 0 && A->n % 32 == 0 && (uintptr_t)X % 16 == 0 &&
         (uintptr_t)A->Vt % 16 == 0 && (int64_t)A->r * A->n * 2 < ((int64_t)1 << 31);
}

void launch_t_mfma(const hss_matrix* A, int b, const void* X, uint16_t* T, int sl, int sc, hipStream_t s) {
  NmTArgs t = {};
  t.X = static_cast<const uint16_t*>(X);
  t.Vt = static_cast<const uint16_t*>(A->Vt);
  t.T = T;
  t.n = A->n; t.r = A->r; t.b = b; t.sc = sc; t.sl = sl;
  t.kw = (A->n / 32 + kNmTWaves - 1) / kNmTWaves * 32;
  const dim3 grid((unsigned)((A->r + 15) / 16), (unsigned)((b + 15) / 16));
  hipLaunchKernelGGL(k_nm_t, grid, dim3(64 * kNmTWaves), 0, s, t);
}

bool nm_mma_supported(const hss_matrix* A, int b) {
  if (A->flags & HSS_DQ4) return false;
  if (A->fmt != HSS_FMT_2OF4 || A->dtype != HSS_BF16) return false;
  if (b < kNmMinCols || b > kNmMaxCols) return false;
  if (A->n % 128 != 0 || (uintptr_t)A->nm_values % 16 || (uintptr_t)A->nm_meta % 16) return false;
  if ((int64_t)A->n * 64 * 2 >= ((int64_t)1 << 31)) return false;          // X offsets of 64 rows (32-bit)
  if ((int64_t)nm_tld(A->r) * 64 * 2 >= ((int64_t)1 << 31)) return false;  // T offsets
  if ((int64_t)A->r * A->n * 2 >= ((int64_t)1 << 31)) return false;         // V^T offsets
  return true;
}

// Scratch: T (bf16).
size_t nm_mma_ws_bytes(const hss_matrix* A, int b) {
  return A->r > 0 ? align256_nm(sizeof(uint16_t) * (size_t)b * nm_tld(A->r)) : 0;
}

template <int RT>
static void launch_nm_rt(NmArgs a, hipStream_t s) {
  a.nbx = (a.m + 32 * RT - 1) / (32 * RT);
  a.nby = (a.b + 31) / 32;
  const unsigned grid = (unsigned)((a.nbx + 7) / 8 * 8 * a.nby);
  hipLaunchKernelGGL((k_nm_smfmac<RT, 2, kNmBlockWaves>), dim3(grid), dim3(64 * kNmBlockWaves), 0, s, a);
}

// X must be 16-byte aligned (the caller routes other X elsewhere).
hss_status launch_nm_mma(const hss_matrix* A, int b, const void* X, void* Y, void* ws, hipStream_t s) {
  NmArgs a = {};
  a.X = static_cast<const uint16_t*>(X);
  a.vals = static_cast<const uint16_t*>(A->nm_values);
  a.meta = A->nm_meta;
  a.U = static_cast<const uint16_t*>(A->U);
  a.T = static_cast<const uint16_t*>(ws);
  a.Y = static_cast<uint16_t*>(Y);
  a.m = A->m; a.n = A->n; a.r = A->r; a.b = b; a.tld = nm_tld(A->r);
  a.uvec = A->r % 8 == 0 && (uintptr_t)A->U % 16 == 0;
  if (A->r > 0 && (prep_t_blocks(A->r, b) <= kNmTVecMaxBlocks || !t_mfma_supported(A, X))) {
    launch_t_vec(A, b, X, a.tld, static_cast<uint16_t*>(ws), s);
  } else if (A->r > 0) {
    launch_t_mfma(A, b, X, static_cast<uint16_t*>(ws), 1, a.tld, s);
  }
  launch_nm_rt<kNmRowTiles>(a, s);
  return hipGetLastError() == hipSuccess ? HSS_OK : HSS_ERR_HIP;
}

}  // namespace hss
