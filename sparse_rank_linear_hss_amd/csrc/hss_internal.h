// Internal helpers shared by the HSS kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hss.h"

#define HSS_WAVE 64

namespace hss {

// Row length of the compact V^T of an HSS_HIER2 matrix: the wider column half.
__host__ __device__ inline int hier_vt_ld(int n) { return n - n / 2; }

// Native 16-byte vector (usable with the nontemporal load/store builtins).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Storage types.  Weights/activations travel as raw bits: uint32_t for fp32,
// uint16_t for bf16.  Arithmetic is always fp32.
// ---------------------------------------------------------------------------
template <int DT> struct Elem;
template <> struct Elem<HSS_F32> {
  using bits_t = uint32_t;
  static constexpr uint32_t key_mask = 0x7fffffffu;  // |w| as an unsigned order
  static constexpr uint32_t key_inf = 0x7f800000u;   // keys >= this: Inf / NaN
  static constexpr int key_bits = 31;
  __device__ __forceinline__ static float to_f(uint32_t b) { return __uint_as_float(b); }
};
template <> struct Elem<HSS_BF16> {
  using bits_t = uint16_t;
  static constexpr uint32_t key_mask = 0x7fffu;
  static constexpr uint32_t key_inf = 0x7f80u;
  static constexpr int key_bits = 15;
  __device__ __forceinline__ static float to_f(uint32_t b) { return __uint_as_float(b << 16); }
};

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16, round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// ---------------------------------------------------------------------------
// Wave-level helpers (64 lanes).
// ---------------------------------------------------------------------------
__device__ __forceinline__ int lane_id() { return __lane_id(); }

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over the 64 lanes, returned wave-uniform.  Must be called with every
// lane active.  Within each row of 16 lanes four DPP steps (quad swaps, half-
// row mirror, row mirror) leave the row's sum in all 16 lanes -- both lanes of
// each exchange add the same two values, so all lanes hold the same bits --
// and the four row sums are read out and added in a fixed order.
// Deterministic; ~5x cheaper than LDS-permute butterflies.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_f<0x141>(v);  // row_half_mirror
  v += dpp_f<0x140>(v);  // row_mirror
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (r0 + r1) + (r2 + r3);
}

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, HSS_WAVE);
  return v;
}

// Exclusive prefix sum across the wave's lanes.
__device__ __forceinline__ uint32_t wave_excl_scan_u32(uint32_t v) {
  const int lane = lane_id();
  uint32_t incl = v;
#pragma unroll
  for (int off = 1; off < HSS_WAVE; off <<= 1) {
    uint32_t t = __shfl_up(incl, off, HSS_WAVE);
    if (lane >= off) incl += t;
  }
  return incl - v;
}

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = lane_id();
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

template <typename T>
__device__ __forceinline__ T uniform(T v) {
  return (T)__builtin_amdgcn_readfirstlane((int)v);
}

}  // namespace hss

// Host-side launchers (defined in the .hip files).
namespace hss {
// Process-wide diagnostic switches (hss_set_option); the environment gives
// their first values, read once.  Cheap to call on every apply.
int option(int opt);
hss_status launch_zero_fill(void* p, size_t bytes, hipStream_t s);

hss_status launch_split_csr(int dt, int m, int n, const void* W, int64_t k, int32_t* row_ptr,
                            int32_t* col_idx, void* values, void* residual, void* ws,
                            hipStream_t stream);
hss_status launch_split_24(int dt, int m, int n, const void* W, void* nm_values, uint32_t* nm_meta,
                           void* residual, void* ws, hipStream_t stream);
size_t split_ws_bytes(int fmt, int m);

size_t apply_ws_bytes(const hss_matrix* A, int b);
size_t apply_route_ws_bytes(const hss_matrix* A, int b, const void* X);
hss_status check_apply_args(const hss_matrix* A, int32_t b, const void* X, void* Y);
hss_status launch_apply(const hss_matrix* A, int b, const void* X, void* Y, void* ws,
                        hipStream_t stream);
size_t apply_group_ws_bytes(const hss_matrix* const* A, int G, int b);
hss_status launch_cols_to_u16(const int32_t* col_idx, int64_t nnz, uint16_t* out, hipStream_t stream);
hss_status launch_apply_group(const hss_matrix* const* A, int G, int b, const void* X, void* const* Y, void* ws,
                              hipStream_t stream);
hss_status rcm_order_host(int n, const int32_t* row_ptr, const int32_t* col_idx, int32_t* perm);
size_t concentration_ws_bytes(int n);
hss_status launch_concentration(int dt, int m, int n, const void* W, const int32_t* perm, double* out, void* ws,
                                hipStream_t s);
hss_status launch_hier_pack(int dt, int m, int n, const int32_t* r, const void* const* U, const void* const* Vt,
                            const int32_t* perm, void* Ucat, void* Vtcat, hipStream_t s);
hss_status launch_hier_pack_compact(int dt, int m, int n, const int32_t* r, const void* const* U,
                                    const void* const* Vt, void* Uc, void* Vtc, hipStream_t s);
hss_status launch_hier_expand(const hss_matrix* A, void* Uf, void* Vtf, hipStream_t s);
hss_status csr_permute_host(int n, const int32_t* row_ptr, const int32_t* col_idx, const int32_t* perm,
                            const int32_t* pos, int32_t* row_ptr_p, int32_t* col_idx_p, int32_t* from);
}  // namespace hss
