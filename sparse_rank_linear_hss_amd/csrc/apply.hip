// hss_apply dispatch: Y = X S^T + (X V) U^T.
//
// [HSS] page "LLMの階層的スパース+低ランク圧縮", section "実装と運用パターン": the
// forward pass of the compressed layer is the sparse product plus two small
// dense products through the factors.
//
// Paths:
//   decode (decode.hip)  up to 8 columns per launch: one fused kernel that
//                        streams S, U and V^T once (HBM-bound regime); fp32
//                        and narrow batches.
//   mfma (mfma.hip)      bf16 with b >= 16: the low-rank products are dense
//                        contractions and run on the matrix cores, with S
//                        densified chunk by chunk into the same GEMM.
#include "hss_internal.h"

namespace hss {

void launch_decode(const hss_matrix* A, int bc, const void* X, void* Y, void* ws, hipStream_t s);
size_t decode_ctl_bytes();
size_t decode_t_bytes(const hss_matrix* A);
int decode_max_cols(const hss_matrix* A);

static constexpr int kDecodeCols = 8;

bool mfma_supported(const hss_matrix* A, int b);
size_t mfma_ws_bytes(const hss_matrix* A, int b);
hss_status launch_mfma(const hss_matrix* A, int b, const void* X, void* Y, void* ws, hipStream_t s);

// Layout: [decode control region | decode T words or MFMA buffers].  The
// control region persists between calls; everything after it is per-call
// scratch, so both paths can share one workspace.
size_t apply_ws_bytes(const hss_matrix* A, int b) {
  const size_t dec = decode_t_bytes(A);
  const size_t mf = mfma_supported(A, b) ? mfma_ws_bytes(A, b) : 0;
  return decode_ctl_bytes() + (dec > mf ? dec : mf);
}

hss_status launch_apply(const hss_matrix* A, int b, const void* X, void* Y, void* ws,
                        hipStream_t stream) {
  if (mfma_supported(A, b))
    return launch_mfma(A, b, X, Y, static_cast<char*>(ws) + decode_ctl_bytes(), stream);
  const size_t es = A->dtype == HSS_F32 ? 4 : 2;
  const int cols = decode_max_cols(A);
  if (cols == 0) return HSS_ERR_UNSUPPORTED;
  for (int c0 = 0; c0 < b; c0 += cols) {
    const int bc = b - c0 < cols ? b - c0 : cols;
    launch_decode(A, bc, static_cast<const char*>(X) + (size_t)c0 * A->n * es,
                  static_cast<char*>(Y) + (size_t)c0 * A->m * es, ws, stream);
  }
  return hipGetLastError() == hipSuccess ? HSS_OK : HSS_ERR_HIP;
}

}  // namespace hss
