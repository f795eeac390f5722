// hss_apply_noalloc: hss_apply with the library's own device scratch instead
// of a caller workspace, for callers that cannot allocate device memory.
//
// The scratch is one file-scope device array per GPU (kScratchBytes, held
// until the process ends).  In host code the array's name is only a host-side
// stand-in, so its device address is looked up once per device with
// hipGetSymbolAddress (with that device current) and only that address is
// passed on.  The first call on a device also clears the whole array with the
// zero-fill kernel, on that call's stream: the fused decode kernel keeps its
// call epoch, arrival counters and tagged T words in the first bytes and needs
// them to start from zeros.  Later calls keep the state the previous call
// left, as the decode kernel expects.  Every call on one GPU shares the array:
// calls that overlap in time on one GPU race and may return wrong values.
#include <mutex>

#include "hss_internal.h"

namespace hss {

static constexpr size_t kScratchBytes = (size_t)16 << 20;  // 16 MiB per GPU
static constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};  // device address of `scratch` on each device, once looked up

// The device address of this device's scratch; clears it on the first call
// (on `stream`).  nullptr (and *st set) if the lookup or the clear fails.
void* device_scratch(hipStream_t stream, hss_status* st) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *st = HSS_ERR_HIP;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      *st = HSS_ERR_HIP;
      return nullptr;
    }
    if (launch_zero_fill(p, kScratchBytes, stream) != HSS_OK) {
      *st = HSS_ERR_HIP;
      return nullptr;
    }
    g_ptr[dev] = p;
  }
  *st = HSS_OK;
  return g_ptr[dev];
}
}  // namespace

}  // namespace hss

extern "C" size_t hss_noalloc_scratch_bytes(void) { return hss::kScratchBytes; }

extern "C" hss_status hss_apply_noalloc(const hss_matrix* A, int32_t b, const void* X, void* Y,
                                        hipStream_t stream) {
  const hss_status st = hss::check_apply_args(A, b, X, Y);
  if (st != HSS_OK) return st;
  if (hss::apply_route_ws_bytes(A, b, X) > hss::kScratchBytes) return HSS_ERR_WORKSPACE;
  hss_status sst = HSS_OK;
  void* ws = hss::device_scratch(stream, &sst);
  if (!ws) return sst;
  return hss::launch_apply(A, b, X, Y, ws, stream);
}
