// Instances of the fused decode kernel (fp32, every format); the kernel is in decode_kernel.h.
#include "decode_kernel.h"

namespace hss {

void decode_launch_f32(const GroupArgs& ga, unsigned grid, int fmt, int bc, int rpw, size_t lds, hipStream_t s) {
  if (fmt == HSS_FMT_CSR) launch_fmt<HSS_F32, HSS_FMT_CSR>(ga, grid, bc, 0, false, 0, rpw, lds, s);
  else if (fmt == kFmtCsr16) launch_fmt<HSS_F32, kFmtCsr16>(ga, grid, bc, 0, false, 0, rpw, lds, s);
  else launch_fmt<HSS_F32, HSS_FMT_2OF4>(ga, grid, bc, 0, false, 0, rpw, lds, s);
}

}  // namespace hss
