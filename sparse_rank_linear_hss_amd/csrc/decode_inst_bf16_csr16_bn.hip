// Instances of the fused decode kernel (bf16 CSR with 16-bit columns, 2 to 8 columns per pass); the kernel is in decode_kernel.h.
#include "decode_kernel.h"

namespace hss {

void decode_launch_bf16_csr16_bn(const GroupArgs& ga, unsigned grid, int bc, int uq, bool fast, int rpw,
                                 size_t lds, hipStream_t s) {
  launch_fmt<HSS_BF16, kFmtCsr16>(ga, grid, bc, uq, fast, 0, rpw, lds, s);
}

}  // namespace hss
