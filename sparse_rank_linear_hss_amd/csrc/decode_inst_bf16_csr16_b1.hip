// Instances of the fused decode kernel (bf16 CSR with 16-bit columns, one column per pass); the kernel is in decode_kernel.h.
#include "decode_kernel.h"

namespace hss {

void decode_launch_bf16_csr16_b1(const GroupArgs& ga, unsigned grid, int uq, bool fast, int mtr, int rpw, int cp,
                                 size_t lds, hipStream_t s) {
  launch_bc<HSS_BF16, kFmtCsr16, 1>(ga, grid, uq, fast, mtr, rpw, cp, lds, s);
}

}  // namespace hss
