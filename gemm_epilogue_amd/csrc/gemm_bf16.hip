// Instantiations of the MFMA GEMM kernel for BF16 operands (one
// translation unit per operand type, so the kernels compile in parallel).
#include "gemm_kernel.h"

namespace ge {

void gemm_dispatch_bf16(int layout, const Plan &pl, const GemmParams &gp, hipStream_t s) {
  launch_layout<bf16_t>(layout, pl, gp, s);
}

}  // namespace ge
