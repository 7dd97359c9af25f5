// Instantiations of the MFMA GEMM kernel for F16 operands (one
// translation unit per operand type, so the kernels compile in parallel).
#include "gemm_kernel.h"

namespace ge {

void gemm_dispatch_f16(int layout, const Plan &pl, const GemmParams &gp, hipStream_t s) {
  launch_layout<half_t>(layout, pl, gp, s);
}

}  // namespace ge
