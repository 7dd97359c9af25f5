// Instantiations of the MFMA GEMM kernel for F32 operands (one
// translation unit per operand type, so the kernels compile in parallel).
#include "gemm_kernel.h"

namespace ge {

void gemm_dispatch_f32(int layout, const Plan &pl, const GemmParams &gp, hipStream_t s) {
  launch_layout<float>(layout, pl, gp, s);
}

}  // namespace ge
