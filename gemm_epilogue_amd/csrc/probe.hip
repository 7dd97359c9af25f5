// Measurement helper: the shader clock under matrix-core load.  Every wave
// runs a chain of independent 32x32x16 MFMAs; lane 0 of each block records
// the shader-clock counter (s_memtime) and the constant 100 MHz reference
// counter (s_memrealtime) around the chain.  Their ratio is the clock the
// MFMA-bound kernels actually run at, which the dense peak assumes is the
// nominal one.
#include "common.h"

namespace ge {

__global__ __launch_bounds__(256) void clock_probe_kernel(int64_t *__restrict__ out, int iters, float seed) {
  f16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (half_t)(seed * (threadIdx.x + i));
    b[i] = (half_t)(seed * i);
  }
  f32x16 acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[i][e] = 0.f;
  const int64_t c0 = __builtin_amdgcn_s_memtime();
  const int64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[i], 0, 0, 0);
  }
  const int64_t c1 = __builtin_amdgcn_s_memtime();
  const int64_t r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += acc[i][0];
  if (threadIdx.x == 0) {
    out[3 * blockIdx.x] = c1 - c0;
    out[3 * blockIdx.x + 1] = r1 - r0;
    out[3 * blockIdx.x + 2] = (int64_t)(s != s);  // keeps the chain live
  }
}

}  // namespace ge

using namespace ge;

extern "C" int ge_clock_probe(int64_t *ticks, int32_t blocks, int32_t iters, ge_stream_t stream) {
  if (ticks == nullptr || blocks < 1 || blocks > 65536 || iters < 1) {
    set_error("ge_clock_probe: ticks NULL, blocks outside [1, 65536] or iters < 1");
    return GE_E_INVALID;
  }
  hipLaunchKernelGGL(clock_probe_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, ticks, iters, 1e-3f);
  return launch_status("ge_clock_probe");
}
