// Bit-exact mode of the primitives: every result is the fixed sequence of
// IEEE binary32 operations the library documents, each rounded to nearest
// even, no fused multiply-add, every sum in linear order (first term first),
// divide and square root correctly rounded.  This is the precision recipe of
// "HIP + Vulkan backends -- Phase 3" ("Phase-3 bug hunt": a linear-order sum
// in place of the hardware reduction tree, a correctly rounded divide, a
// refined rsqrt -- here a correctly rounded sqrt and reciprocal), which turns
// tolerance parity into bitwise parity with a CPU that runs the same
// sequence.  Speed is secondary: one thread owns each output and walks its
// sum in order.
//
// The file is built with -ffp-contract=off (and says so below as well), so
// every +, -, * and / here, including those of the inlined header helpers,
// is one IEEE operation rounded to nearest even; HIP's single-precision
// divide and sqrt are correctly rounded by default.
#include "common.h"

#pragma clang fp contract(off)

namespace ge {

namespace {

__device__ __forceinline__ float add(float a, float b) { return a + b; }
__device__ __forceinline__ float sub(float a, float b) { return a - b; }
__device__ __forceinline__ float mul(float a, float b) { return a * b; }
__device__ __forceinline__ float dvd(float a, float b) { return a / b; }
__device__ __forceinline__ float sqrt_rn(float a) { return __builtin_sqrtf(a); }

constexpr int kTile = 64, kBK = 16;

template <typename T, int LAYOUT>
__device__ __forceinline__ float a_at(const T *A, int64_t lda, int64_t m, int64_t k) {
  return to_f32(LAYOUT == GE_TN ? A[k * lda + m] : A[m * lda + k]);
}
template <typename T, int LAYOUT>
__device__ __forceinline__ float b_at(const T *B, int64_t ldb, int64_t k, int64_t n) {
  return to_f32(LAYOUT == GE_NT ? B[n * ldb + k] : B[k * ldb + n]);
}

// 64x64 outputs per block of 16x16 threads, 4x4 per thread; K in chunks of
// 16 through LDS, each output's products added in k order
template <typename T, int LAYOUT>
__global__ __launch_bounds__(256) void gemm_exact_kernel(ge_gemm_args a) {
  __shared__ float As[kBK][kTile + 1];
  __shared__ float Bs[kBK][kTile + 1];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int64_t m0 = (int64_t)blockIdx.y * kTile, n0 = (int64_t)blockIdx.x * kTile;
  const T *A = (const T *)a.A;
  const T *B = (const T *)a.B;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
  for (int64_t k0 = 0; k0 < a.K; k0 += kBK) {
    const int kn = (int)min<int64_t>(kBK, a.K - k0);
    for (int e = threadIdx.x; e < kBK * kTile; e += 256) {
      const int kk = e / kTile, mm = e % kTile;
      const bool ok = kk < kn;
      As[kk][mm] = ok && m0 + mm < a.M ? a_at<T, LAYOUT>(A, a.lda, m0 + mm, k0 + kk) : 0.f;
      Bs[kk][mm] = ok && n0 + mm < a.N ? b_at<T, LAYOUT>(B, a.ldb, k0 + kk, n0 + mm) : 0.f;
    }
    __syncthreads();
    for (int kk = 0; kk < kn; ++kk) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[j] = Bs[kk][tx + 16 * j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = add(acc[i][j], mul(av[i], bv[j]));
    }
    __syncthreads();
  }
  const float c2 = mul(mul(2.f, a.act_slope), a.act_slope);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t m = m0 + ty * 4 + i;
    if (m >= a.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t n = n0 + tx + 16 * j;
      if (n >= a.N) continue;
      float v = mul(a.alpha, acc[i][j]);
      if (a.bias) v = add(v, a.bias[n]);
      if (a.pre) store_any(a.pre, m * a.ld_pre + n, a.pre_type, v);
      if (a.act == GE_ACT_RELU) {
        v = v > 0.f ? v : 0.f;
      } else if (a.act == GE_ACT_LRELU_SQ) {
        const float t = v > 0.f ? v : mul(a.act_slope, v);
        v = mul(t, t);
      } else if (a.act == GE_ACT_RELU_MASK_BWD) {
        v = mul(v, load_any(a.aux, m * a.ld_aux + n, a.aux_type) > 0.f ? 1.f : 0.f);
      } else if (a.act == GE_ACT_LRELU_SQ_BWD) {
        const float u = load_any(a.aux, m * a.ld_aux + n, a.aux_type);
        v = mul(v, u > 0.f ? mul(2.f, u) : mul(c2, u));
      }
      if (a.residual) v = add(v, load_any(a.residual, m * a.ld_res + n, a.res_type));
      store_any(a.C, m * a.ldc + n, a.c_type, v);
    }
  }
}

template <typename T>
int gemm_exact_t(const ge_gemm_args &a, hipStream_t s) {
  const dim3 grid((unsigned)((a.N + kTile - 1) / kTile), (unsigned)((a.M + kTile - 1) / kTile));
  switch (a.layout) {
    case GE_NN: hipLaunchKernelGGL((gemm_exact_kernel<T, GE_NN>), grid, dim3(256), 0, s, a); break;
    case GE_NT: hipLaunchKernelGGL((gemm_exact_kernel<T, GE_NT>), grid, dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL((gemm_exact_kernel<T, GE_TN>), grid, dim3(256), 0, s, a); break;
  }
  return launch_status("gemm_bias_act (bit-exact)");
}

// one thread per column, rows in order
__global__ __launch_bounds__(256) void colsum_exact_kernel(const void *X, int64_t M, int64_t N, int64_t ldx, int xt,
                                                           float alpha, float *out, int accumulate) {
  const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (n >= N) return;
  float s = 0.f;
  for (int64_t m = 0; m < M; ++m) s = add(s, load_any(X, m * ldx + n, xt));
  const float t = mul(alpha, s);
  out[n] = accumulate ? add(out[n], t) : t;
}

__global__ __launch_bounds__(256) void sgd_exact_kernel(float *w, const float *g, float *v, float lr, float mu,
                                                        int64_t n, void *wl, int lt) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const float vel = sub(mul(mu, v[i]), mul(lr, g[i]));
  v[i] = vel;
  const float wn = add(w[i], vel);
  w[i] = wn;
  if (wl) store_any(wl, i, lt, wn);
}

// one thread per row
__global__ __launch_bounds__(256) void rms_fwd_exact_kernel(ge_rmsnorm_args a) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= a.rows) return;
  const int64_t D = a.D;
  float ss = 0.f;
  for (int64_t j = 0; j < D; ++j) {
    const float x = load_any(a.x, i * a.ld_x + j, a.x_type);
    ss = add(ss, mul(x, x));
  }
  const float r = dvd(1.f, sqrt_rn(add(dvd(ss, (float)D), a.eps)));
  a.r[i] = r;
  for (int64_t j = 0; j < D; ++j) {
    float y = mul(load_any(a.x, i * a.ld_x + j, a.x_type), r);
    if (a.gamma) y = mul(y, a.gamma[j]);
    store_any(a.y, i * a.ld_y + j, a.y_type, y);
  }
}

__global__ __launch_bounds__(256) void rms_bwd_exact_kernel(ge_rmsnorm_args a) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= a.rows) return;
  const int64_t D = a.D;
  const float r = a.r[i];
  float s = 0.f;
  for (int64_t j = 0; j < D; ++j) {
    const float xh = mul(load_any(a.x, i * a.ld_x + j, a.x_type), r);
    float g = load_any(a.dy, i * a.ld_dy + j, a.dy_type);
    if (a.gamma) g = mul(g, a.gamma[j]);
    s = add(s, mul(g, xh));
  }
  const float c = dvd(s, (float)D);
  for (int64_t j = 0; j < D; ++j) {
    const float xh = mul(load_any(a.x, i * a.ld_x + j, a.x_type), r);
    float g = load_any(a.dy, i * a.ld_dy + j, a.dy_type);
    if (a.gamma) g = mul(g, a.gamma[j]);
    float dx = mul(r, sub(g, mul(xh, c)));
    if (a.dres) dx = add(dx, load_any(a.dres, i * a.ld_dres + j, a.dres_type));
    store_any(a.dx, i * a.ld_dx + j, a.dx_type, dx);
  }
}

// dgamma[j]: one thread per column, rows in order
__global__ __launch_bounds__(256) void rms_dgamma_exact_kernel(ge_rmsnorm_args a) {
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (j >= a.D) return;
  float s = 0.f;
  for (int64_t i = 0; i < a.rows; ++i) {
    const float xh = mul(load_any(a.x, i * a.ld_x + j, a.x_type), a.r[i]);
    s = add(s, mul(load_any(a.dy, i * a.ld_dy + j, a.dy_type), xh));
  }
  a.dgamma[j] = s;
}

unsigned blocks_for(int64_t n) { return (unsigned)((n + 255) / 256); }

}  // namespace

int gemm_exact_launch(const ge_gemm_args &a, hipStream_t s) {
  if (a.M == 0 || a.N == 0) return GE_OK;
  if ((a.N + kTile - 1) / kTile > 0x7fffffff || (a.M + kTile - 1) / kTile > 65535) {
    set_error("gemm_bias_act (bit-exact): M too large for the grid");
    return GE_E_INVALID;
  }
  if (a.ab_type == GE_F16) return gemm_exact_t<half_t>(a, s);
  if (a.ab_type == GE_BF16) return gemm_exact_t<bf16_t>(a, s);
  return gemm_exact_t<float>(a, s);
}

int colsum_exact_launch(const void *X, int64_t M, int64_t N, int64_t ldx, int xt, float alpha, float *out,
                        int accumulate, hipStream_t s) {
  if (N == 0) return GE_OK;
  hipLaunchKernelGGL(colsum_exact_kernel, dim3(blocks_for(N)), dim3(256), 0, s, X, M, N, ldx, xt, alpha, out,
                     accumulate);
  return launch_status("colsum (bit-exact)");
}

int sgd_exact_launch(float *w, const float *g, float *v, float lr, float mu, int64_t n, void *wl, int lt,
                     hipStream_t s) {
  if (n == 0) return GE_OK;
  hipLaunchKernelGGL(sgd_exact_kernel, dim3(blocks_for(n)), dim3(256), 0, s, w, g, v, lr, mu, n, wl, lt);
  return launch_status("sgd_momentum (bit-exact)");
}

int rmsnorm_exact_launch(const ge_rmsnorm_args &a, hipStream_t s) {
  if (a.rows == 0) return GE_OK;
  if (a.pass == GE_FWD) {
    hipLaunchKernelGGL(rms_fwd_exact_kernel, dim3(blocks_for(a.rows)), dim3(256), 0, s, a);
    return launch_status("rmsnorm_fwd_bwd (bit-exact forward)");
  }
  hipLaunchKernelGGL(rms_bwd_exact_kernel, dim3(blocks_for(a.rows)), dim3(256), 0, s, a);
  int st = launch_status("rmsnorm_fwd_bwd (bit-exact backward)");
  if (st != GE_OK || !a.dgamma) return st;
  hipLaunchKernelGGL(rms_dgamma_exact_kernel, dim3(blocks_for(a.D)), dim3(256), 0, s, a);
  return launch_status("rmsnorm_fwd_bwd (bit-exact dgamma)");
}

}  // namespace ge
