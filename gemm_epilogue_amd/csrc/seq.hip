// Kernels of the recurrent (GRU) language-model step, for gfx950 (wave64):
// token re-ordering, embedding gather and its gradient, and the GRU gate
// arithmetic of one timestep, forward and backward.  The gate math stays in
// FP32 and only the copies that feed GEMMs are FP16 ("The Work Moved Down a
// Layer", sections "The Work Moved Down a Layer" (GRU gates) and "The
// Debugging Lesson Was Numerical" (recurrent state in FP32)).  The pages give
// no GRU equations; the cell is the standard one with gate blocks (r, z, n):
//   r = s(GI_r + GH_r), z = s(GI_z + GH_z), n = tanh(GI_n + r GH_n),
//   h = (1 - z) n + z h_prev.
#include <algorithm>

#include "common.h"

namespace ge {

// tokens [B x (T+1)] -> time-major inputs inp[t*B + b] = tok[b][t] and
// targets tgt[t*B + b] = tok[b][t+1]
__global__ void tokens_time_major_kernel(const int32_t *__restrict__ tok, int B, int T, int32_t *__restrict__ inp,
                                         int32_t *__restrict__ tgt) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= B * T) return;
  const int t = i / B, b = i % B;
  inp[i] = tok[(int64_t)b * (T + 1) + t];
  tgt[i] = tok[(int64_t)b * (T + 1) + t + 1];
}

__global__ void fill_zero_kernel(uint32_t *__restrict__ p, int64_t n_words) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n_words) p[i] = 0u;
}

// out[i, :] = table[idx[i], :]; an index outside [0, V) gives a zero row.
__global__ void embedding_gather_kernel(const void *__restrict__ table, int V, int H, int64_t ldt, int tt,
                                        const int32_t *__restrict__ idx, int n, void *__restrict__ out,
                                        int64_t ldo, int ot) {
  const int row = blockIdx.x;
  if (row >= n) return;
  const int v = idx[row];
  const bool ok = (unsigned)v < (unsigned)V;
  for (int j = threadIdx.x; j < H; j += blockDim.x)
    store_any(out, (int64_t)row * ldo + j, ot, ok ? load_any(table, (int64_t)v * ldt + j, tt) : 0.f);
}

// dE[v, j] = alpha * sum over i with idx[i] == v (in increasing i) of dX[i, j].
// Block (v, column chunk of 256); the index list is staged through LDS in
// chunks and scanned in order by every thread, so each sum has a fixed order.
__global__ __launch_bounds__(256) void embedding_grad_kernel(const void *__restrict__ dX, int64_t ldx, int xt,
                                                             const int32_t *__restrict__ idx, int n, int V,
                                                             int H, float alpha, float *__restrict__ dE,
                                                             int64_t lde) {
  __shared__ int32_t sidx[2048];
  const int v = blockIdx.x;
  const int j = blockIdx.y * 256 + threadIdx.x;
  float s = 0.f;
  for (int c0 = 0; c0 < n; c0 += 2048) {
    const int cn = min(2048, n - c0);
    __syncthreads();
    for (int i = threadIdx.x; i < cn; i += 256) sidx[i] = idx[c0 + i];
    __syncthreads();
    if (j < H) {
      for (int i = 0; i < cn; ++i)
        if (sidx[i] == v) s += load_any(dX, (int64_t)(c0 + i) * ldx + j, xt);
    }
  }
  if (j < H) dE[(int64_t)v * lde + j] = alpha * s;
}

__device__ __forceinline__ float sigmoid_f(float x) { return 1.f / (1.f + expf(-x)); }

// One forward timestep over B x H (four hidden units per thread).
// GI, GH: [B x 3H] f32 rows (r | z | n blocks); hp: h_{t-1} f32 [B x H].
// Writes r, z, n (f32, saved for the backward), h (f32) and h16 (f16 copy).
__global__ __launch_bounds__(256) void gru_fwd_kernel(const float *__restrict__ GI, const float *__restrict__ GH,
                                                      const float *__restrict__ hp, int B, int H,
                                                      float *__restrict__ R, float *__restrict__ Z,
                                                      float *__restrict__ Nn, float *__restrict__ h,
                                                      half_t *__restrict__ h16) {
  const int64_t i4 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i4 >= (int64_t)B * H) return;
  const int b = (int)(i4 / H), j = (int)(i4 % H);
  const int64_t g = (int64_t)b * 3 * H + j;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (j + q >= H) break;
    const float r = sigmoid_f(GI[g + q] + GH[g + q]);
    const float z = sigmoid_f(GI[g + H + q] + GH[g + H + q]);
    const float nn = tanhf(GI[g + 2 * H + q] + r * GH[g + 2 * H + q]);
    const float hv = (1.f - z) * nn + z * hp[i4 + q];
    R[i4 + q] = r;
    Z[i4 + q] = z;
    Nn[i4 + q] = nn;
    h[i4 + q] = hv;
    h16[i4 + q] = (half_t)hv;
  }
}

// One backward timestep.  dh = dh_out + carry (carry = gradient from t+1),
//   dn = dh (1 - z), dz = dh (h_prev - n), dh_dir = dh z,
//   dnh = dn (1 - n^2), dr = dnh GH_n,
//   dG_r = dr r (1 - r), dG_z = dz z (1 - z),
//   dGH = [dG_r, dG_z, dnh r] and dGI = [dG_r, dG_z, dnh] (FP16 GEMM inputs).
__global__ __launch_bounds__(256) void gru_bwd_kernel(const float *__restrict__ dh_out,
                                                      const float *__restrict__ carry, const float *__restrict__ R,
                                                      const float *__restrict__ Z, const float *__restrict__ Nn,
                                                      const float *__restrict__ GH, const float *__restrict__ hp,
                                                      int B, int H, half_t *__restrict__ dGH,
                                                      half_t *__restrict__ dGI, float *__restrict__ dh_dir) {
  const int64_t i4 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i4 >= (int64_t)B * H) return;
  const int b = (int)(i4 / H), j = (int)(i4 % H);
  const int64_t g = (int64_t)b * 3 * H + j;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (j + q >= H) break;
    const int64_t i = i4 + q;
    const float dh = dh_out[i] + carry[i];
    const float r = R[i], z = Z[i], nn = Nn[i];
    const float dn = dh * (1.f - z);
    const float dz = dh * (hp[i] - nn);
    const float dnh = dn * (1.f - nn * nn);
    const float dr = dnh * GH[g + 2 * H + q];
    const float dgr = dr * r * (1.f - r);
    const float dgz = dz * z * (1.f - z);
    dh_dir[i] = dh * z;
    dGH[g + q] = (half_t)dgr;
    dGH[g + H + q] = (half_t)dgz;
    dGH[g + 2 * H + q] = (half_t)(dnh * r);
    dGI[g + q] = (half_t)dgr;
    dGI[g + H + q] = (half_t)dgz;
    dGI[g + 2 * H + q] = (half_t)dnh;
  }
}

// ---- launchers ------------------------------------------------------------------
int tokens_time_major_launch(const int32_t *tok, int B, int T, int32_t *inp, int32_t *tgt, hipStream_t s) {
  const int n = B * T;
  hipLaunchKernelGGL(tokens_time_major_kernel, dim3((n + 255) / 256), dim3(256), 0, s, tok, B, T, inp, tgt);
  return launch_status("tokens_time_major");
}

int fill_zero_launch(void *p, int64_t bytes, hipStream_t s) {
  const int64_t words = bytes / 4;
  if (words == 0) return GE_OK;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, s, (uint32_t *)p,
                     words);
  return launch_status("fill_zero");
}

int embedding_gather_launch(const void *table, int64_t V, int64_t H, int64_t ldt, int tt, const int32_t *idx,
                            int64_t n, void *out, int64_t ldo, int ot, hipStream_t s) {
  if (n == 0 || H == 0) return GE_OK;
  hipLaunchKernelGGL(embedding_gather_kernel, dim3((unsigned)n), dim3(256), 0, s, table, (int)V, (int)H, ldt, tt,
                     idx, (int)n, out, ldo, ot);
  return launch_status("embedding_gather");
}

int embedding_grad_launch(const void *dX, int64_t ldx, int xt, const int32_t *idx, int64_t n, int64_t V,
                          int64_t H, float alpha, float *dE, int64_t lde, hipStream_t s) {
  if (V == 0 || H == 0) return GE_OK;
  hipLaunchKernelGGL(embedding_grad_kernel, dim3((unsigned)V, (unsigned)((H + 255) / 256)), dim3(256), 0, s, dX,
                     ldx, xt, idx, (int)n, (int)V, (int)H, alpha, dE, lde);
  return launch_status("embedding_grad");
}

int gru_fwd_launch(const float *GI, const float *GH, const float *hp, int B, int H, float *R, float *Z, float *N,
                   float *h, half_t *h16, hipStream_t s) {
  const int64_t items = ((int64_t)B * H + 3) / 4;
  hipLaunchKernelGGL(gru_fwd_kernel, dim3((unsigned)((items + 255) / 256)), dim3(256), 0, s, GI, GH, hp, B, H, R,
                     Z, N, h, h16);
  return launch_status("gru_fwd");
}

int gru_bwd_launch(const float *dh_out, const float *carry, const float *R, const float *Z, const float *N,
                   const float *GH, const float *hp, int B, int H, half_t *dGH, half_t *dGI, float *dh_dir,
                   hipStream_t s) {
  const int64_t items = ((int64_t)B * H + 3) / 4;
  hipLaunchKernelGGL(gru_bwd_kernel, dim3((unsigned)((items + 255) / 256)), dim3(256), 0, s, dh_out, carry, R, Z,
                     N, GH, hp, B, H, dGH, dGI, dh_dir);
  return launch_status("gru_bwd");
}

}  // namespace ge
