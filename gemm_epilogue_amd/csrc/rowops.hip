// Bandwidth-bound kernels of the training step, for gfx950 (wave64):
// column sums (bias gradients), stable softmax cross-entropy, RMSNorm forward
// and backward, and the flat SGD-momentum update.
//
// All reductions run in FP32 in a fixed order (per-lane sequential sums, then
// a fixed butterfly across the 64 lanes, then a fixed order across waves and
// blocks), so results are bitwise reproducible ("The Work Moved Down a Layer",
// section "The Debugging Lesson Was Numerical": reductions for softmax and
// loss in FP32).  Loads and stores are 16-byte (FP32) or 8-byte (16-bit)
// vectors of four consecutive elements wherever alignment allows.
#include <algorithm>

#include "common.h"

namespace ge {

// =========================== column sums ====================================
// "Capstone 5: train a network with your CUDA kernels", section "Work through
// the backward pass": db = sum_rows(dZ), a reduction across the batch.
//
// A block of 256 threads owns a strip of 256 bytes of every row (64 FP32 or
// 128 16-bit columns: 16 lanes of 16 bytes) and a contiguous range of rows,
// read in batches of 256 rows: lane l of wave w takes, for u = 0..15, row
// 16 u + 4 w + l / 16 of the batch, so each wave has all sixteen of its
// 16-byte loads in flight at once.  A lane adds its rows in order (u, then
// batch); the four lanes of a column within a wave are added pairwise
// ((g0 + g1) + (g2 + g3), the same value in every lane as addition commutes),
// then the four waves in wave order.  With several row ranges the partials go
// to a workspace and colsum_final adds them: wave w of a final block takes
// ranges w, w+4, ... in order and the four wave sums are again added in wave
// order.
constexpr int CS_BATCH = 256;  // rows per block batch
constexpr int CS_U = 16;       // loads in flight per lane

template <typename T, int VEC>
__device__ __forceinline__ void cs_load(const T *__restrict__ X, int64_t i, bool full, int left, float (&v)[VEC]) {
  if (full) {
    if constexpr (sizeof(T) == 4) {
      const f32x4 a = *(const f32x4 *)(X + i);
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = a[j];
    } else {
      typedef T T8 __attribute__((ext_vector_type(8)));
      const T8 x = *(const T8 *)(X + i);
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = (float)x[j];
    }
  } else {
#pragma unroll
    for (int j = 0; j < VEC; ++j) v[j] = j < left ? (float)X[i + j] : 0.f;
  }
}

template <typename T>
__global__ __launch_bounds__(256) void colsum_partial_kernel(const T *__restrict__ X, int M, int N, int64_t ldx,
                                                             int vec, int rows_per, float alpha,
                                                             float *__restrict__ out, int accumulate) {
  constexpr int VEC = 16 / (int)sizeof(T);
  constexpr int CW = 16 * VEC;  // columns per block
  __shared__ float red[3][CW];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int cl = lane & 15, rg = lane >> 4;
  const int n = blockIdx.x * CW + cl * VEC;
  const int r0 = blockIdx.y * rows_per;
  const int r1 = min(M, r0 + rows_per);
  float s[VEC];
#pragma unroll
  for (int j = 0; j < VEC; ++j) s[j] = 0.f;
  if (n < N) {
    const bool full = vec && n + VEC <= N;
    const int left = N - n;
    for (int rb = r0; rb < r1; rb += CS_BATCH) {
      float v[CS_U][VEC];
#pragma unroll
      for (int u = 0; u < CS_U; ++u) {
        const int r = rb + 16 * u + 4 * wave + rg;
        if (r < r1) {
          cs_load<T, VEC>(X, (int64_t)r * ldx + n, full, left, v[u]);
        } else {
#pragma unroll
          for (int j = 0; j < VEC; ++j) v[u][j] = 0.f;
        }
      }
#pragma unroll
      for (int u = 0; u < CS_U; ++u)
#pragma unroll
        for (int j = 0; j < VEC; ++j) s[j] += v[u][j];
    }
  }
  // the four row groups of the wave: (g0 + g1) + (g2 + g3)
#pragma unroll
  for (int j = 0; j < VEC; ++j) {
    s[j] += __shfl_xor(s[j], 16, 64);
    s[j] += __shfl_xor(s[j], 32, 64);
  }
  if (wave > 0 && rg == 0) {
#pragma unroll
    for (int j = 0; j < VEC; ++j) red[wave - 1][cl * VEC + j] = s[j];
  }
  __syncthreads();
  if (wave == 0 && rg == 0 && n < N) {
    float *dst = out + (int64_t)blockIdx.y * N;
#pragma unroll
    for (int j = 0; j < VEC; ++j) {
      const int c = cl * VEC + j;
      const float t = ((s[j] + red[0][c]) + red[1][c]) + red[2][c];
      if (n + j < N) dst[n + j] = accumulate ? dst[n + j] + alpha * t : alpha * t;
    }
  }
}

__global__ __launch_bounds__(256) void colsum_final_kernel(const float *__restrict__ part, int splits, int N,
                                                           float alpha, float *__restrict__ out, int accumulate) {
  __shared__ float red[3][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = blockIdx.x * 64 + lane;
  float s = 0.f;
  if (n < N) {
    // eight ranges' loads in flight, added in range order
    for (int k = wave; k < splits; k += 4 * 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = k + 4 * u < splits ? part[(int64_t)(k + 4 * u) * N + n] : 0.f;
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (k + 4 * u < splits) s += v[u];
    }
  }
  if (wave > 0) red[wave - 1][lane] = s;
  __syncthreads();
  if (wave == 0 && n < N) {
    const float t = alpha * (((s + red[0][lane]) + red[1][lane]) + red[2][lane]);
    out[n] = accumulate ? out[n] + t : t;
  }
}

namespace {
int colsum_splits(int64_t M, int64_t N) {
  if (M < 1024) return 1;  // one pass: a block reads all rows of its columns
  // about 2048 strips of 64 columns x 256 rows, at most 64 ranges (the
  // final pass adds them per column); independent of the element type
  const int64_t units = (N + 63) / 64;
  const int64_t want = (2048 + units - 1) / units;
  return (int)std::max<int64_t>(1, std::min<int64_t>({want, (M + CS_BATCH - 1) / CS_BATCH, 64}));
}

template <typename T>
void colsum_partial(dim3 grid, hipStream_t st, const void *X, int M, int N, int64_t ldx, int vec, int rows_per,
                    float alpha, float *out, int acc) {
  hipLaunchKernelGGL(colsum_partial_kernel<T>, grid, dim3(256), 0, st, (const T *)X, M, N, ldx, vec, rows_per,
                     alpha, out, acc);
}

void colsum_partial_any(int xt, dim3 grid, hipStream_t st, const void *X, int M, int N, int64_t ldx, int vec,
                        int rows_per, float alpha, float *out, int acc) {
  if (xt == GE_F32) colsum_partial<float>(grid, st, X, M, N, ldx, vec, rows_per, alpha, out, acc);
  else if (xt == GE_F16) colsum_partial<half_t>(grid, st, X, M, N, ldx, vec, rows_per, alpha, out, acc);
  else colsum_partial<bf16_t>(grid, st, X, M, N, ldx, vec, rows_per, alpha, out, acc);
}
}  // namespace

int colsum_rows_launch(const float *part, int64_t rows, int64_t N, float alpha, float *out, hipStream_t st) {
  if (N == 0) return GE_OK;
  hipLaunchKernelGGL(colsum_final_kernel, dim3((unsigned)((N + 63) / 64)), dim3(256), 0, st, part, (int)rows,
                     (int)N, alpha, out, 0);
  return launch_status("colsum (rows)");
}

int64_t colsum_ws_bytes(int64_t M, int64_t N) {
  if (M <= 0 || N <= 0) return 0;
  const int s = colsum_splits(M, N);
  return s > 1 ? (int64_t)s * N * 4 : 0;
}

int colsum_launch(const void *X, int64_t M, int64_t N, int64_t ldx, int xt, float alpha, float *out,
                  void *ws, int64_t ws_bytes, hipStream_t st, int accumulate) {
  if (N == 0) return GE_OK;
  const int vec = vec_aligned(X, ldx, dtype_size(xt), 16);
  const int colblocks = (int)((N * dtype_size(xt) + 255) / 256);
  const int splits = M > 0 ? colsum_splits(M, N) : 1;
  if (splits == 1) {
    colsum_partial_any(xt, dim3(colblocks, 1), st, X, (int)M, (int)N, ldx, vec, (int)std::max<int64_t>(M, 1),
                       alpha, out, accumulate);
    return launch_status("colsum");
  }
  const int64_t need = (int64_t)splits * N * 4;
  if (ws == nullptr || ws_bytes < need) {
    set_error("colsum: %lld rows need %lld workspace bytes", (long long)M, (long long)need);
    return GE_E_WORKSPACE;
  }
  const int rows_per = (int)((M + splits - 1) / splits);
  colsum_partial_any(xt, dim3(colblocks, splits), st, X, (int)M, (int)N, ldx, vec, rows_per, 1.0f, (float *)ws, 0);
  int s = launch_status("colsum (partial)");
  if (s != GE_OK) return s;
  hipLaunchKernelGGL(colsum_final_kernel, dim3((unsigned)((N + 63) / 64)), dim3(256), 0, st,
                     (const float *)ws, splits, (int)N, alpha, out, accumulate);
  return launch_status("colsum (final)");
}

// ====================== softmax cross-entropy ===============================
// "Capstone 5", sections "The minimum model" and "Read the worked reference":
// stable softmax cross-entropy -- subtract the row maximum before exp -- gives
// the loss and dZ.  One wavefront per row; lanes stride the classes.
__global__ __launch_bounds__(256) void xent_rows_kernel(const float *__restrict__ Z, int B, int C, int64_t ld,
                                                        const int32_t *__restrict__ labels, float gscale,
                                                        float *__restrict__ row_loss, void *__restrict__ dZ,
                                                        int64_t ldd, int dt, int32_t *__restrict__ amax) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= B) return;
  const float *z = Z + (int64_t)row * ld;
  // max and lowest index of the max
  float m = -INFINITY;
  int mi = 0x7fffffff;
  for (int c = lane; c < C; c += 64) {
    const float v = z[c];
    if (v > m) { m = v; mi = c; }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float om = __shfl_xor(m, o, 64);
    const int oi = __shfl_xor(mi, o, 64);
    if (om > m || (om == m && oi < mi)) { m = om; mi = oi; }
  }
  // The sum of exp(z - m) is 1 (the maximum's own term) plus the sum of the
  // other terms, s_rest.  Keeping s_rest apart avoids two cancellations in
  // FP32 when one class dominates: lse - m = log1p(s_rest) instead of
  // log(1 + s_rest), and for the label class p - 1 = -(sum of the other
  // classes' terms) / s instead of a subtraction from 1.
  const int y = labels[row];
  const bool yok = (unsigned)y < (unsigned)C;
  float s_rest = 0.f, e_y = 0.f;
  for (int c = lane; c < C; c += 64) {
    const float e = expf(z[c] - m);
    if (c != mi) s_rest += e;
    if (c == y) e_y = e;
  }
  s_rest = wave_sum(s_rest);
  e_y = wave_sum(e_y);  // exactly one lane holds it
  const float l1p = log1pf(s_rest);
  const float lse = m + l1p;
  const float s = 1.f + s_rest;
  if (lane == 0) {
    // a label outside [0, C) reads nothing and yields a NaN row loss
    row_loss[row] = yok ? (m - z[y]) + l1p : NAN;
    if (amax) amax[row] = mi;
  }
  if (dZ) {
    // sum of the terms of every class but the label's
    const float s_noty = (y == mi) ? s_rest : s - e_y;
    for (int c = lane; c < C; c += 64) {
      const float g = (c == y) ? -(s_noty / s) : expf(z[c] - lse);
      store_any(dZ, (int64_t)row * ldd + c, dt, gscale * g);
    }
  }
}

// mean of the row losses: one block, fixed order (thread t sums rows t, t+256,
// ..., then a fixed tree over the 256 partials).  With `bad` it also counts
// the labels outside [0, C) (an integer count, so the order does not matter).
__global__ __launch_bounds__(256) void xent_mean_kernel(const float *__restrict__ row_loss, int B,
                                                        float *__restrict__ out, const int32_t *__restrict__ labels,
                                                        int C, int32_t *__restrict__ bad) {
  __shared__ float red[256];
  __shared__ int nbad[256];
  float s = 0.f;
  int nb = 0;
  for (int i = threadIdx.x; i < B; i += 256) {
    s += row_loss[i];
    if (bad) nb += (unsigned)labels[i] >= (unsigned)C;
  }
  red[threadIdx.x] = s;
  nbad[threadIdx.x] = nb;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) {
      red[threadIdx.x] += red[threadIdx.x + w];
      nbad[threadIdx.x] += nbad[threadIdx.x + w];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    out[0] = B > 0 ? red[0] / (float)B : 0.f;
    if (bad) bad[0] = nbad[0];
  }
}

int xent_launch(const float *Z, int64_t B, int64_t C, int64_t ld, const int32_t *labels, float gscale,
                float *loss_mean, float *row_loss, void *dZ, int64_t ldd, int dt, int32_t *amax,
                hipStream_t st, int32_t *bad_label_count) {
  if (B > 0) {
    hipLaunchKernelGGL(xent_rows_kernel, dim3((unsigned)((B + 3) / 4)), dim3(256), 0, st, Z, (int)B, (int)C,
                       ld, labels, gscale, row_loss, dZ, ldd, dt, amax);
    int s = launch_status("softmax_xent_fwd_bwd (rows)");
    if (s != GE_OK) return s;
  }
  hipLaunchKernelGGL(xent_mean_kernel, dim3(1), dim3(256), 0, st, row_loss, (int)B, loss_mean, labels, (int)C,
                     bad_label_count);
  return launch_status("softmax_xent_fwd_bwd (mean)");
}

// ============================== RMSNorm =====================================
// FP32 statistics ("The Work Moved Down a Layer", "The Debugging Lesson Was
// Numerical"); the block's first step ("Full-Depth MLP Megakernel ...", "What
// Worked").  One wavefront per row; the row lives in registers (CH chunks of
// four elements per lane, D <= 256*CH).
template <int CH>
__global__ __launch_bounds__(256) void rms_fwd_kernel(ge_rmsnorm_args a, int vx, int vy) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.rows) return;
  const int D = (int)a.D;
  float x[CH][4];
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int j = (c * 64 + lane) * 4;
    if (j + 3 < D) {
      load4_any(a.x, row * a.ld_x + j, a.x_type, vx, x[c]);
    } else {
      for (int e = 0; e < 4; ++e) x[c][e] = (j + e < D) ? load_any(a.x, row * a.ld_x + j + e, a.x_type) : 0.f;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) ss += x[c][e] * x[c][e];
  }
  ss = wave_sum(ss);
  const float r = 1.0f / sqrtf(ss / (float)D + a.eps);
  if (lane == 0) a.r[row] = r;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int j = (c * 64 + lane) * 4;
    if (j >= D) continue;
    float y[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) y[e] = x[c][e] * r * (a.gamma && j + e < D ? a.gamma[j + e] : 1.f);
    if (j + 3 < D) {
      store4_any(a.y, row * a.ld_y + j, a.y_type, vy, y);
    } else {
      for (int e = 0; e < 4; ++e)
        if (j + e < D) store_any(a.y, row * a.ld_y + j + e, a.y_type, y[e]);
    }
  }
}

// dx = r * (g - xh * mean(g * xh)) + dres,  xh = x * r,  g = dy * gamma.
// With dgamma requested, each block also writes its partial sum_rows dy * xh
// for its 4 rows into the workspace ([blocks x D], block order).
template <int CH>
__global__ __launch_bounds__(256) void rms_bwd_kernel(ge_rmsnorm_args a, int vx, int vdy, int vres, int vdx,
                                                      float *__restrict__ dg_part) {
  __shared__ float dgs[4][256 * CH];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row = blockIdx.x * 4 + wave;
  const bool live = row < a.rows;
  const int D = (int)a.D;
  float xh[CH][4], g[CH][4], rs[CH][4];
  float dot = 0.f;
  const float r = live ? a.r[row] : 0.f;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int j = (c * 64 + lane) * 4;
    float xv[4], dv[4];
    // the residual gradient is read with x and dy, so the row's reads all
    // go out before the reduction
    if (live && j + 3 < D) {
      load4_any(a.x, row * a.ld_x + j, a.x_type, vx, xv);
      load4_any(a.dy, row * a.ld_dy + j, a.dy_type, vdy, dv);
      if (a.dres) load4_any(a.dres, row * a.ld_dres + j, a.dres_type, vres, rs[c]);
      else
        for (int e = 0; e < 4; ++e) rs[c][e] = 0.f;
    } else {
      for (int e = 0; e < 4; ++e) {
        const bool ok = live && j + e < D;
        xv[e] = ok ? load_any(a.x, row * a.ld_x + j + e, a.x_type) : 0.f;
        dv[e] = ok ? load_any(a.dy, row * a.ld_dy + j + e, a.dy_type) : 0.f;
        rs[c][e] = ok && a.dres ? load_any(a.dres, row * a.ld_dres + j + e, a.dres_type) : 0.f;
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      xh[c][e] = xv[e] * r;
      g[c][e] = dv[e] * ((a.gamma && j + e < D) ? a.gamma[j + e] : 1.f);
      dot += g[c][e] * xh[c][e];
      if (dg_part) dgs[wave][c * 256 + lane * 4 + e] = dv[e] * xh[c][e];
    }
  }
  dot = wave_sum(dot);
  const float cm = dot / (float)D;
  if (live) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int j = (c * 64 + lane) * 4;
      if (j >= D) continue;
      float dx[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) dx[e] = r * (g[c][e] - xh[c][e] * cm) + rs[c][e];
      if (j + 3 < D) {
        store4_any(a.dx, row * a.ld_dx + j, a.dx_type, vdx, dx);
      } else {
        for (int e = 0; e < 4; ++e)
          if (j + e < D) store_any(a.dx, row * a.ld_dx + j + e, a.dx_type, dx[e]);
      }
    }
  }
  if (dg_part) {
    __syncthreads();
    for (int i = threadIdx.x; i < D; i += 256) {
      // column i of chunk layout: chunk c = i / 256, lane*4+e = i % 256
      const int c = i / 256, o = i % 256;
      const float t = ((dgs[0][c * 256 + o] + dgs[1][c * 256 + o]) + dgs[2][c * 256 + o]) + dgs[3][c * 256 + o];
      dg_part[(int64_t)blockIdx.x * D + i] = t;
    }
  }
}

// dgamma[j] = sum over blocks of the partials, in block order
__global__ __launch_bounds__(256) void rms_dgamma_final(const float *__restrict__ part, int nb, int D,
                                                        float *__restrict__ dgamma) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= D) return;
  float s = 0.f;
  for (int b = 0; b < nb; ++b) s += part[(int64_t)b * D + j];
  dgamma[j] = s;
}

int64_t rmsnorm_ws_bytes(int64_t rows, int64_t D) { return ((rows + 3) / 4) * D * 4; }

namespace {
template <int CH> int rms_dispatch(const ge_rmsnorm_args &a, hipStream_t st) {
  const unsigned blocks = (unsigned)((a.rows + 3) / 4);
  auto al = [](const void *p, int64_t ld, int t) { return p ? (int)vec_aligned(p, ld, dtype_size(t), 4 * dtype_size(t)) : 0; };
  if (a.pass == GE_FWD) {
    hipLaunchKernelGGL(rms_fwd_kernel<CH>, dim3(blocks), dim3(256), 0, st, a, al(a.x, a.ld_x, a.x_type),
                       al(a.y, a.ld_y, a.y_type));
    return launch_status("rmsnorm_fwd_bwd (fwd)");
  }
  float *part = nullptr;
  if (a.dgamma) {
    if (a.workspace == nullptr || a.workspace_bytes < rmsnorm_ws_bytes(a.rows, a.D)) {
      set_error("rmsnorm_fwd_bwd: dgamma needs %lld workspace bytes", (long long)rmsnorm_ws_bytes(a.rows, a.D));
      return GE_E_WORKSPACE;
    }
    part = (float *)a.workspace;
  }
  hipLaunchKernelGGL(rms_bwd_kernel<CH>, dim3(blocks), dim3(256), 0, st, a, al(a.x, a.ld_x, a.x_type),
                     al(a.dy, a.ld_dy, a.dy_type), al(a.dres, a.ld_dres, a.dres_type),
                     al(a.dx, a.ld_dx, a.dx_type), part);
  int s = launch_status("rmsnorm_fwd_bwd (bwd)");
  if (s != GE_OK || !a.dgamma) return s;
  hipLaunchKernelGGL(rms_dgamma_final, dim3((unsigned)((a.D + 255) / 256)), dim3(256), 0, st,
                     (const float *)part, (int)blocks, (int)a.D, a.dgamma);
  return launch_status("rmsnorm_fwd_bwd (dgamma)");
}
}  // namespace

int rmsnorm_launch(const ge_rmsnorm_args &a, hipStream_t st) {
  if (a.rows == 0) return GE_OK;
  if (a.D <= 256) return rms_dispatch<1>(a, st);
  if (a.D <= 512) return rms_dispatch<2>(a, st);
  if (a.D <= 1024) return rms_dispatch<4>(a, st);
  if (a.D <= 2048) return rms_dispatch<8>(a, st);
  return rms_dispatch<16>(a, st);
}

// =========================== SGD momentum ===================================
// "Capstone 5", section "Read the worked reference": one grid-stride update
// over the flat parameter buffer: vel = mu * v - lr * g; v = vel; w += vel.
// Four elements per thread per iteration (16-byte accesses).  Optionally the
// gradient of up to four segments of the buffer is formed here first: alpha
// times the sum of `rows` partial rows (added in row order), also written to
// g, so the column sums or split-K GEMMs that produced the partials need no
// finishing launch of their own.
struct SgdSegment {
  const float *part;  // [rows x len]
  int64_t g0, len;    // the segment is g[g0 .. g0 + len)
  int rows;
  float alpha;
  int vec4;  // part 16-byte aligned, g0 and len multiples of 4
};
struct SgdSegments {
  SgdSegment s[kSgdMaxSegments];
  int n;
};

// the segment holding element k, or -1
__device__ __forceinline__ int sgd_segment_of(const SgdSegments &sg, int64_t k) {
#pragma unroll
  for (int j = 0; j < kSgdMaxSegments; ++j)
    if (j < sg.n && k >= sg.s[j].g0 && k < sg.s[j].g0 + sg.s[j].len) return j;
  return -1;
}
// the segment's gradient at k (also stored to g[k])
__device__ __forceinline__ float sgd_segment_grad(float *g, const SgdSegment &sg, int64_t k) {
  const float *pp = sg.part + (k - sg.g0);
  float t = 0.f;
  for (int r = 0; r < sg.rows; ++r) t += pp[(int64_t)r * sg.len];
  t *= sg.alpha;
  g[k] = t;
  return t;
}

__global__ __launch_bounds__(256) void sgd_kernel(float *__restrict__ w, float *g, float *__restrict__ v, float lr,
                                                  float mu, int64_t n, void *__restrict__ wl, int lt, int vec,
                                                  SgdSegments sg) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x * 4;
  for (int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4; i < n; i += stride) {
    // a quad lies in at most one segment when every segment is vec4; else
    // each element looks its own up
    const int j0 = sgd_segment_of(sg, i), j3 = sgd_segment_of(sg, i + 3);
    if (vec && i + 3 < n) {
      f32x4 wv = *(f32x4 *)(w + i);
      f32x4 vv = *(f32x4 *)(v + i);
      f32x4 gv;
      if (j0 >= 0 && j0 == j3 && sg.s[j0].vec4) {
        // the whole quad: rows of 16-byte loads, eight in flight
        const SgdSegment &sj = sg.s[j0];
        const float *pp = sj.part + (i - sj.g0);
        f32x4 t = f32x4{0.f, 0.f, 0.f, 0.f};
        int r = 0;
        for (; r + 8 <= sj.rows; r += 8) {
          f32x4 x[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) x[u] = *(const f32x4 *)(pp + (int64_t)(r + u) * sj.len);
#pragma unroll
          for (int u = 0; u < 8; ++u) t += x[u];
        }
        for (; r < sj.rows; ++r) t += *(const f32x4 *)(pp + (int64_t)r * sj.len);
#pragma unroll
        for (int e = 0; e < 4; ++e) gv[e] = sj.alpha * t[e];
        *(f32x4 *)(g + i) = gv;
      } else if (j0 >= 0 || j3 >= 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = sgd_segment_of(sg, i + e);
          gv[e] = j >= 0 ? sgd_segment_grad(g, sg.s[j], i + e) : g[i + e];
        }
      } else {
        gv = *(const f32x4 *)(g + i);
      }
      float out[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float vel = mu * vv[e] - lr * gv[e];
        vv[e] = vel;
        wv[e] = wv[e] + vel;
        out[e] = wv[e];
      }
      *(f32x4 *)(v + i) = vv;
      *(f32x4 *)(w + i) = wv;
      if (wl) store4_any(wl, i, lt, true, out);
    } else {
      for (int64_t k = i; k < n && k < i + 4; ++k) {
        const int j = sgd_segment_of(sg, k);
        const float gk = j >= 0 ? sgd_segment_grad(g, sg.s[j], k) : g[k];
        const float vel = mu * v[k] - lr * gk;
        v[k] = vel;
        w[k] = w[k] + vel;
        if (wl) store_any(wl, k, lt, w[k]);
      }
    }
  }
}

int sgd_launch(float *w, float *g, float *v, float lr, float mu, int64_t n, void *wl, int lt, hipStream_t st,
               const SgdSegmentDesc *segs, int nseg) {
  if (n == 0) return GE_OK;
  const int vec = ((uintptr_t)w % 16 == 0) && ((uintptr_t)g % 16 == 0) && ((uintptr_t)v % 16 == 0) &&
                  (wl == nullptr || (uintptr_t)wl % 8 == 0);
  const int64_t items = (n + 3) / 4;
  const unsigned blocks = (unsigned)std::min<int64_t>((items + 255) / 256, 2048);
  if (nseg < 0 || nseg > kSgdMaxSegments || (nseg > 0 && segs == nullptr)) {
    set_error("sgd_momentum: at most %d gradient segments", kSgdMaxSegments);
    return GE_E_INVALID;
  }
  SgdSegments sg;
  sg.n = 0;
  for (int j = 0; j < kSgdMaxSegments; ++j) sg.s[j] = SgdSegment{nullptr, 0, 0, 0, 1.f, 0};
  for (int j = 0; j < nseg; ++j) {
    const SgdSegmentDesc &d = segs[j];
    if (d.part == nullptr || d.rows < 1 || d.g0 < 0 || d.len < 0 || d.g0 + d.len > n) {
      set_error("sgd_momentum: gradient segment out of range");
      return GE_E_INVALID;
    }
    for (int k = 0; k < sg.n; ++k)
      if (d.g0 < sg.s[k].g0 + sg.s[k].len && sg.s[k].g0 < d.g0 + d.len) {
        set_error("sgd_momentum: gradient segments overlap");
        return GE_E_INVALID;
      }
    sg.s[sg.n++] = SgdSegment{d.part, d.g0, d.len, d.rows, d.alpha,
                              ((uintptr_t)d.part % 16 == 0) && d.g0 % 4 == 0 && d.len % 4 == 0};
  }
  hipLaunchKernelGGL(sgd_kernel, dim3(blocks), dim3(256), 0, st, w, g, v, lr, mu, n, wl, lt, vec, sg);
  return launch_status("sgd_momentum");
}

// ======================= low-precision working copy =========================
// w_lowp[i] = convert(w[i]) with round-to-nearest-even: the copy the update
// keeps in step, formed here for the initial parameters.
__global__ __launch_bounds__(256) void to_lowp_kernel(const float *__restrict__ w, int64_t n, void *__restrict__ wl,
                                                      int lt, int vec) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x * 4;
  for (int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4; i < n; i += stride) {
    if (vec && i + 3 < n) {
      const f32x4 x = *(const f32x4 *)(w + i);
      const float o[4] = {x[0], x[1], x[2], x[3]};
      store4_any(wl, i, lt, true, o);
    } else {
      for (int64_t k = i; k < n && k < i + 4; ++k) store_any(wl, k, lt, w[k]);
    }
  }
}

int to_lowp_launch(const float *w, int64_t n, void *wl, int lt, hipStream_t st) {
  if (n == 0) return GE_OK;
  const int vec = ((uintptr_t)w % 16 == 0) && ((uintptr_t)wl % 8 == 0);
  const int64_t items = (n + 3) / 4;
  const unsigned blocks = (unsigned)std::min<int64_t>((items + 255) / 256, 2048);
  hipLaunchKernelGGL(to_lowp_kernel, dim3(blocks), dim3(256), 0, st, w, n, wl, lt, vec);
  return launch_status("params_to_lowp");
}

}  // namespace ge
