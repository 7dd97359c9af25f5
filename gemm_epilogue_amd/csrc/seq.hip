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

// dE[v, :] = alpha * sum over i with idx[i] == v of dX[i, :], in O(n H + V H):
//
// 1. emb_sort_kernel (one block) orders the positions by token value, stably
//    (a counting sort): NW waves each own a contiguous range of positions and
//    count its values into their own LDS histogram; the histograms give every
//    (value, wave) pair its first slot; each wave then walks its range 64
//    positions at a time, a lane's slot being its wave's cursor for the value
//    plus the number of earlier lanes with the same value.  Positions whose
//    index is outside [0, V) are left out.  seg[v] .. seg[v+1] is then the run
//    of value v in `order`, positions increasing.
// 2. emb_segsum_kernel: block (v, 256 columns), 16 waves; wave w adds rows
//    order[seg[v] + ...] of its sixteenth of the run in order, and the sixteen
//    partial sums are added in wave order.  The order of every sum is fixed, so
//    results are bitwise reproducible, and each dX row is read once.
constexpr int EMB_HIST_INTS = 16384;  // LDS ints for the per-wave histograms

__global__ __launch_bounds__(1024) void emb_sort_kernel(const int32_t *__restrict__ idx, int n, int V, int NW,
                                                        int32_t *__restrict__ order, int32_t *__restrict__ seg) {
  __shared__ int hist[EMB_HIST_INTS];  // [NW][V]: counts, then cursors
  __shared__ int tot[1024];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < NW * V; i += 1024) hist[i] = 0;
  __syncthreads();
  const int per = (n + NW - 1) / NW;
  const int p0 = min(n, wave * per), p1 = min(n, p0 + per);
  if (wave < NW) {
    for (int i = p0 + lane; i < p1; i += 64) {
      const int v = idx[i];
      if ((unsigned)v < (unsigned)V) atomicAdd(&hist[wave * V + v], 1);
    }
  }
  __syncthreads();
  // per value: total over waves; exclusive prefix over values (thread t owns
  // a contiguous block of values); per-wave cursors
  const int vpt = (V + 1023) / 1024;
  const int v0 = min(V, tid * vpt), v1 = min(V, v0 + vpt);
  int run = 0;
  for (int v = v0; v < v1; ++v)
    for (int w = 0; w < NW; ++w) run += hist[w * V + v];
  tot[tid] = run;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {  // inclusive scan of the 1024 block totals
    const int x = tid >= o ? tot[tid - o] : 0;
    __syncthreads();
    tot[tid] += x;
    __syncthreads();
  }
  int base = tot[tid] - run;
  for (int v = v0; v < v1; ++v) {
    seg[v] = base;
    for (int w = 0; w < NW; ++w) {
      const int c = hist[w * V + v];
      hist[w * V + v] = base;
      base += c;
    }
  }
  if (tid == 1023) seg[V] = tot[1023];
  __syncthreads();
  if (wave < NW) {
    for (int c0 = p0; c0 < p1; c0 += 64) {
      const int i = c0 + lane;
      const int v = i < p1 ? idx[i] : -1;
      const bool ok = (unsigned)v < (unsigned)V;
      int rank = 0, cnt = 0;
      for (int l = 0; l < 64; ++l) {
        const int u = __shfl(v, l, 64);
        rank += (l < lane) & (u == v);
        cnt += u == v;
      }
      int *cur = ok ? &hist[wave * V + v] : nullptr;
      const int slot = ok ? *cur + rank : 0;
      if (ok) order[slot] = i;
      // all lanes have read their cursor; one lane per value moves it on
      __builtin_amdgcn_wave_barrier();
      if (ok && rank == cnt - 1) *cur += cnt;
      __builtin_amdgcn_wave_barrier();
    }
  }
}

__global__ __launch_bounds__(1024) void emb_segsum_kernel(const void *__restrict__ dX, int64_t ldx, int xt, int vec,
                                                          const int32_t *__restrict__ order,
                                                          const int32_t *__restrict__ seg, int H, float alpha,
                                                          float *__restrict__ dE, int64_t lde) {
  __shared__ f32x4 part[16][64];
  const int v = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = blockIdx.y * 256 + lane * 4;
  const int s0 = seg[v], s1 = seg[v + 1];
  const int per = (s1 - s0 + 15) / 16;
  const int r0 = min(s1, s0 + wave * per), r1 = min(s1, r0 + per);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (j < H) {
    const bool full = vec && j + 3 < H;
    int r = r0;
    for (; r + 3 < r1; r += 4) {
      float x[4][4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t row = order[r + u];
        if (full) load4_any(dX, row * ldx + j, xt, true, x[u]);
        else
#pragma unroll
          for (int q = 0; q < 4; ++q) x[u][q] = j + q < H ? load_any(dX, row * ldx + j + q, xt) : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[q] += x[u][q];
    }
    for (; r < r1; ++r) {
      const int64_t row = order[r];
      float x[4];
      if (full) load4_any(dX, row * ldx + j, xt, true, x);
      else
#pragma unroll
        for (int q = 0; q < 4; ++q) x[q] = j + q < H ? load_any(dX, row * ldx + j + q, xt) : 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] += x[q];
    }
  }
  part[wave][lane] = acc;
  __syncthreads();
  if (wave == 0 && j < H) {
    f32x4 t = part[0][lane];
    for (int w = 1; w < 16; ++w) t += part[w][lane];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (j + q < H) dE[(int64_t)v * lde + j + q] = alpha * t[q];
  }
}

__device__ __forceinline__ float sigmoid_f(float x) { return 1.f / (1.f + expf(-x)); }

// One forward timestep over B x H, four consecutive hidden units per thread
// (H % 4 == 0, rows 16-byte aligned: one 16-byte access per tensor).
// GI, GH: [B x 3H] f32 rows (r | z | n blocks); hp: h_{t-1} f32 [B x H], or
// NULL for h_0 = 0.  Writes r, z, n (f32, kept for the backward), h (f32) and
// h16 (f16 copy that feeds the next recurrent GEMM; may be NULL).
__global__ __launch_bounds__(256) void gru_fwd_kernel(const float *__restrict__ GI, const float *__restrict__ GH,
                                                      const float *__restrict__ hp, int B, int H,
                                                      float *__restrict__ R, float *__restrict__ Z,
                                                      float *__restrict__ Nn, float *__restrict__ h,
                                                      half_t *__restrict__ h16) {
  const int64_t i4 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i4 >= (int64_t)B * H) return;
  const int b = (int)(i4 / H), j = (int)(i4 % H);
  const int64_t g = (int64_t)b * 3 * H + j;
  const f32x4 gir = *(const f32x4 *)(GI + g), giz = *(const f32x4 *)(GI + g + H),
              gin = *(const f32x4 *)(GI + g + 2 * H);
  const f32x4 ghr = *(const f32x4 *)(GH + g), ghz = *(const f32x4 *)(GH + g + H),
              ghn = *(const f32x4 *)(GH + g + 2 * H);
  const f32x4 hv0 = hp ? *(const f32x4 *)(hp + i4) : f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 r, z, nn, hv;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    r[q] = sigmoid_f(gir[q] + ghr[q]);
    z[q] = sigmoid_f(giz[q] + ghz[q]);
    nn[q] = tanhf(gin[q] + r[q] * ghn[q]);
    hv[q] = (1.f - z[q]) * nn[q] + z[q] * hv0[q];
  }
  *(f32x4 *)(R + i4) = r;
  *(f32x4 *)(Z + i4) = z;
  *(f32x4 *)(Nn + i4) = nn;
  *(f32x4 *)(h + i4) = hv;
  if (h16) *(f16x4 *)(h16 + i4) = f16x4{(half_t)hv[0], (half_t)hv[1], (half_t)hv[2], (half_t)hv[3]};
}

// One backward timestep (same thread mapping).  dh = dh_out + carry (carry =
// gradient reaching h_t from step t+1, NULL for the last step),
//   dn = dh (1 - z), dz = dh (h_prev - n), dh_dir = dh z,
//   dnh = dn (1 - n^2), dr = dnh GH_n,
//   dG_r = dr r (1 - r), dG_z = dz z (1 - z),
//   dGH = [dG_r, dG_z, dnh r] and dGI = [dG_r, dG_z, dnh] (FP16 GEMM inputs).
// hp NULL means h_prev = 0.
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
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  const f32x4 dho = *(const f32x4 *)(dh_out + i4), cin = carry ? *(const f32x4 *)(carry + i4) : zero;
  const f32x4 r = *(const f32x4 *)(R + i4), z = *(const f32x4 *)(Z + i4), nn = *(const f32x4 *)(Nn + i4);
  const f32x4 ghn = *(const f32x4 *)(GH + g + 2 * H);
  const f32x4 h0 = hp ? *(const f32x4 *)(hp + i4) : zero;
  f32x4 dd;
  f16x4 gr, gz, gn, gnh;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float dh = dho[q] + cin[q];
    const float dn = dh * (1.f - z[q]);
    const float dz = dh * (h0[q] - nn[q]);
    const float dnh = dn * (1.f - nn[q] * nn[q]);
    const float dr = dnh * ghn[q];
    dd[q] = dh * z[q];
    gr[q] = (half_t)(dr * r[q] * (1.f - r[q]));
    gz[q] = (half_t)(dz * z[q] * (1.f - z[q]));
    gn[q] = (half_t)(dnh * r[q]);
    gnh[q] = (half_t)dnh;
  }
  *(f32x4 *)(dh_dir + i4) = dd;
  *(f16x4 *)(dGH + g) = gr;
  *(f16x4 *)(dGH + g + H) = gz;
  *(f16x4 *)(dGH + g + 2 * H) = gn;
  *(f16x4 *)(dGI + g) = gr;
  *(f16x4 *)(dGI + g + H) = gz;
  *(f16x4 *)(dGI + g + 2 * H) = gnh;
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

int64_t embedding_grad_ws_bytes(int64_t n, int64_t V) { return (n + V + 1) * 4; }

int embedding_grad_launch(const void *dX, int64_t ldx, int xt, const int32_t *idx, int64_t n, int64_t V,
                          int64_t H, float alpha, float *dE, int64_t lde, void *ws, int64_t ws_bytes,
                          hipStream_t s) {
  if (V == 0 || H == 0) return GE_OK;
  if (ws == nullptr || ws_bytes < embedding_grad_ws_bytes(n, V) || (uintptr_t)ws % 4 != 0) {
    set_error("embedding_grad: needs %lld workspace bytes", (long long)embedding_grad_ws_bytes(n, V));
    return GE_E_WORKSPACE;
  }
  int32_t *order = (int32_t *)ws, *seg = order + n;
  const int NW = (int)std::min<int64_t>(16, EMB_HIST_INTS / V);
  hipLaunchKernelGGL(emb_sort_kernel, dim3(1), dim3(1024), 0, s, idx, (int)n, (int)V, NW, order, seg);
  int st = launch_status("embedding_grad (sort)");
  if (st != GE_OK) return st;
  const int vec = vec_aligned(dX, ldx, dtype_size(xt), 4 * dtype_size(xt));
  hipLaunchKernelGGL(emb_segsum_kernel, dim3((unsigned)V, (unsigned)((H + 255) / 256)), dim3(1024), 0, s, dX, ldx,
                     xt, vec, order, seg, (int)H, alpha, dE, lde);
  return launch_status("embedding_grad (sums)");
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
