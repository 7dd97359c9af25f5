// The whole training step of a one-hidden-layer FP32 ReLU MLP (784-256-10 at
// batch 128 is the case it is built for) as ONE launch of resident blocks: the
// persistent single-kernel step that removes the per-launch cost the step's
// ten small kernels pay ("Capstone 5: train a network with your CUDA
// kernels", "Explain a different result" and "Checked results": the step
// there is bound by kernel launches, not by arithmetic).
//
// The arithmetic is the launch chain's ("The minimum model", "Work through
// the backward pass", "Read the worked reference"):
//   phase 1  H = ReLU(X W1 + b1)                         16x16 tiles on the
//            FP32 MFMA (v_mfma_f32_16x16x4f32), K split over the 4 waves of
//            a block and summed in LDS in wave order;
//   -- grid barrier --
//   phase 2  one wave per batch row: Z = H W2 + b2, the stable softmax CE
//            (row loss, dZ = (p - onehot) / B), and the masked input gradient
//            dH = (dZ W2^T) * (H > 0), with W2 in LDS since the launch began;
//   -- grid barrier --
//   phase 3  dW1 = X^T dH and dW2 = H^T dZ as 16x16 MFMA tiles over K = B,
//            each layer input extended by a row of ones so one more tile row
//            yields db1 / db2 (the column sums of dH / dZ); the mean loss;
//            and the momentum update of every parameter right where its
//            gradient is formed: vel = mu v - lr g; v = vel; w += vel.
// The step writes what the chain writes: the flat gradient, H, Z, dZ, the row
// losses and dH in the same workspace slots, and the mean loss.
//
// MFMA operand mapping of v_mfma_f32_16x16x4f32 (one 16x16 block, K = 4):
// lane l supplies A[l % 16][l / 16] and B[l / 16][l % 16] and holds
// D[4 (l / 16) + q][l % 16] in accumulator element q.  Within a 16-wide k
// chunk, MFMA j of the chunk gives lane group g the k index 4 g + j, so a
// lane's four A values of the chunk are one 16-byte load.
#include "common.h"
#include "persist.h"

namespace ge {

namespace {

constexpr int kMaxD0 = 1024, kMaxD1 = 512, kMaxB = 128;
constexpr int kMaxChunks = kMaxD0 / 16 / 4;  // 16-wide k chunks of one wave in phase 1
constexpr int kKB = kMaxB / 16;              // 16-row batch chunks of a phase-3 tile
constexpr int kW2Regs = kMaxD1 * 16 / 256;   // W2 values a thread stages into LDS
constexpr int kPersistBlocks = 128;          // >= kMaxB / 4: phase 2 takes one row per wave

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// A phase-3 gradient tile: rows m0 .. m0 + 15 of S^T D over the batch, where
// S is the layer input (rows < srows) extended by a row of ones (row srows),
// so the tile that holds row srows also yields the bias gradient, the column
// sum of D.  D has ncols columns; the tile covers n0 .. n0 + 15.
struct GradTile {
  const float *S, *D;
  int srows, ncols, m0, n0;
  int64_t wbase, bbase;  // flat offsets of the weight [srows x ncols] and the bias [ncols]
};

__device__ __forceinline__ GradTile grad_tile(const MlpPersistArgs &a, int it, int nw2, int nt1) {
  GradTile t;
  const int D0 = a.D0, D1 = a.D1, C = a.C;
  const int64_t oB1 = (int64_t)D0 * D1, oW2 = oB1 + D1, oB2 = oW2 + (int64_t)D1 * C;
  if (it < nw2) {  // dW2 = H^T dZ and db2
    t.S = a.H; t.D = a.Gz; t.srows = D1; t.ncols = C; t.m0 = it * 16; t.n0 = 0; t.wbase = oW2; t.bbase = oB2;
  } else {         // dW1 = X^T dH and db1
    const int i = it - nw2;
    t.S = a.X; t.D = a.dH; t.srows = D0; t.ncols = D1; t.m0 = (i / nt1) * 16; t.n0 = (i % nt1) * 16;
    t.wbase = 0; t.bbase = oB1;
  }
  return t;
}

// flat index of the parameter that tile row r, column n updates, or -1
__device__ __forceinline__ int64_t tile_param(const GradTile &t, int r, int n) {
  if (n >= t.ncols) return -1;
  return r < t.srows ? t.wbase + (int64_t)r * t.ncols + n : (r == t.srows ? t.bbase + n : -1);
}

// the tile's operands, and the parameters and velocities its lane updates
__device__ __forceinline__ void load_tile(const MlpPersistArgs &a, const GradTile &t, int B, int nkb, int r16, int g4,
                                          float x[kKB][4], float y[kKB][4], float pw[4], float vw[4]) {
  const int m = t.m0 + r16, n = t.n0 + r16;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t i = tile_param(t, t.m0 + 4 * g4 + q, n);
    pw[q] = i >= 0 ? a.P[i] : 0.f;
    vw[q] = i >= 0 ? a.V[i] : 0.f;
  }
#pragma unroll
  for (int kb = 0; kb < kKB; ++kb) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int b = kb * 16 + 4 * g4 + j;
      const bool ok = kb < nkb && b < B;
      x[kb][j] = !ok ? 0.f : m < t.srows ? t.S[(int64_t)b * t.srows + m] : (m == t.srows ? 1.f : 0.f);
      y[kb][j] = ok && n < t.ncols ? t.D[(int64_t)b * t.ncols + n] : 0.f;
    }
  }
}

__device__ __forceinline__ void finish_tile(const MlpPersistArgs &a, const GradTile &t, int nkb, int r16, int g4,
                                            const float x[kKB][4], const float y[kKB][4], const float pw[4],
                                            const float vw[4]) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kb = 0; kb < kKB; ++kb) {
    if (kb < nkb) {
#pragma unroll
      for (int j = 0; j < 4; ++j) acc = mfma4(x[kb][j], y[kb][j], acc);
    }
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t i = tile_param(t, t.m0 + 4 * g4 + q, t.n0 + r16);
    if (i >= 0) {
      const float vel = a.mu * vw[q] - a.lr * acc[q];
      a.Gr[i] = acc[q];
      a.V[i] = vel;
      a.P[i] = pw[q] + vel;
    }
  }
}

}  // namespace

__global__ __launch_bounds__(256, 1) void mlp_persist_kernel(MlpPersistArgs a) {
  __shared__ __attribute__((aligned(16))) float w2s[kMaxD1 * 16];  // W2 [D1][16], zero beyond C
  __shared__ f32x4 red[3][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int B = a.B, D0 = a.D0, D1 = a.D1, C = a.C;
  const int64_t oB1 = (int64_t)D0 * D1, oW2 = oB1 + D1, oB2 = oW2 + (int64_t)D1 * C;
  const float *W1 = a.P, *b1 = a.P + oB1, *W2 = a.P + oW2, *b2 = a.P + oB2;

  // W2 into registers now, into LDS after phase 1: its latency hides there
  float w2r[kW2Regs];
#pragma unroll
  for (int i = 0; i < kW2Regs; ++i) {
    const int e = tid + 256 * i, k = e >> 4, c = e & 15;
    w2r[i] = k < D1 && c < C ? W2[(int64_t)k * C + c] : 0.f;
  }

  // ---- phase 1: H = ReLU(X W1 + b1) ---------------------------------------
  const int mt1 = (B + 15) / 16, nt1 = D1 / 16, nkc = (D0 + 15) / 16;
  for (int tile = blockIdx.x; tile < mt1 * nt1; tile += gridDim.x) {
    const int m0 = (tile / nt1) * 16, n0 = (tile % nt1) * 16;
    const int row = m0 + r16, col = n0 + r16;
    f32x4 av[kMaxChunks];
    float bv[kMaxChunks][4];
#pragma unroll
    for (int i = 0; i < kMaxChunks; ++i) {
      const int kc = wave + 4 * i;
      const int k = kc * 16 + 4 * g4;
      const bool ok = kc < nkc && k < D0;
      av[i] = ok && row < B ? *(const f32x4 *)(a.X + (int64_t)row * D0 + k) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[i][j] = ok ? W1[(int64_t)(k + j) * D1 + col] : 0.f;
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < kMaxChunks; ++i) {
      if (wave + 4 * i < nkc) {
#pragma unroll
        for (int j = 0; j < 4; ++j) acc = mfma4(av[i][j], bv[i][j], acc);
      }
    }
    if (wave > 0) red[wave - 1][lane] = acc;
    __syncthreads();
    if (wave == 0) {
      const f32x4 s = ((acc + red[0][lane]) + red[1][lane]) + red[2][lane];
      const float bias = b1[col];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = m0 + 4 * g4 + q;
        if (r < B) a.H[(int64_t)r * D1 + col] = fmaxf(s[q] + bias, 0.f);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < kW2Regs; ++i) w2s[tid + 256 * i] = w2r[i];
  // phase 2 takes one batch row per wave (the grid has at least B / 4
  // blocks); its label and the output bias do not wait for the barrier
  const int b = blockIdx.x * 4 + wave;
  const int y = b < B ? a.labels[b] : 0;
  const float bias2 = r16 < C ? b2[r16] : 0.f;
  if (!grid_barrier(a.sync, gridDim.x, a.sync + 1)) {
    if (tid == 0) a.loss[0] = NAN;  // a barrier that gave up leaves the step undone: say so in the loss
    return;
  }

  // ---- phase 2: logits, softmax CE, dZ, dH (one wave per row) -------------
  const float gscale = 1.f / (float)B;
  if (b < B) {
    const float *hrow = a.H + (int64_t)b * D1;
    // lane (quarter g4, class r16): its quarter's share of z_c
    const int ql = D1 / 4;
    float zp = 0.f;
#pragma unroll 8
    for (int i = 0; i < ql; i += 4) {
      const int k = g4 * ql + i;
      const f32x4 h = *(const f32x4 *)(hrow + k);
#pragma unroll
      for (int e = 0; e < 4; ++e) zp += h[e] * w2s[(k + e) * 16 + r16];
    }
    zp += __shfl_xor(zp, 16, 64);
    zp += __shfl_xor(zp, 32, 64);
    const bool cls = r16 < C;
    const float z = cls ? zp + bias2 : -INFINITY;
    // max and lowest index of the max over the 16 classes
    float m = z;
    int mi = cls ? r16 : 0x7fffffff;
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) {
      const float om = __shfl_xor(m, o, 64);
      const int oi = __shfl_xor(mi, o, 64);
      if (om > m || (om == m && oi < mi)) { m = om; mi = oi; }
    }
    const bool yok = (unsigned)y < (unsigned)C;
    const float e = cls ? expf(z - m) : 0.f;
    float s_rest = r16 != mi ? e : 0.f;
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) s_rest += __shfl_xor(s_rest, o, 64);
    const float e_y = __shfl(e, yok ? y : 0, 64);
    const float z_y = __shfl(z, yok ? y : 0, 64);
    const float l1p = log1pf(s_rest);
    const float lse = m + l1p;
    const float s = 1.f + s_rest;
    const float s_noty = (y == mi) ? s_rest : s - e_y;
    const float gz = gscale * ((r16 == y) ? -(s_noty / s) : expf(z - lse));
    if (lane == 0) a.row_loss[b] = yok ? (m - z_y) + l1p : NAN;
    if (g4 == 0 && cls) {
      a.Zl[(int64_t)b * C + r16] = z;
      a.Gz[(int64_t)b * C + r16] = gz;
    }
    float gc[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) gc[c] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cls ? gz : 0.f), c));
    for (int k4 = lane; k4 < D1 / 4; k4 += 64) {
      const int k = 4 * k4;
      const f32x4 h = *(const f32x4 *)(hrow + k);
      f32x4 d;
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const float *wr = w2s + (k + e2) * 16;
        float t = 0.f;
#pragma unroll
        for (int c = 0; c < 16; ++c) t += gc[c] * wr[c];
        d[e2] = h[e2] > 0.f ? t : 0.f;
      }
      *(f32x4 *)(a.dH + (int64_t)b * D1 + k) = d;
    }
  }
  if (!grid_barrier(a.sync, 2 * gridDim.x, a.sync + 1)) {
    if (tid == 0) a.loss[0] = NAN;
    return;
  }

  // ---- phase 3: gradients and the momentum update --------------------------
  // the last wave of the grid also forms the mean loss
  const int gw = blockIdx.x * 4 + wave, nw = gridDim.x * 4;
  if (gw == nw - 1) {
    float t = 0.f;
    for (int b = lane; b < B; b += 64) t += a.row_loss[b];
    t = wave_sum(t);
    if (lane == 0) a.loss[0] = t / (float)B;
  }
  // tiles: (D1 + 1) / 16 rounded up for dW2 + db2, then (D0 + 1) / 16 x D1 / 16
  // for dW1 + db1; a wave loads its next tile while it multiplies this one
  const int nkb = (B + 15) / 16, nw2 = (D1 + 16) / 16, mt3 = (D0 + 16) / 16;
  const int items = nw2 + mt3 * nt1;
  float xa[kKB][4], ya[kKB][4], xb[kKB][4], yb[kKB][4], pa[4], va[4], pb[4], vb[4];
  int it = gw;
  GradTile ta, tb;
  if (it < items) {
    ta = grad_tile(a, it, nw2, nt1);
    load_tile(a, ta, B, nkb, r16, g4, xa, ya, pa, va);
  }
  while (it < items) {
    int nx = it + nw;
    if (nx < items) {
      tb = grad_tile(a, nx, nw2, nt1);
      load_tile(a, tb, B, nkb, r16, g4, xb, yb, pb, vb);
    }
    finish_tile(a, ta, nkb, r16, g4, xa, ya, pa, va);
    it = nx;
    if (it >= items) break;
    nx = it + nw;
    if (nx < items) {
      ta = grad_tile(a, nx, nw2, nt1);
      load_tile(a, ta, B, nkb, r16, g4, xa, ya, pa, va);
    }
    finish_tile(a, tb, nkb, r16, g4, xb, yb, pb, vb);
    it = nx;
  }
}

bool mlp_persist_supported(int64_t B, int64_t D0, int64_t D1, int64_t C) {
  if (B < 1 || B > kMaxB || D0 < 4 || D0 > kMaxD0 || D0 % 4 != 0) return false;
  if (D1 < 64 || D1 > kMaxD1 || D1 % 64 != 0 || C < 1 || C > 16) return false;
  // every block of the grid must be resident at once for its barriers
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return false;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void *)mlp_persist_kernel, 256, 0) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  return (int64_t)per_cu * cus >= kPersistBlocks;
}

int fill_zero_launch(void *p, int64_t bytes, hipStream_t s);

int mlp_persist_launch(const MlpPersistArgs &args, hipStream_t s) {
  if ((uintptr_t)args.X % 16 != 0 || (uintptr_t)args.H % 16 != 0 || (uintptr_t)args.dH % 16 != 0) {
    set_error("mlp_train_step (persistent): X, H and dH must be 16-byte aligned");
    return GE_E_INVALID;
  }
  int st = fill_zero_launch(args.sync, 2 * sizeof(unsigned), s);
  if (st != GE_OK) return st;
  // An ordinary launch: the grid is one block per compute unit on at most
  // half of them, and mlp_persist_supported checked that it fits resident;
  // a cooperative launch adds about 20 us of host-side work per step here.
  hipLaunchKernelGGL(mlp_persist_kernel, dim3(kPersistBlocks), dim3(256), 0, s, args);
  return launch_status("mlp_train_step (persistent)");
}

}  // namespace ge
