// Fused output layer of the MLP step for narrow outputs (C <= 16 classes),
// FP16 storage, for gfx950.
//
// "Capstone 5: train a network with your CUDA kernels": the last layer's
// logits Z = H W + b ("The minimum model"), the stable softmax cross-entropy
// and its gradient dZ ("Read the worked reference"), the bias gradient
// db = sum_rows(dZ) and the masked input gradient dH = (dZ W^T) * [H > 0]
// ("Work through the backward pass").  With ten classes each of these is a
// GEMM or reduction only ten columns wide; as separate launches they are
// bound by launch and memory latency, so one kernel computes them all from
// one pass over H (the weight gradient dW = H^T dZ stays a GEMM).
//
// A prep kernel writes W (D x C, row-major) in the two layouts the MFMAs
// read, zero-padded to 16 classes: W^T (16 x D) and W (D x 16), 128 KiB for
// D = 2048, which stay in L2.  A block of NW waves (eight when D is a
// multiple of 256, else four) takes 16 rows and splits D NW ways: each wave
// accumulates its share of the logits, the shares are added through LDS in
// wave order (so every wave holds the same logits and computes the same loss
// and G), and each wave then forms dH for its own share of the hidden units.
// H is read once; eight waves keep twice the loads in flight per CU.
//  * Z: v_mfma_f32_16x16x32_f16 over D in chunks of 32, the W^T fragment in
//    the first operand slot, so lane l owns Z[row l%16][4(l/16) .. +3].
//  * loss and G: the four lanes of a row (l, l^16, l^32, l^48) reduce the
//    row maximum (lowest index on ties), the sum of the other terms and the
//    label's term; the formulas are those of xent_rows_kernel.  G is rounded
//    to FP16 once and that value is what every later use sees.
//  * dH: per 16 hidden units h0.., v_mfma_f32_16x16x16_f16 with W[h][4q..]
//    and the lane's own four G values gives lane l the four values
//    dH[row l%16][h0 + 4(l/16) .. +3], masked by H of the same elements.
//  * partial sums per block (in a fixed order): column sums of the rounded G
//    and the sum of the row losses, and column sums of the stored dH (the
//    bias gradient of the layer below); final kernels add them over the
//    blocks in a fixed order.
#include "common.h"

namespace ge {

namespace {

constexpr int HEAD_ROWS = 16;   // rows per block (its waves splitting D)
constexpr int HEAD_PART = 17;   // floats per block partial: 16 column sums + loss sum
constexpr int HEAD_DMAX = 2048; // widest input (a wave keeps the ReLU mask of its share in registers)

typedef uint32_t hu32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t hu32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float h2f(uint32_t bits16) {
  return (float)__builtin_bit_cast(half_t, (uint16_t)bits16);
}

// Sum over each row of 16 lanes, valid in the row's lane 15: an inclusive
// scan by DPP row shifts (1, 2, 4, 8; lanes shifted in from outside the row
// read zero), VALU only and in a fixed order.
__device__ __forceinline__ float row16_sum(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x111, 0xf, 0xf, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x112, 0xf, 0xf, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x114, 0xf, 0xf, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x118, 0xf, 0xf, true));
  return v;
}

}  // namespace

// W (D x C) -> WT (16 x D) and WP (D x 16), classes C..15 zero.  Thread i
// writes element i of each layout, so both stores are consecutive across
// the threads; the reads of W (40 KB at D = 2048) gather from L2.
__global__ __launch_bounds__(256) void mlp_head_prep_kernel(const half_t *__restrict__ W, int D, int C,
                                                            half_t *__restrict__ WT, half_t *__restrict__ WP) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= D * 16) return;
  {
    const int k = i >> 4, c = i & 15;  // WP[k][c]
    WP[i] = c < C ? W[(int64_t)k * C + c] : (half_t)0.f;
  }
  {
    const int c = i / D, k = i - c * D;  // WT[c][k]
    WT[i] = c < C ? W[(int64_t)k * C + c] : (half_t)0.f;
  }
}

template <int NW>
__global__ __launch_bounds__(NW * 64) void mlp_head_kernel(const half_t *__restrict__ H, int B, int D,
                                                      const half_t *__restrict__ WT,
                                                      const half_t *__restrict__ WP, const float *__restrict__ bias,
                                                      int C, const int32_t *__restrict__ labels, float gscale,
                                                      float *__restrict__ Z, half_t *__restrict__ G,
                                                      float *__restrict__ row_loss, half_t *__restrict__ dH,
                                                      float *__restrict__ part, float *__restrict__ dpart) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q = lane >> 4, r16 = lane & 15;
  __shared__ f32x4 red[NW][64];

  const int row = blockIdx.x * HEAD_ROWS + r16;
  const bool rok = row < B;
  const half_t *hrow = H + (int64_t)min(row, B - 1) * D;

  // ---- Z = H W (FP32 accumulation), lane: row r16, classes 4q .. 4q+3.
  // Wave w takes chunks w*nch .. (w+1)*nch - 1 of 32 units (nch = D / (32 NW)).  In each chunk
  // lane q supplies units 8q .. 8q+7 -- the units it owns in dH below -- so
  // the ReLU mask [H > 0] is kept here as bits (8 per chunk).  The wave's
  // chunks are loaded 8 at a time, two batches in flight; the loops are
  // unrolled over the widest D so the mask bits stay in registers.
  constexpr int NCH = HEAD_DMAX / (32 * NW);  // chunks per wave at the widest D
  const int nch = D / (32 * NW);
  const int cbase = wave * nch;
  uint32_t mb[NCH / 4];
#pragma unroll
  for (int i = 0; i < NCH / 4; ++i) mb[i] = 0u;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  {
    const half_t *wrow = WT + (int64_t)r16 * D + q * 8 + 32 * cbase;
    const half_t *hp = hrow + q * 8 + 32 * cbase;
    constexpr int U = 8;
    hu32x4 av[2][U], bv[2][U];
    auto load = [&](int bf, int c0) {
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (c0 + u < nch) {
          av[bf][u] = *(const hu32x4 *)(hp + 32 * (c0 + u));
          bv[bf][u] = *(const hu32x4 *)(wrow + 32 * (c0 + u));
        }
    };
    auto mma = [&](int bf, int c0) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + u;
        if (c < nch) {
          const hu32x4 a4 = av[bf][u];
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, bv[bf][u]),
                                                       __builtin_bit_cast(f16x8, a4), acc, 0, 0, 0);
          uint32_t bits = 0u;
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            const uint32_t hb = (a4[t >> 1] >> (16 * (t & 1))) & 0xffffu;
            bits |= (h2f(hb) > 0.f ? 1u : 0u) << t;
          }
          mb[c >> 2] |= bits << (8 * (c & 3));
        }
      }
    };
    load(0, 0);
#pragma unroll
    for (int c0 = 0; c0 < NCH; c0 += 2 * U) {
      if (c0 + U < nch) load(1, c0 + U);
      mma(0, c0);
      if (c0 + U < nch) {
        if (c0 + 2 * U < nch) load(0, c0 + 2 * U);
        mma(1, c0 + U);
      }
    }
  }
  // the NW shares, added in wave order
  red[wave][lane] = acc;
  __syncthreads();
  acc = red[0][lane];
#pragma unroll
  for (int w = 1; w < NW; ++w) acc += red[w][lane];

  // ---- stable softmax cross-entropy of the row, shared by its four lanes
  float z[4];
  float m = -INFINITY;
  int mi = 0x7fffffff;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int c = 4 * q + t;
    z[t] = c < C ? acc[t] + bias[c] : -INFINITY;
    if (c < C && z[t] > m) {
      m = z[t];
      mi = c;
    }
  }
#pragma unroll
  for (int o = 16; o <= 32; o <<= 1) {
    const float om = __shfl_xor(m, o, 64);
    const int oi = __shfl_xor(mi, o, 64);
    if (om > m || (om == m && oi < mi)) {
      m = om;
      mi = oi;
    }
  }
  const int y = rok ? labels[row] : -1;
  const bool yok = (unsigned)y < (unsigned)C;
  float s_rest = 0.f, e_y = 0.f, z_y = 0.f;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int c = 4 * q + t;
    const float e = c < C ? expf(z[t] - m) : 0.f;
    if (c < C && c != mi) s_rest += e;
    if (c == y) {
      e_y = e;
      z_y = z[t];
    }
  }
#pragma unroll
  for (int o = 16; o <= 32; o <<= 1) {
    s_rest += __shfl_xor(s_rest, o, 64);
    e_y += __shfl_xor(e_y, o, 64);  // exactly one lane of the row holds it
    z_y += __shfl_xor(z_y, o, 64);
  }
  const float l1p = log1pf(s_rest);
  const float lse = m + l1p;
  const float s = 1.f + s_rest;
  const float s_noty = (y == mi) ? s_rest : s - e_y;
  const float rl = yok ? (m - z_y) + l1p : NAN;

  // G (rounded to FP16 once), Z and the row loss
  half_t g16[4];
  float gsum[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int c = 4 * q + t;
    const float g = (c == y) ? -(s_noty / s) : expf(z[t] - lse);
    g16[t] = (half_t)(c < C ? gscale * g : 0.f);
    gsum[t] = rok ? (float)g16[t] : 0.f;
  }
  if (rok && wave == 0) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int c = 4 * q + t;
      if (c < C) {
        Z[(int64_t)row * C + c] = z[t];
        G[(int64_t)row * C + c] = g16[t];
      }
    }
    if (q == 0) row_loss[row] = rl;
  }

  // ---- block partials: column sums of G over the block's rows, sum of row losses
  {
    float lsum = (rok && q == 0) ? rl : 0.f;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
#pragma unroll
      for (int t = 0; t < 4; ++t) gsum[t] += __shfl_xor(gsum[t], o, 64);
      lsum += __shfl_xor(lsum, o, 64);
    }
    float *dst = part + (int64_t)blockIdx.x * HEAD_PART;
    if (r16 == 0 && wave == 0) {
#pragma unroll
      for (int t = 0; t < 4; ++t) dst[4 * q + t] = gsum[t];
      if (q == 0) dst[16] = lsum;
    }
  }

  // ---- dH = (G W^T) * [H > 0] per chunk c of 32 units, in two 16x16x16
  // MFMAs whose 16 W rows are units 32c + 8(i/4) + (i%4) (first) and
  // 32c + 8(i/4) + 4 + (i%4) (second) for output row i; lane l then holds
  // units 32c + 8q .. 8q+7 of row r16 -- one 16-byte store, masked by the
  // chunk's bits.  The W loads of 8 chunks are issued together, two batches
  // in flight.
  {
    const f16x4 gy = {g16[0], g16[1], g16[2], g16[3]};
    half_t *drow = dH + (int64_t)row * D + 8 * q + 32 * cbase;
    const int hl = 8 * (r16 >> 2) + (r16 & 3);  // unit of W row r16 in the first MFMA
    const half_t *wq = WP + (int64_t)(hl + 32 * cbase) * 16 + 4 * q;
    constexpr int U = 8;
    f16x4 w0[2][U], w1[2][U];
    auto load = [&](int bf, int c0) {
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (c0 + u < nch) {
          const half_t *w = wq + (int64_t)(c0 + u) * 32 * 16;
          w0[bf][u] = *(const f16x4 *)w;
          w1[bf][u] = *(const f16x4 *)(w + 4 * 16);
        }
    };
    auto compute = [&](int bf, int c0) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + u;
        if (c < nch) {
          const f32x4 z0 = {0.f, 0.f, 0.f, 0.f};
          const f32x4 d0 = __builtin_amdgcn_mfma_f32_16x16x16f16(w0[bf][u], gy, z0, 0, 0, 0);
          const f32x4 d1 = __builtin_amdgcn_mfma_f32_16x16x16f16(w1[bf][u], gy, z0, 0, 0, 0);
          const uint32_t bits = (mb[c >> 2] >> (8 * (c & 3))) & 0xffu;
          f16x8 o;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            o[t] = (half_t)(((bits >> t) & 1u) ? d0[t] : 0.f);
            o[4 + t] = (half_t)(((bits >> (4 + t)) & 1u) ? d1[t] : 0.f);
          }
          if (rok) *(f16x8 *)(drow + 32 * c) = o;
          // column sums of the stored dH over the block's rows (the bias
          // gradient of the layer below), a fixed butterfly over the rows
          float cs[8];
#pragma unroll
          for (int t = 0; t < 8; ++t) cs[t] = row16_sum(rok ? (float)o[t] : 0.f);
          if (r16 == 15) {
            float *dp = dpart + (int64_t)blockIdx.x * D + 32 * (cbase + c) + 8 * q;
            *(f32x4 *)dp = f32x4{cs[0], cs[1], cs[2], cs[3]};
            *(f32x4 *)(dp + 4) = f32x4{cs[4], cs[5], cs[6], cs[7]};
          }
        }
      }
    };
    load(0, 0);
#pragma unroll
    for (int c0 = 0; c0 < NCH; c0 += 2 * U) {
      if (c0 + U < nch) load(1, c0 + U);
      compute(0, c0);
      if (c0 + U < nch) {
        if (c0 + 2 * U < nch) load(0, c0 + 2 * U);
        compute(1, c0 + U);
      }
    }
  }
}

// Block partials -> bias gradient (alpha * column sums) and mean loss, and
// the bias gradient of the layer below from the per-block column sums of dH.
// Block 0: each of the 17 class sums has 32 threads; thread j adds blocks j,
// j+32, ... in order, then a fixed butterfly over the 32 threads.  Blocks
// 1..: 64 columns each; wave w adds partial rows w, w+8, ..., then the eight
// wave sums are added in wave order.
__global__ __launch_bounds__(HEAD_PART * 32) void mlp_head_final_kernel(const float *__restrict__ part,
                                                                         int nblocks, int B, int C, float alpha,
                                                                         float *__restrict__ db,
                                                                         float *__restrict__ loss,
                                                                         const float *__restrict__ dpart, int D,
                                                                         float *__restrict__ db_below) {
  if (blockIdx.x == 0) {
    const int col = threadIdx.x >> 5, j = threadIdx.x & 31;
    float s = 0.f;
    int b = j;
    for (; b + 32 * 7 < nblocks; b += 32 * 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = part[(int64_t)(b + 32 * u) * HEAD_PART + col];
#pragma unroll
      for (int u = 0; u < 8; ++u) s += v[u];
    }
    for (; b < nblocks; b += 32) s += part[(int64_t)b * HEAD_PART + col];
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
    if (j == 0) {
      if (col < C) db[col] = alpha * s;
      if (col == 16) loss[0] = B > 0 ? s / (float)B : 0.f;
    }
    return;
  }
  __shared__ float red[7][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;  // wave 8 (half a wave) idles
  const int n = (blockIdx.x - 1) * 64 + lane;
  float s = 0.f;
  if (wave < 8 && n < D) {
    int k = wave;
    for (; k + 8 * 7 < nblocks; k += 8 * 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = dpart[(int64_t)(k + 8 * u) * D + n];
#pragma unroll
      for (int u = 0; u < 8; ++u) s += v[u];
    }
    for (; k < nblocks; k += 8) s += dpart[(int64_t)k * D + n];
  }
  if (wave > 0 && wave < 8) red[wave - 1][lane] = s;
  __syncthreads();
  if (wave == 0 && n < D) {
#pragma unroll
    for (int w = 0; w < 7; ++w) s += red[w][lane];
    db_below[n] = alpha * s;
  }
}

bool head_supported(int64_t B, int64_t D, int64_t C) {
  return B >= 1 && C >= 1 && C <= 16 && D >= 128 && D <= HEAD_DMAX && D % 128 == 0;
}

// loss / class-column partials, the two layouts of W, then the per-block
// column sums of dH (each region 256-byte aligned)
int64_t head_ws_bytes(int64_t B, int64_t D) {
  const int64_t nb = (B + HEAD_ROWS - 1) / HEAD_ROWS;
  const int64_t p = (nb * HEAD_PART * 4 + 255) / 256 * 256;
  return p + 2 * D * 16 * 2 + nb * D * 4;
}

int head_launch(const half_t *H, int64_t B, int64_t D, const half_t *W, const float *bias, int64_t C,
                const int32_t *labels, float gscale, float alpha, float *Z, half_t *G, float *row_loss,
                half_t *dH, float *db, float *db_below, float *loss, void *ws, hipStream_t st) {
  const int nblocks = (int)((B + HEAD_ROWS - 1) / HEAD_ROWS);
  float *part = (float *)ws;
  const int64_t p = ((int64_t)nblocks * HEAD_PART * 4 + 255) / 256 * 256;
  half_t *WT = (half_t *)((char *)ws + p);
  half_t *WP = WT + D * 16;
  float *dpart = (float *)(WP + D * 16);
  hipLaunchKernelGGL(mlp_head_prep_kernel, dim3((unsigned)((D * 16 + 255) / 256)), dim3(256), 0, st, W, (int)D,
                     (int)C, WT, WP);
  int s = launch_status("mlp head (prep)");
  if (s != GE_OK) return s;
  if (D % 256 == 0)
    hipLaunchKernelGGL(mlp_head_kernel<8>, dim3(nblocks), dim3(512), 0, st, H, (int)B, (int)D, (const half_t *)WT,
                       (const half_t *)WP, bias, (int)C, labels, gscale, Z, G, row_loss, dH, part, dpart);
  else
    hipLaunchKernelGGL(mlp_head_kernel<4>, dim3(nblocks), dim3(256), 0, st, H, (int)B, (int)D, (const half_t *)WT,
                       (const half_t *)WP, bias, (int)C, labels, gscale, Z, G, row_loss, dH, part, dpart);
  s = launch_status("mlp head");
  if (s != GE_OK) return s;
  hipLaunchKernelGGL(mlp_head_final_kernel, dim3((unsigned)(1 + (D + 63) / 64)), dim3(HEAD_PART * 32), 0, st,
                     (const float *)part, nblocks, (int)B, (int)C, alpha, db, loss, (const float *)dpart, (int)D,
                     db_below);
  return launch_status("mlp head (final)");
}

}  // namespace ge
