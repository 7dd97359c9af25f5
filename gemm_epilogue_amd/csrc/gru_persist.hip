// Persistent recurrence of the byte-level GRU LM: all T timesteps of the
// forward recurrence in one launch, and all T timesteps of backpropagation
// through time in another, with each block's slice of the recurrent weight
// W_h resident in LDS for the whole launch ("The Work Moved Down a Layer",
// section "Keep state resident"; the tiny serialized per-timestep jobs are
// the cost that section and "Why This Belongs in a Game Engine" point at).
//
// Block b of the NB = H / 16 blocks owns hidden units u0 = 16 b .. u0 + 15.
//   forward step t:  GH[:, g H + u0 + j] = h16_{t-1} W_h[:, g H + u0 + j] + b_h
//                    for the three gate blocks g (r, z, n) and j < 16 -- a
//                    [B x H] x [H x 48] product on MFMA with the 48 columns of
//                    W_h in LDS -- then the gate arithmetic for its units, the
//                    stores of r, z, n, h, the FP16 copy of h and GH; then one
//                    grid-wide barrier (every block needs all of h16_t next).
//   backward step t: dh = dh_out + carry for its units (the carry is the
//                    block's own, kept in registers), the gate backward, the
//                    stores of dGH, dGI; one grid-wide barrier (every block
//                    needs all of dGH_t); then carry = dh z + dGH_t W_h[u0 +
//                    j, :]^T, a [B x 3H] x [3H x 16] product with the 16 rows
//                    of W_h in LDS.
// Wave w of a block handles batch rows 16 w .. 16 w + 15, so B <= 64 and
// B % 16 == 0; H % 16 == 0 and the W_h slice (48 H or 48 H bytes) must fit LDS.
// The gate arithmetic and every stored tensor are those of gru_fwd_kernel /
// gru_bwd_kernel (seq.hip); only the GEMM's summation order differs.
//
// The grid barrier is a counter that every block increments once per barrier
// and polls until it reaches (barriers so far) x NB.  The launch is
// cooperative, so all blocks are resident; the poll is still bounded, and a
// block that gives up sets an error word and every block leaves the kernel.
#include "common.h"

namespace ge {

namespace {

typedef __attribute__((address_space(3))) f16x8 lds_f16x8_t;

constexpr int kSpinLimit = 1 << 22;  // polls of about 64 cycles each before giving up

// returns false when the barrier timed out (or another block reported that)
__device__ __forceinline__ bool grid_barrier(unsigned *count, unsigned target, unsigned *err) {
  __syncthreads();
  __shared__ int ok;
  if (threadIdx.x == 0) {
    __threadfence();
    atomicAdd(count, 1u);
    int good = 1;
    int spins = 0;
    while (__hip_atomic_load(count, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) < target) {
      if (__hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u || ++spins > kSpinLimit) {
        atomicOr(err, 1u);
        good = 0;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    __threadfence();
    ok = good;
  }
  __syncthreads();
  return ok != 0;
}

__device__ __forceinline__ float sigm(float x) { return 1.f / (1.f + expf(-x)); }

// 16-byte chunk c of LDS row r sits at chunk c ^ (r & 15): the 16 lanes of a
// fragment read (16 rows, one chunk) hit 16 distinct bank groups
__device__ __forceinline__ int swz(int r, int c) { return c ^ (r & 15); }

}  // namespace

__global__ __launch_bounds__(256, 1) void gru_rec_fwd_kernel(const float *__restrict__ GI, const half_t *__restrict__ Wh,
                                                             const float *__restrict__ bh, int B, int H, int T,
                                                             float *__restrict__ GH, float *__restrict__ R,
                                                             float *__restrict__ Z, float *__restrict__ Nn,
                                                             float *__restrict__ HS, half_t *__restrict__ H16,
                                                             unsigned *__restrict__ sync) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  half_t *w = (half_t *)smem;  // [48][H]: row c = gate c / 16, unit c % 16; k contiguous, chunks swizzled
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int u0 = blockIdx.x * 16;
  const int H3 = 3 * H, KC = H / 8;  // 16-byte chunks per LDS row
  // W_h columns of this block, transposed into LDS: thread takes (k, gate),
  // reads the 16 units of row k of that gate block and writes them to 16 rows
  for (int p = tid; p < H * 3; p += 256) {
    const int k = p / 3, g = p % 3;
    const f16x8 a = *(const f16x8 *)(Wh + (int64_t)k * H3 + g * H + u0);
    const f16x8 b = *(const f16x8 *)(Wh + (int64_t)k * H3 + g * H + u0 + 8);
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int row = g * 16 + u;
      const int c = k >> 3;
      w[row * H + swz(row, c) * 8 + (k & 7)] = u < 8 ? a[u] : b[u - 8];
    }
  }
  const int m = wave * 16 + (lane & 15);  // batch row of this lane
  const int j0 = 4 * (lane >> 4);         // its four units within the block
  const bool live = wave * 16 < B;
  f32x4 bias[3];
#pragma unroll
  for (int g = 0; g < 3; ++g) bias[g] = *(const f32x4 *)(bh + g * H + u0 + j0);
  __syncthreads();
  for (int t = 0; t < T; ++t) {
    if (live) {
      f32x4 acc[3] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
      if (t > 0) {
        // h16_{t-1} row m, chunks of 32 k; the lane's 8 k values of each chunk
        const half_t *hrow = H16 + ((int64_t)t * B + m) * H + 8 * (lane >> 4);
        for (int k0 = 0; k0 < H; k0 += 256) {
          f16x8 hv[8];
#pragma unroll
          for (int s = 0; s < 8; ++s) hv[s] = *(const f16x8 *)(hrow + k0 + 32 * s);
#pragma unroll
          for (int s = 0; s < 8; ++s) {
            const int c = (k0 + 32 * s) / 8 + (lane >> 4);
#pragma unroll
            for (int g = 0; g < 3; ++g) {
              const int row = g * 16 + (lane & 15);
              const f16x8 wv = *(const lds_f16x8_t *)(w + row * H + swz(row, c) * 8);
              acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wv, hv[s], acc[g], 0, 0, 0);
            }
          }
        }
      }
      // lane holds GH[m][g H + u0 + j0 .. +3] (before the bias)
      const int64_t row = (int64_t)t * B + m;
      const float *gi = GI + row * H3 + u0 + j0;
      const f32x4 gir = *(const f32x4 *)gi, giz = *(const f32x4 *)(gi + H), gin = *(const f32x4 *)(gi + 2 * H);
      const f32x4 hp = t > 0 ? *(const f32x4 *)(HS + (row - B) * H + u0 + j0) : f32x4{0.f, 0.f, 0.f, 0.f};
      f32x4 gh[3], r, z, nn, hv;
#pragma unroll
      for (int g = 0; g < 3; ++g) gh[g] = acc[g] + bias[g];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        r[q] = sigm(gir[q] + gh[0][q]);
        z[q] = sigm(giz[q] + gh[1][q]);
        nn[q] = tanhf(gin[q] + r[q] * gh[2][q]);
        hv[q] = (1.f - z[q]) * nn[q] + z[q] * hp[q];
      }
      const int64_t o = row * H + u0 + j0;
      *(f32x4 *)(R + o) = r;
      *(f32x4 *)(Z + o) = z;
      *(f32x4 *)(Nn + o) = nn;
      *(f32x4 *)(HS + o) = hv;
      *(f16x4 *)(H16 + (row + B) * H + u0 + j0) = f16x4{(half_t)hv[0], (half_t)hv[1], (half_t)hv[2], (half_t)hv[3]};
#pragma unroll
      for (int g = 0; g < 3; ++g) *(f32x4 *)(GH + row * H3 + g * H + u0 + j0) = gh[g];
    }
    if (t + 1 < T && !grid_barrier(sync, (unsigned)((t + 1) * gridDim.x), sync + 1)) return;
  }
}

__global__ __launch_bounds__(256, 1) void gru_rec_bwd_kernel(const float *__restrict__ dh_out,
                                                             const half_t *__restrict__ Wh, const float *__restrict__ R,
                                                             const float *__restrict__ Z, const float *__restrict__ Nn,
                                                             const float *__restrict__ GH, const float *__restrict__ HS,
                                                             int B, int H, int T, half_t *__restrict__ dGH,
                                                             half_t *__restrict__ dGI, unsigned *__restrict__ sync) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  half_t *w = (half_t *)smem;  // [16][3H]: rows u0 .. u0 + 15 of W_h, chunks swizzled
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int u0 = blockIdx.x * 16;
  const int H3 = 3 * H, KC = H3 / 8;
  for (int p = tid; p < 16 * KC; p += 256) {
    const int u = p / KC, c = p % KC;
    *(f16x8 *)(w + u * H3 + swz(u, c) * 8) = *(const f16x8 *)(Wh + (int64_t)(u0 + u) * H3 + 8 * c);
  }
  const int m = wave * 16 + (lane & 15);
  const int j0 = 4 * (lane >> 4);
  const bool live = wave * 16 < B;
  f32x4 carry = {0.f, 0.f, 0.f, 0.f};
  __syncthreads();
  int nbar = 0;
  for (int t = T - 1; t >= 0; --t) {
    f32x4 dd = {0.f, 0.f, 0.f, 0.f};
    if (live) {
      const int64_t row = (int64_t)t * B + m;
      const int64_t o = row * H + u0 + j0;
      const f32x4 dho = *(const f32x4 *)(dh_out + o);
      const f32x4 r = *(const f32x4 *)(R + o), z = *(const f32x4 *)(Z + o), nn = *(const f32x4 *)(Nn + o);
      const f32x4 ghn = *(const f32x4 *)(GH + row * H3 + 2 * H + u0 + j0);
      const f32x4 h0 = t > 0 ? *(const f32x4 *)(HS + o - (int64_t)B * H) : f32x4{0.f, 0.f, 0.f, 0.f};
      f16x4 gr, gz, gn, gnh;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float dh = dho[q] + carry[q];
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
      const int64_t g0 = row * H3 + u0 + j0;
      *(f16x4 *)(dGH + g0) = gr;
      *(f16x4 *)(dGH + g0 + H) = gz;
      *(f16x4 *)(dGH + g0 + 2 * H) = gn;
      *(f16x4 *)(dGI + g0) = gr;
      *(f16x4 *)(dGI + g0 + H) = gz;
      *(f16x4 *)(dGI + g0 + 2 * H) = gnh;
    }
    if (t == 0) break;
    ++nbar;
    if (!grid_barrier(sync, (unsigned)(nbar * gridDim.x), sync + 1)) return;
    if (live) {
      // carry for step t-1: dh z + dGH_t[m, :] W_h[u0 + j, :]^T over the 3H columns
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      const half_t *grow = dGH + ((int64_t)t * B + m) * H3 + 8 * (lane >> 4);
      for (int k0 = 0; k0 < H3; k0 += 256) {
        f16x8 gv[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) gv[s] = *(const f16x8 *)(grow + k0 + 32 * s);
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const int c = (k0 + 32 * s) / 8 + (lane >> 4);
          const int wr = lane & 15;
          const f16x8 wv = *(const lds_f16x8_t *)(w + wr * H3 + swz(wr, c) * 8);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(wv, gv[s], acc, 0, 0, 0);
        }
      }
      carry = acc + dd;
    }
  }
}

// ---- launchers ------------------------------------------------------------------
bool gru_persist_supported(int64_t B, int64_t H) {
  if (B < 1 || B > 64 || B % 16 != 0 || H % 256 != 0 || H < 256) return false;
  if ((int64_t)48 * H * 2 > 160 * 1024) return false;
  int dev = 0, coop = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  if (hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) != hipSuccess || !coop) return false;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return false;
  return H / 16 <= cus;
}

namespace {
int coop_launch(const void *fn, int blocks, size_t lds, void **args, hipStream_t s, const char *what) {
  // the dynamic LDS above the default limit has to be granted per kernel
  static size_t granted[2] = {0, 0};
  const int which = fn == (const void *)gru_rec_fwd_kernel ? 0 : 1;
  if (lds > granted[which]) {
    if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess) {
      (void)hipGetLastError();
      set_error("%s: cannot grant %zu bytes of LDS", what, lds);
      return GE_E_LAUNCH;
    }
    granted[which] = lds;
  }
  hipError_t e = hipLaunchCooperativeKernel(fn, dim3(blocks), dim3(256), args, (unsigned)lds, s);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    set_error("%s: cooperative launch failed: %s", what, hipGetErrorString(e));
    return GE_E_LAUNCH;
  }
  return launch_status(what);
}
}  // namespace

int fill_zero_launch(void *p, int64_t bytes, hipStream_t s);

// sync: device unsigned [2] (barrier counter, error word), cleared here first
int gru_rec_fwd_launch(const float *GI, const half_t *Wh, const float *bh, int B, int H, int T, float *GH, float *R,
                       float *Z, float *N, float *HS, half_t *H16, unsigned *sync, hipStream_t s) {
  int st = fill_zero_launch(sync, 2 * sizeof(unsigned), s);
  if (st != GE_OK) return st;
  void *args[] = {&GI, &Wh, &bh, &B, &H, &T, &GH, &R, &Z, &N, &HS, &H16, &sync};
  return coop_launch((const void *)gru_rec_fwd_kernel, H / 16, (size_t)48 * H * 2, args, s, "gru recurrence (forward)");
}

int gru_rec_bwd_launch(const float *dh_out, const half_t *Wh, const float *R, const float *Z, const float *N,
                       const float *GH, const float *HS, int B, int H, int T, half_t *dGH, half_t *dGI, unsigned *sync,
                       hipStream_t s) {
  int st = fill_zero_launch(sync, 2 * sizeof(unsigned), s);
  if (st != GE_OK) return st;
  void *args[] = {&dh_out, &Wh, &R, &Z, &N, &GH, &HS, &B, &H, &T, &dGH, &dGI, &sync};
  return coop_launch((const void *)gru_rec_bwd_kernel, H / 16, (size_t)16 * 3 * H * 2, args, s,
                     "gru recurrence (backward)");
}

}  // namespace ge
