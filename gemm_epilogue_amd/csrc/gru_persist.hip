// Persistent recurrence of the byte-level GRU LM: all T timesteps of the
// forward recurrence in one launch, and all T timesteps of backpropagation
// through time in another, with each block's slice of the recurrent weight
// W_h resident in LDS for the whole launch ("The Work Moved Down a Layer",
// section "Keep state resident"; the tiny serialized per-timestep jobs are
// the cost that section and "Why This Belongs in a Game Engine" point at).
//
// Forward: block g of the H / 16 blocks owns hidden units u0 = 16 g .. u0 + 15
// for all B rows; wave w takes batch rows 16 w .. 16 w + 15.
//   step t: GH[rows, g' H + u0 + j] = h16_{t-1}[rows] W_h[:, g' H + u0 + j] + b_h
//           for the three gate blocks g' (r, z, n) and j < 16 -- a [16 x H] x
//           [H x 48] product per wave on MFMA with the 48 columns of W_h in
//           LDS -- then the gate arithmetic, the stores of r, z, n, h, the FP16
//           copy of h and GH, and one grid barrier (every block needs all of
//           h16_t next).  A lane's h_{t-1} is its own previous output
//           (registers), the next step's GI is fetched before the barrier, and
//           a wave issues all of its h16 loads before its first MFMA.
// Backward: block (g, q) of the (H / 16) x (B / 16) blocks owns units u0 =
// 16 g .. u0 + 15 for batch rows 16 q .. 16 q + 15; a row group q is an
// independent recurrence, so its H / 16 blocks meet at a barrier of their own.
//   step t: dh = dh_out + carry for the block's units and rows (the carry
//           stays in registers), the gate backward, the stores of dGH, dGI,
//           the row group's barrier, then carry = dh z + dGH_t[rows]
//           W_h[u0 + j, :]^T, a [16 x 3H] x [3H x 16] product with the 16 rows
//           of W_h in LDS, 3H split over the block's four waves and summed in
//           LDS in wave order.
// The two layouts are the measured better ones for each direction: splitting
// the forward by row group as well (256 blocks, K split over the waves) made
// a step 12.3 us instead of 11.4 (its barrier fences scale with the block
// count), while the backward went from 16.6 us (64 blocks of 1,024 threads)
// to 12.5.  B <= 64 and B % 16 == 0; H = 256 KB for KB = 1 .. 4, so the W_h
// slice fits LDS and a lane's loads of one step fit its registers.  The gate
// arithmetic and every stored tensor are those of gru_fwd_kernel /
// gru_bwd_kernel (seq.hip); only the GEMM's summation order differs.
#include "common.h"
#include "persist.h"

namespace ge {

namespace {

typedef __attribute__((address_space(3))) f16x8 lds_f16x8_t;

__device__ __forceinline__ float sigm(float x) { return 1.f / (1.f + expf(-x)); }

// 16-byte chunk c of LDS row r sits at chunk c ^ (r & 15): the 16 lanes of a
// fragment read (16 rows, one chunk) hit 16 distinct bank groups
__device__ __forceinline__ int swz(int r, int c) { return c ^ (r & 15); }

}  // namespace

// barrier words: a counter per row group, 256 bytes apart, then the error word
constexpr int kSyncStride = 64;  // unsigned words
constexpr int kSyncWords = 5 * kSyncStride;

template <int KB>
__global__ __launch_bounds__(256, 1) void gru_rec_fwd_kernel(const float *__restrict__ GI, const half_t *__restrict__ Wh,
                                                             const float *__restrict__ bh, int B, int T,
                                                             float *__restrict__ GH, float *__restrict__ R,
                                                             float *__restrict__ Z, float *__restrict__ Nn,
                                                             float *__restrict__ HS, half_t *__restrict__ H16,
                                                             unsigned *__restrict__ sync) {
  constexpr int H = 256 * KB, H3 = 3 * H;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  half_t *w = (half_t *)smem;  // [48][H]: row c = gate c / 16, unit c % 16; k contiguous, chunks swizzled
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int u0 = blockIdx.x * 16;
  unsigned *count = sync, *err = sync + 4 * kSyncStride;
  // a barrier that gives up (it also sets the error word) turns every later
  // hidden state this block writes into NaN, so the step's loss shows it;
  // later barriers see the error word and return at once
  bool dead = false;
  // W_h columns of this block, transposed into LDS: thread takes (k, gate),
  // reads the 16 units of row k of that gate block and writes them to 16 rows
  for (int p = tid; p < H * 3; p += 256) {
    const int k = p / 3, g = p % 3;
    const f16x8 a = *(const f16x8 *)(Wh + (int64_t)k * H3 + g * H + u0);
    const f16x8 b = *(const f16x8 *)(Wh + (int64_t)k * H3 + g * H + u0 + 8);
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int row = g * 16 + u;
      w[row * H + swz(row, k >> 3) * 8 + (k & 7)] = u < 8 ? a[u] : b[u - 8];
    }
  }
  const int m = wave * 16 + (lane & 15);  // batch row of this lane
  const int j0 = 4 * (lane >> 4);         // its four units within the block
  const bool live = wave * 16 < B;
  f32x4 bias[3], gi[3];
  f32x4 hp = {0.f, 0.f, 0.f, 0.f};  // h_{t-1} of the lane's (row, units)
#pragma unroll
  for (int g = 0; g < 3; ++g) bias[g] = *(const f32x4 *)(bh + g * H + u0 + j0);
  if (live) {
#pragma unroll
    for (int g = 0; g < 3; ++g) gi[g] = *(const f32x4 *)(GI + (int64_t)m * H3 + g * H + u0 + j0);
  }
  __syncthreads();
  for (int t = 0; t < T; ++t) {
    if (live) {
      f32x4 acc[3] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
      if (t > 0) {
        // h16_{t-1} row m: the lane's 8 k values of each 32-wide chunk
        const half_t *hrow = H16 + ((int64_t)t * B + m) * H + 8 * (lane >> 4);
        f16x8 hv[8 * KB];
#pragma unroll
        for (int s = 0; s < 8 * KB; ++s) hv[s] = *(const f16x8 *)(hrow + 32 * s);
#pragma unroll
        for (int s = 0; s < 8 * KB; ++s) {
          const int c = 4 * s + (lane >> 4);
#pragma unroll
          for (int g = 0; g < 3; ++g) {
            const int row = g * 16 + (lane & 15);
            const f16x8 wv = *(const lds_f16x8_t *)(w + row * H + swz(row, c) * 8);
            acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wv, hv[s], acc[g], 0, 0, 0);
          }
        }
      }
      // lane holds GH[m][g H + u0 + j0 .. +3] (before the bias)
      const int64_t row = (int64_t)t * B + m;
      f32x4 gh[3], r, z, nn, hv;
#pragma unroll
      for (int g = 0; g < 3; ++g) gh[g] = acc[g] + bias[g];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        r[q] = sigm(gi[0][q] + gh[0][q]);
        z[q] = sigm(gi[1][q] + gh[1][q]);
        nn[q] = tanhf(gi[2][q] + r[q] * gh[2][q]);
        hv[q] = dead ? NAN : (1.f - z[q]) * nn[q] + z[q] * hp[q];
      }
      const int64_t o = row * H + u0 + j0;
      *(f32x4 *)(R + o) = r;
      *(f32x4 *)(Z + o) = z;
      *(f32x4 *)(Nn + o) = nn;
      *(f32x4 *)(HS + o) = hv;
      *(f16x4 *)(H16 + (row + B) * H + u0 + j0) = f16x4{(half_t)hv[0], (half_t)hv[1], (half_t)hv[2], (half_t)hv[3]};
#pragma unroll
      for (int g = 0; g < 3; ++g) *(f32x4 *)(GH + row * H3 + g * H + u0 + j0) = gh[g];
      hp = hv;
      if (t + 1 < T) {
#pragma unroll
        for (int g = 0; g < 3; ++g) gi[g] = *(const f32x4 *)(GI + (row + B) * H3 + g * H + u0 + j0);
      }
    }
    if (t + 1 < T && !grid_barrier(count, (unsigned)((t + 1) * gridDim.x), err)) dead = true;
  }
}

template <int KB>
__global__ __launch_bounds__(256, 1) void gru_rec_bwd_kernel(const float *__restrict__ dh_out,
                                                             const half_t *__restrict__ Wh, const float *__restrict__ R,
                                                             const float *__restrict__ Z, const float *__restrict__ Nn,
                                                             const float *__restrict__ GH, const float *__restrict__ HS,
                                                             int B, int T, half_t *__restrict__ dGH,
                                                             half_t *__restrict__ dGI, unsigned *__restrict__ sync) {
  constexpr int H = 256 * KB, H3 = 3 * H, KC = H3 / 8;  // 16-byte chunks per W row
  constexpr int NS = KC / 16;                           // chunk groups (of 4) per wave
  extern __shared__ __attribute__((aligned(16))) char smem[];
  half_t *w = (half_t *)smem;                  // [16][3H]: rows u0 .. u0 + 15 of W_h, chunks swizzled
  f32x4 *red = (f32x4 *)(smem + 16 * H3 * 2);  // [3 waves][64] partial carries
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nug = H / 16;
  const int ug = blockIdx.x % nug, rg = blockIdx.x / nug;
  const int u0 = ug * 16;
  unsigned *count = sync + kSyncStride * rg, *err = sync + 4 * kSyncStride;
  for (int p = tid; p < 16 * KC; p += 256) {
    const int u = p / KC, c = p % KC;
    *(f16x8 *)(w + u * H3 + swz(u, c) * 8) = *(const f16x8 *)(Wh + (int64_t)(u0 + u) * H3 + 8 * c);
  }
  const int m = rg * 16 + (lane & 15);
  const int j0 = 4 * (lane >> 4);
  const bool gate = wave == 0;  // the wave that runs the gate backward and owns the carry
  bool dead = false;            // as in the forward: NaN gradients after a barrier that gave up
  f32x4 carry = {0.f, 0.f, 0.f, 0.f};
  f32x4 dho, r, z, nn, ghn, h0;
  auto fetch = [&](int t) {
    const int64_t row = (int64_t)t * B + m;
    const int64_t o = row * H + u0 + j0;
    dho = *(const f32x4 *)(dh_out + o);
    r = *(const f32x4 *)(R + o);
    z = *(const f32x4 *)(Z + o);
    nn = *(const f32x4 *)(Nn + o);
    ghn = *(const f32x4 *)(GH + row * H3 + 2 * H + u0 + j0);
    h0 = t > 0 ? *(const f32x4 *)(HS + o - (int64_t)B * H) : f32x4{0.f, 0.f, 0.f, 0.f};
  };
  if (gate) fetch(T - 1);
  __syncthreads();
  int nbar = 0;
  for (int t = T - 1; t >= 0; --t) {
    f32x4 dd = {0.f, 0.f, 0.f, 0.f};
    if (gate) {
      const int64_t row = (int64_t)t * B + m;
      f16x4 gr, gz, gn, gnh;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float dh = dead ? NAN : dho[q] + carry[q];
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
      if (t > 0) fetch(t - 1);
    }
    if (t == 0) break;
    ++nbar;
    if (!grid_barrier(count, (unsigned)(nbar * nug), err)) dead = true;
    // carry for step t-1: dh z + dGH_t[m, :] W_h[u0 + j, :]^T over the 3H
    // columns; wave `wave` takes chunks wave KC/4 .. (wave + 1) KC/4
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    {
      const half_t *grow = dGH + ((int64_t)t * B + m) * H3 + wave * (H3 / 4) + 8 * (lane >> 4);
      f16x8 gv[NS];
#pragma unroll
      for (int s = 0; s < NS; ++s) gv[s] = *(const f16x8 *)(grow + 32 * s);
      const int wr = lane & 15;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int c = wave * (KC / 4) + 4 * s + (lane >> 4);
        const f16x8 wv = *(const lds_f16x8_t *)(w + wr * H3 + swz(wr, c) * 8);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(wv, gv[s], acc, 0, 0, 0);
      }
      if (wave > 0) red[(wave - 1) * 64 + lane] = acc;
    }
    __syncthreads();
    if (gate) carry = ((acc + red[lane]) + red[64 + lane]) + red[128 + lane] + dd;
    // the next writes to red follow the next barrier's workgroup barrier
  }
}

// ---- launchers ------------------------------------------------------------------
namespace {

const void *fwd_kernel(int KB) {
  switch (KB) {
    case 1: return (const void *)gru_rec_fwd_kernel<1>;
    case 2: return (const void *)gru_rec_fwd_kernel<2>;
    case 3: return (const void *)gru_rec_fwd_kernel<3>;
    default: return (const void *)gru_rec_fwd_kernel<4>;
  }
}

const void *bwd_kernel(int KB) {
  switch (KB) {
    case 1: return (const void *)gru_rec_bwd_kernel<1>;
    case 2: return (const void *)gru_rec_bwd_kernel<2>;
    case 3: return (const void *)gru_rec_bwd_kernel<3>;
    default: return (const void *)gru_rec_bwd_kernel<4>;
  }
}

size_t fwd_lds(int H) { return (size_t)48 * H * 2; }
size_t bwd_lds(int H) { return (size_t)16 * 3 * H * 2 + (size_t)3 * 64 * 16; }

// the dynamic LDS above the default limit has to be granted per kernel
bool grant(const void *fn, int slot, size_t lds) {
  static size_t granted[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (lds <= granted[slot]) return true;
  if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  granted[slot] = lds;
  return true;
}

int coop_launch(const void *fn, int slot, int blocks, size_t lds, void **args, hipStream_t s, const char *what) {
  if (!grant(fn, slot, lds)) {
    set_error("%s: cannot grant %zu bytes of LDS", what, lds);
    return GE_E_LAUNCH;
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

int64_t gru_sync_bytes() { return (int64_t)kSyncWords * 4; }

bool gru_persist_supported(int64_t B, int64_t H) {
  if (B < 1 || B > 64 || B % 16 != 0 || H % 256 != 0 || H < 256 || H > 1024) return false;
  int dev = 0, coop = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  if (hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) != hipSuccess || !coop) return false;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return false;
  // every block of either kernel must be resident at once
  const int KB = (int)(H / 256);
  const void *fns[2] = {fwd_kernel(KB), bwd_kernel(KB)};
  const size_t lds[2] = {fwd_lds((int)H), bwd_lds((int)H)};
  const int64_t blocks[2] = {H / 16, H / 16 * (B / 16)};
  for (int i = 0; i < 2; ++i) {
    int per_cu = 0;
    if (!grant(fns[i], i * 4 + KB - 1, lds[i]) ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fns[i], 256, lds[i]) != hipSuccess) {
      (void)hipGetLastError();
      return false;
    }
    if ((int64_t)per_cu * cus < blocks[i]) return false;
  }
  return true;
}

int fill_zero_launch(void *p, int64_t bytes, hipStream_t s);

// sync: device unsigned [gru_sync_bytes() / 4] (a barrier counter per row
// group and the error word), cleared here first
int gru_rec_fwd_launch(const float *GI, const half_t *Wh, const float *bh, int B, int H, int T, float *GH, float *R,
                       float *Z, float *N, float *HS, half_t *H16, unsigned *sync, hipStream_t s) {
  int st = fill_zero_launch(sync, gru_sync_bytes(), s);
  if (st != GE_OK) return st;
  const int KB = H / 256;
  void *args[] = {&GI, &Wh, &bh, &B, &T, &GH, &R, &Z, &N, &HS, &H16, &sync};
  return coop_launch(fwd_kernel(KB), KB - 1, H / 16, fwd_lds(H), args, s, "gru recurrence (forward)");
}

int gru_rec_bwd_launch(const float *dh_out, const half_t *Wh, const float *R, const float *Z, const float *N,
                       const float *GH, const float *HS, int B, int H, int T, half_t *dGH, half_t *dGI, unsigned *sync,
                       hipStream_t s) {
  int st = fill_zero_launch(sync, gru_sync_bytes(), s);
  if (st != GE_OK) return st;
  const int KB = H / 256;
  void *args[] = {&dh_out, &Wh, &R, &Z, &N, &GH, &HS, &B, &T, &dGH, &dGI, &sync};
  return coop_launch(bwd_kernel(KB), 4 + KB - 1, H / 16 * (B / 16), bwd_lds(H), args, s,
                     "gru recurrence (backward)");
}

}  // namespace ge
