// The transformer MLP block's forward pass as ONE kernel: RMSNorm, up
// projection, LeakyReLU squared, down projection and residual, with the
// F-wide intermediate accumulated chunk by chunk on chip and never written to
// HBM ("Full-Depth MLP Megakernel + Fused Attention Preprocessing", "What
// Worked": one kernel whose hidden activations stay in registers and are
// accumulated in narrow chunks; "What Didn't Work" / "The Key Insight": that
// kernel lost 15-41 % to library GEMMs on its GPU, so here it is an A/B variant
// of the GEMM chain, measured, not the default).
//
// Same arithmetic and storage as the forward half of the chain (block.cpp):
//   r = 1 / sqrt(mean_j x^2 + eps);  n = convert(x r);
//   u = n W_up (FP32);  a = convert((u > 0 ? u : slope u)^2);
//   y = convert(x + a W_down).
//
// A block takes 64 rows; its four waves are (row half rh, column half eh).
// * RMSNorm: a lane holds row 32 rh + l % 32 of x in the B-fragment layout of
//   the 32x32x16 MFMA (8 consecutive d of each 16-wide k step, d = 16 s +
//   8 (l / 32)), so the row's sum of squares is the lane's own 256 squares plus
//   one exchange with lane l ^ 32, and n stays in registers for the whole
//   kernel (32 fragments).
// * For each chunk of 64 hidden units: the wave forms u^T for 32 of them
//   (eh picks which) against its 32 rows: 32 MFMAs with W_up^T rows from LDS,
//   alternating between two accumulators so two chains are in flight.
//   The accumulator of lane l holds u for row l % 32 and four runs of four
//   consecutive units, so a = LeakyReLU^2(u) goes to a small LDS tile [64 rows
//   x 64 units] as 8-byte stores.  After a workgroup barrier every wave adds
//   a W_down for its 32 rows and its 256 output columns: 8 output tiles x 4 k
//   steps, the a fragment read once per k step, W_down^T rows from LDS.
// * The weight slices stream from global memory straight into LDS (buffer
//   loads that write LDS, no register round trip): the next chunk's W_up^T
//   while this chunk's down-projection MFMAs run, the next W_down^T while the
//   next up-projection runs.  Each lane loads the 16 bytes that belong at its
//   LDS position, so the swizzle is folded into the global offset.  The kernel reads the weights as transposed copies that a
//   small kernel writes first (unit-major W_up^T, output-major W_down^T), so
//   every MFMA operand is a 16-byte LDS read of 8 consecutive k.  Per CU the
//   weights stream at 64 bytes of weights per 4 x 1,024 FLOP, which is what
//   bounds the kernel: each 64-row block reads all of both matrices.
// LDS: W_up^T slice 64 KB, W_down^T slice 64 KB, a tile 8 KB.
#include "common.h"

namespace ge {

namespace {

typedef uint32_t mk_u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) mk_u32x4 lds_mk_u32x4;
typedef uint32_t mk_u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) mk_u32x2 lds_mk_u32x2;

constexpr int MD = 512;       // model width the kernel is built for
constexpr int MC = 64;        // hidden units per chunk
constexpr int MBR = 64;       // rows per block
constexpr int MKS = MD / 16;  // 16-wide k steps over D
constexpr int WU_BYTES = MC * MD * 2;   // the W_up^T slice [MC][MD]
constexpr int WD_BYTES = MD * MC * 2;   // the W_down^T slice [MD][MC]
constexpr int AS_BYTES = MBR * MC * 2;  // the a tile [MBR][MC]

template <typename T> struct MkMfma;
template <> struct MkMfma<bf16_t> {
  typedef bf16x8 V;
  static __device__ __forceinline__ f32x16 mma(V a, V b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct MkMfma<half_t> {
  typedef f16x8 V;
  static __device__ __forceinline__ f32x16 mma(V a, V b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

// 16-byte chunk c of a 1 KB W_up^T row r sits at chunk c ^ (r & 15); of a
// 128-byte row (W_down^T, the a tile) at c ^ ((r / 2) & 7): the 16 lanes of one
// fragment read hit 16 distinct bank groups.  Both maps are their own inverse.
__device__ __forceinline__ int swz_wu(int r, int c) { return c ^ (r & 15); }
__device__ __forceinline__ int swz_128(int r, int c) { return c ^ ((r >> 1) & 7); }

template <typename T>
__device__ __forceinline__ T lrelu_sq(float u, float slope) {
  const float t = u > 0.f ? u : slope * u;
  return from_f32<T>(t * t);
}

}  // namespace

// W_up [D x F] -> W_up^T [F x D];  W_down [F x D] -> W_down^T [D x F]
template <typename T>
__global__ __launch_bounds__(256) void mk_transpose_kernel(const T *__restrict__ wu, const T *__restrict__ wd,
                                                           T *__restrict__ wut, T *__restrict__ wdt, int D, int F) {
  __shared__ T tile[32][33];
  const int tiles_u = (D / 32) * (F / 32);
  int t = blockIdx.x;
  const bool up = t < tiles_u;
  if (!up) t -= tiles_u;
  // source [R x Cc] row-major -> destination [Cc x R]
  const int R = up ? D : F, Cc = up ? F : D;
  const T *src = up ? wu : wd;
  T *dst = up ? wut : wdt;
  const int r0 = (t / (Cc / 32)) * 32, c0 = (t % (Cc / 32)) * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
#pragma unroll
  for (int i = 0; i < 4; ++i) tile[ty + 8 * i][tx] = src[(int64_t)(r0 + ty + 8 * i) * Cc + c0 + tx];
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) dst[(int64_t)(c0 + ty + 8 * i) * R + r0 + tx] = tile[tx][ty + 8 * i];
}

template <typename T>
__global__ __launch_bounds__(256, 1) void mlp_block_fused_kernel(const T *__restrict__ x, const T *__restrict__ wut,
                                                                 const T *__restrict__ wdt, int64_t rows, int F,
                                                                 float eps, float slope, T *__restrict__ y,
                                                                 float *__restrict__ r_out, T *__restrict__ n_out,
                                                                 T *__restrict__ u_out, T *__restrict__ a_out) {
  typedef typename MkMfma<T>::V V;
  __shared__ __attribute__((aligned(1024))) char smem[WU_BYTES + WD_BYTES + AS_BYTES];
  char *const Wu = smem, *const Wd = smem + WU_BYTES, *const As = smem + WU_BYTES + WD_BYTES;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rh = wave & 1, eh = wave >> 1;
  const int lr = lane & 31, lh = lane >> 5;
  const int64_t b0 = (int64_t)blockIdx.x * MBR;
  const int64_t row = b0 + 32 * rh + lr;  // the row this lane holds
  const bool rok = row < rows;
  const int nch = F / MC;

  // ---- weight slices: buffer loads that write LDS ---------------------------
  // a wave's load instruction fills 1 KB of LDS, lane i the 16 bytes at i * 16;
  // a slice is 64 such instructions, 16 per wave
  const u32x4 rwu = raw_buffer_rsrc(wut), rwd = raw_buffer_rsrc(wdt);
  auto issue_wu = [&](int c) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int ins = wave * 16 + j, p = ins * 64 + lane;  // LDS chunk position this lane fills
      const int rr = p >> 6, cc = swz_wu(rr, p & 63);
      const uint32_t vo = (uint32_t)(((int64_t)(c * MC + rr) * MD + cc * 8) * (int64_t)sizeof(T));
      lds_dma16(rwu, vo, 0, Wu + ins * 1024);
    }
  };
  auto issue_wd = [&](int c) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int ins = wave * 16 + j, p = ins * 64 + lane;
      const int e = p >> 3, cc = swz_128(e, p & 7);
      const uint32_t vo = (uint32_t)(((int64_t)e * F + c * MC + cc * 8) * (int64_t)sizeof(T));
      lds_dma16(rwd, vo, 0, Wd + ins * 1024);
    }
  };
  issue_wu(0);
  issue_wd(0);

  // ---- RMSNorm in the fragment layout --------------------------------------
  V nf[MKS];
  {
    // rows past the end read the last row and are never stored
    const T *xr = x + (rok ? row : rows - 1) * MD + 8 * lh;
    float ss = 0.f;
#pragma unroll
    for (int s = 0; s < MKS; ++s) {
      nf[s] = *(const V *)(xr + 16 * s);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = to_f32(nf[s][e]);
        ss += v * v;
      }
    }
    ss += __shfl_xor(ss, 32, 64);
    const float rs = 1.0f / sqrtf(ss / (float)MD + eps);
#pragma unroll
    for (int s = 0; s < MKS; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) nf[s][e] = from_f32<T>(to_f32(nf[s][e]) * rs);
    if (rok && eh == 0) {
      if (r_out && lh == 0) r_out[row] = rs;
      if (n_out) {
#pragma unroll
        for (int s = 0; s < MKS; ++s) *(V *)(n_out + row * MD + 16 * s + 8 * lh) = nf[s];
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0070);  // this wave's slices are in LDS
  __syncthreads();

  f32x16 yacc[8];
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) yacc[t][e] = 0.f;

  const int ar = 32 * rh + lr;  // this lane's row of the a tile
  for (int c = 0; c < nch; ++c) {
    const bool more = c + 1 < nch;
    // u^T for units 32 eh .. +31 of the chunk against this wave's 32 rows, the
    // k steps alternating between two accumulators (two independent chains)
    f32x16 ua, ub;
#pragma unroll
    for (int e = 0; e < 16; ++e) ua[e] = ub[e] = 0.f;
    {
      const int ur = 32 * eh + lr;
      const char *wrow = Wu + ur * 1024;
#pragma unroll
      for (int s = 0; s < MKS; s += 2) {
        const V p0 = __builtin_bit_cast(V, *(const lds_mk_u32x4 *)(wrow + swz_wu(ur, 2 * s + lh) * 16));
        const V p1 = __builtin_bit_cast(V, *(const lds_mk_u32x4 *)(wrow + swz_wu(ur, 2 * s + 2 + lh) * 16));
        ua = MkMfma<T>::mma(p0, nf[s], ua);
        ub = MkMfma<T>::mma(p1, nf[s + 1], ub);
      }
    }
    // lane: row ar, units 32 eh + 8 g + 4 lh + (0..3), g = 0..3
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      T av[4], uv[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float u = ua[4 * g + q] + ub[4 * g + q];
        av[q] = lrelu_sq<T>(u, slope);
        uv[q] = from_f32<T>(u);
      }
      const int unit = 32 * eh + 8 * g + 4 * lh;
      *(lds_mk_u32x2 *)(As + ar * 128 + swz_128(ar, unit >> 3) * 16 + 8 * lh) = __builtin_bit_cast(mk_u32x2, av);
      if (u_out && rok) *(mk_u32x2 *)(u_out + row * F + c * MC + unit) = __builtin_bit_cast(mk_u32x2, uv);
      if (a_out && rok) *(mk_u32x2 *)(a_out + row * F + c * MC + unit) = __builtin_bit_cast(mk_u32x2, av);
    }
    // the a tile is complete, W_up^T is read, W_down^T of this chunk has landed
    __builtin_amdgcn_s_waitcnt(0x0070);
    __syncthreads();
    if (more) issue_wu(c + 1);
    // y^T += W_down^T a^T for output columns 256 eh .. +255 and this wave's rows
#pragma unroll
    for (int ks = 0; ks < MC / 16; ++ks) {
      const V q = __builtin_bit_cast(V, *(const lds_mk_u32x4 *)(As + ar * 128 + swz_128(ar, 2 * ks + lh) * 16));
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int er = 256 * eh + 32 * t + lr;
        const V p = __builtin_bit_cast(V, *(const lds_mk_u32x4 *)(Wd + er * 128 + swz_128(er, 2 * ks + lh) * 16));
        yacc[t] = MkMfma<T>::mma(p, q, yacc[t]);
      }
    }
    // W_down^T and the a tile are read, W_up^T of the next chunk has landed
    __builtin_amdgcn_s_waitcnt(0x0070);
    __syncthreads();
    if (more) issue_wd(c + 1);
  }

  // ---- residual and store: lane holds y[row][256 eh + 32 t + 8 g + 4 lh + q] ----
  if (!rok) return;
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int64_t o = row * MD + 256 * eh + 32 * t + 8 * g + 4 * lh;
      const mk_u32x2 xr = *(const mk_u32x2 *)(x + o);
      const T *xv = (const T *)&xr;
      T yv[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) yv[q] = from_f32<T>(yacc[t][4 * g + q] + to_f32(xv[q]));
      *(mk_u32x2 *)(y + o) = __builtin_bit_cast(mk_u32x2, yv);
    }
}

int64_t block_fused_ws_bytes(int64_t D, int64_t F) { return 2 * D * F * 2; }

template <typename T>
int block_fused_t(const ge_block_fused_args &a, hipStream_t s) {
  T *wut = (T *)a.workspace;
  T *wdt = wut + a.D * a.F;
  const int tiles = 2 * (int)((a.D / 32) * (a.F / 32));
  hipLaunchKernelGGL(mk_transpose_kernel<T>, dim3(tiles), dim3(256), 0, s, (const T *)a.w_up, (const T *)a.w_down,
                     wut, wdt, (int)a.D, (int)a.F);
  int st = launch_status("mlp_block_fwd_fused (weight transpose)");
  if (st != GE_OK || a.rows == 0) return st;
  const unsigned blocks = (unsigned)((a.rows + MBR - 1) / MBR);
  hipLaunchKernelGGL(mlp_block_fused_kernel<T>, dim3(blocks), dim3(256), 0, s, (const T *)a.x, (const T *)wut,
                     (const T *)wdt, a.rows, (int)a.F, a.eps, a.slope, (T *)a.y, a.r, (T *)a.n, (T *)a.u,
                     (T *)a.a);
  return launch_status("mlp_block_fwd_fused");
}

int block_fused_launch(const ge_block_fused_args &a, hipStream_t s) {
  if (a.D != MD) {
    set_error("mlp_block_fwd_fused: D must be %d (got %lld)", MD, (long long)a.D);
    return GE_E_UNSUPPORTED;
  }
  if (a.F < 64 || a.F % 64 != 0 || a.F > (1 << 20)) {
    set_error("mlp_block_fwd_fused: F must be a positive multiple of 64");
    return GE_E_UNSUPPORTED;
  }
  if (a.rows / MBR >= 0x7fffffff) {
    set_error("mlp_block_fwd_fused: too many rows");
    return GE_E_INVALID;
  }
  return a.type == GE_BF16 ? block_fused_t<bf16_t>(a, s) : block_fused_t<half_t>(a, s);
}

}  // namespace ge
