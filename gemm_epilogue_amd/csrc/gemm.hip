// MFMA GEMM with a fused FP32 epilogue, for gfx950 (CDNA4, wave64).
//
// C = act(alpha * op(A) op(B) + bias) [+ residual], layouts NN / NT / TN.
// Bias and activation are applied to the FP32 accumulator and the value is
// converted once at the final store ("The Work Moved Down a Layer", section
// "The Debugging Lesson Was Numerical"; "Capstone 5: train a network with your
// CUDA kernels", section "Read the worked reference").  The backward GEMMs of
// "Capstone 5", section "Work through the backward pass" (dW = X^T dH,
// dX = dH W^T, dH masked by H > 0) are the TN / NT layouts and the *_BWD
// epilogues.
//
// Design (ours, not the pages'): a block of 4 wavefronts computes a BM x BN
// tile; A and B tiles of BK along k are staged through LDS, double-buffered,
// always stored k-contiguous ([row][k], rows padded by 16 bytes) so each MFMA
// fragment is one 16-byte LDS read per lane.  Operands that are contiguous
// along m/n in memory (B of NN, both of TN) are transposed in registers on
// their way into LDS.  MFMA 16x16 tiles are issued with the B tile in the
// instruction's first operand slot, so each lane ends up owning four
// consecutive columns of one output row (16-byte FP32 / 8-byte 16-bit stores).
// FP16/BF16 use v_mfma_f32_16x16x32_{f16,bf16}; FP32 uses v_mfma_f32_16x16x4_f32.
// Split-K writes FP32 partials to a workspace and a finishing kernel sums
// them in split order, then applies the same epilogue.
#include <algorithm>

#include "common.h"

namespace ge {

struct EpiParams {
  float alpha;
  const float *bias;
  int act;
  float slope;
  const void *aux;
  int64_t ld_aux;
  int aux_type;
  const void *res;
  int64_t ld_res;
  int res_type;
  void *C;
  int64_t ldc;
  int c_type;
  void *pre;
  int64_t ld_pre;
  int pre_type;
  int M, N;
  int aux_vec, res_vec, c_vec, pre_vec, bias_vec;
};

struct GemmParams {
  const void *A;
  const void *B;
  int64_t lda, ldb;
  int M, N, K;
  int a_vec, b_vec;
  int tiles_m, tiles_n;
  int ktiles_per_split;
  int splits;
  float *partial;  // [splits][M][N] when splits > 1
  EpiParams ep;
};

// Epilogue for four consecutive columns n..n+3 of row m (FP32 values v).
__device__ __forceinline__ void epilogue4(const EpiParams &e, int m, int n, float v[4]) {
  if (m >= e.M || n >= e.N) return;
  const bool full = (n + 3) < e.N;
  float b[4] = {0.f, 0.f, 0.f, 0.f};
  if (e.bias) {
    if (full && e.bias_vec) {
      f32x4 x = *(const f32x4 *)(e.bias + n);
      b[0] = x[0]; b[1] = x[1]; b[2] = x[2]; b[3] = x[3];
    } else {
      for (int j = 0; j < 4; ++j) b[j] = (n + j < e.N) ? e.bias[n + j] : 0.f;
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) v[j] = e.alpha * v[j] + b[j];
  if (e.pre) {
    if (full) store4_any(e.pre, (int64_t)m * e.ld_pre + n, e.pre_type, e.pre_vec, v);
    else
      for (int j = 0; j < 4; ++j)
        if (n + j < e.N) store_any(e.pre, (int64_t)m * e.ld_pre + n + j, e.pre_type, v[j]);
  }
  if (e.act == GE_ACT_RELU) {
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = fmaxf(v[j], 0.f);
  } else if (e.act == GE_ACT_LRELU_SQ) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float t = v[j] > 0.f ? v[j] : e.slope * v[j];
      v[j] = t * t;
    }
  } else if (e.act == GE_ACT_RELU_MASK_BWD || e.act == GE_ACT_LRELU_SQ_BWD) {
    float a[4];
    if (full) load4_any(e.aux, (int64_t)m * e.ld_aux + n, e.aux_type, e.aux_vec, a);
    else
      for (int j = 0; j < 4; ++j)
        a[j] = (n + j < e.N) ? load_any(e.aux, (int64_t)m * e.ld_aux + n + j, e.aux_type) : 0.f;
    if (e.act == GE_ACT_RELU_MASK_BWD) {
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = a[j] > 0.f ? v[j] : 0.f;
    } else {
      const float s2 = 2.f * e.slope * e.slope;
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] *= (a[j] > 0.f ? 2.f * a[j] : s2 * a[j]);
    }
  }
  if (e.res) {
    float r[4];
    if (full) load4_any(e.res, (int64_t)m * e.ld_res + n, e.res_type, e.res_vec, r);
    else
      for (int j = 0; j < 4; ++j)
        r[j] = (n + j < e.N) ? load_any(e.res, (int64_t)m * e.ld_res + n + j, e.res_type) : 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] += r[j];
  }
  if (full) store4_any(e.C, (int64_t)m * e.ldc + n, e.c_type, e.c_vec, v);
  else
    for (int j = 0; j < 4; ++j)
      if (n + j < e.N) store_any(e.C, (int64_t)m * e.ldc + n + j, e.c_type, v[j]);
}

// ---- MFMA wrappers: acc += hwA * hwB over one 16-byte-per-lane k chunk -----
template <typename T> struct Frag;
template <> struct Frag<half_t> {
  typedef f16x8 V;
  static __device__ __forceinline__ f32x4 mma(V a, V b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};
template <> struct Frag<bf16_t> {
  typedef bf16x8 V;
  static __device__ __forceinline__ f32x4 mma(V a, V b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct Frag<float> {
  typedef f32x4 V;
  // four k-steps of 16x16x4: step e pairs element e of both operands, so both
  // operands see the same k assignment and the sum over the chunk is complete.
  static __device__ __forceinline__ f32x4 mma(V a, V b, f32x4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], c, 0, 0, 0);
    return c;
  }
};

// raw 16-byte vector of T elements
struct alignas(16) Raw16 {
  uint32_t w[4];
};

template <typename T> __device__ __forceinline__ T zero_of() { return (T)0.f; }

// ---- tile loaders ------------------------------------------------------------
// k-contiguous source: R rows (m or n) x BK, each row contiguous along k.
template <typename T, int R, int BK, int NT> struct LoaderKC {
  static constexpr int VEC = 16 / sizeof(T);
  static constexpr int VPR = BK / VEC;  // vectors per row
  static constexpr int NV = R * VPR / NT;
  static_assert(NV >= 1 && (R * VPR) % NT == 0, "tile / thread mismatch");
  Raw16 r[NV];

  __device__ __forceinline__ void load(const T *__restrict__ p, int64_t ld, int r0, int rmax, int k0,
                                       int kmax, bool vec, int tid) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int v = tid + i * NT;
      const int row = v / VPR, kv = v % VPR;
      const int gr = r0 + row, gk = k0 + kv * VEC;
      if (vec && gr < rmax && gk + VEC <= kmax) {
        r[i] = *(const Raw16 *)(p + (int64_t)gr * ld + gk);
      } else {
        T tmp[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e)
          tmp[e] = (gr < rmax && gk + e < kmax) ? p[(int64_t)gr * ld + gk + e] : zero_of<T>();
        r[i] = *(Raw16 *)tmp;
      }
    }
  }
  __device__ __forceinline__ void store(T *s, int stride, int tid) const {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int v = tid + i * NT;
      const int row = v / VPR, kv = v % VPR;
      *(Raw16 *)(s + row * stride + kv * VEC) = r[i];
    }
  }
};

// m/n-contiguous source: BK k-rows, each contiguous along the R dimension.
// Each thread reads KB consecutive k-rows of one 16-byte vector and writes
// them transposed: VEC LDS rows of KB k-values.
template <typename T, int R, int BK, int NT> struct LoaderMC {
  static constexpr int VEC = 16 / sizeof(T);
  static constexpr int RV = R / VEC;  // vectors per k-row
  static constexpr int KB = BK * RV / NT;
  static_assert(KB >= 1 && (BK * RV) % NT == 0 && BK % KB == 0, "tile / thread mismatch");
  T x[KB][VEC];

  __device__ __forceinline__ void load(const T *__restrict__ p, int64_t ld, int r0, int rmax, int k0,
                                       int kmax, bool vec, int tid) {
    const int rv = tid % RV, kg = tid / RV;
    const int gr = r0 + rv * VEC;
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      const int gk = k0 + kg * KB + j;
      if (vec && gk < kmax && gr + VEC <= rmax) {
        Raw16 t = *(const Raw16 *)(p + (int64_t)gk * ld + gr);
        const T *tt = (const T *)&t;
#pragma unroll
        for (int e = 0; e < VEC; ++e) x[j][e] = tt[e];
      } else {
#pragma unroll
        for (int e = 0; e < VEC; ++e)
          x[j][e] = (gk < kmax && gr + e < rmax) ? p[(int64_t)gk * ld + gr + e] : zero_of<T>();
      }
    }
  }
  __device__ __forceinline__ void store(T *s, int stride, int tid) const {
    const int rv = tid % RV, kg = tid / RV;
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      T col[KB];
#pragma unroll
      for (int j = 0; j < KB; ++j) col[j] = x[j][e];
      T *dst = s + (rv * VEC + e) * stride + kg * KB;
      if constexpr (KB * sizeof(T) == 16) {
        *(Raw16 *)dst = *(Raw16 *)col;
      } else if constexpr (KB * sizeof(T) == 8) {
        *(uint2 *)dst = *(uint2 *)col;
      } else {
#pragma unroll
        for (int j = 0; j < KB; ++j) dst[j] = col[j];
      }
    }
  }
};

template <typename T, bool KC, int R, int BK, int NT> struct Loader;
template <typename T, int R, int BK, int NT> struct Loader<T, true, R, BK, NT> : LoaderKC<T, R, BK, NT> {};
template <typename T, int R, int BK, int NT> struct Loader<T, false, R, BK, NT> : LoaderMC<T, R, BK, NT> {};

// ---- the kernel ---------------------------------------------------------------
template <typename T, int LAYOUT, int BM, int BN, int BK>
__global__ __launch_bounds__(256) void gemm_kernel(GemmParams p) {
  constexpr int NT = 256;
  constexpr int VEC = 16 / sizeof(T);
  constexpr int KCH = 4 * VEC;  // k covered by one 16-byte-per-lane fragment
  constexpr int STRIDE = BK + VEC;
  constexpr int WTM = BM / 2, WTN = BN / 2;
  constexpr int FM = WTM / 16, FN = WTN / 16;
  constexpr bool A_KC = (LAYOUT != GE_TN);
  constexpr bool B_KC = (LAYOUT == GE_NT);
  static_assert(BK % KCH == 0, "BK must hold whole fragments");
  typedef typename Frag<T>::V V;

  __shared__ __attribute__((aligned(16))) T sA[2][BM * STRIDE];
  __shared__ __attribute__((aligned(16))) T sB[2][BN * STRIDE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm0 = (wave >> 1) * WTM, wn0 = (wave & 1) * WTN;

  // block -> tile: spread consecutive tiles over one XCD, then group along M
  int bid = blockIdx.x;
  const int total = p.tiles_m * p.tiles_n;
  if ((total & 7) == 0) bid = (bid & 7) * (total >> 3) + (bid >> 3);
  constexpr int GROUP = 8;
  const int per_group = GROUP * p.tiles_n;
  const int first_m = (bid / per_group) * GROUP;
  const int gsize = min(p.tiles_m - first_m, GROUP);
  const int tm = first_m + (bid % per_group) % gsize;
  const int tn = (bid % per_group) / gsize;
  const int bm0 = tm * BM, bn0 = tn * BN;

  const int nk_total = (p.K + BK - 1) / BK;
  const int kt0 = blockIdx.z * p.ktiles_per_split;
  const int kt1 = min(nk_total, kt0 + p.ktiles_per_split);

  const T *__restrict__ Ap = (const T *)p.A;
  const T *__restrict__ Bp = (const T *)p.B;

  Loader<T, A_KC, BM, BK, NT> la;
  Loader<T, B_KC, BN, BK, NT> lb;

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (kt0 < kt1) {
    la.load(Ap, p.lda, bm0, p.M, kt0 * BK, p.K, p.a_vec, tid);
    lb.load(Bp, p.ldb, bn0, p.N, kt0 * BK, p.K, p.b_vec, tid);
    la.store(sA[0], STRIDE, tid);
    lb.store(sB[0], STRIDE, tid);
    __syncthreads();
  }
  for (int kt = kt0; kt < kt1; ++kt) {
    const int cur = (kt - kt0) & 1;
    const bool more = kt + 1 < kt1;
    if (more) {
      la.load(Ap, p.lda, bm0, p.M, (kt + 1) * BK, p.K, p.a_vec, tid);
      lb.load(Bp, p.ldb, bn0, p.N, (kt + 1) * BK, p.K, p.b_vec, tid);
    }
    const T *a_s = sA[cur];
    const T *b_s = sB[cur];
#pragma unroll
    for (int c = 0; c < BK / KCH; ++c) {
      const int koff = c * KCH + (lane >> 4) * VEC;
      V af[FM], bf[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) af[i] = *(const V *)(a_s + (wm0 + i * 16 + (lane & 15)) * STRIDE + koff);
#pragma unroll
      for (int j = 0; j < FN; ++j) bf[j] = *(const V *)(b_s + (wn0 + j * 16 + (lane & 15)) * STRIDE + koff);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = Frag<T>::mma(bf[j], af[i], acc[i][j]);
    }
    if (more) {
      la.store(sA[cur ^ 1], STRIDE, tid);
      lb.store(sB[cur ^ 1], STRIDE, tid);
    }
    __syncthreads();
  }

  // lane owns C[m][n..n+3] of each 16x16 fragment
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int m = bm0 + wm0 + i * 16 + (lane & 15);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int n = bn0 + wn0 + j * 16 + (lane >> 4) * 4;
      float v[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
      if (p.splits == 1) {
        epilogue4(p.ep, m, n, v);
      } else if (m < p.M && n < p.N) {
        float *dst = p.partial + ((int64_t)blockIdx.z * p.M + m) * p.N + n;
        if (n + 3 < p.N && (p.N & 3) == 0) {
          *(f32x4 *)dst = acc[i][j];
        } else {
          for (int e = 0; e < 4; ++e)
            if (n + e < p.N) dst[e] = v[e];
        }
      }
    }
  }
}

// Sums split-K partials in split order and applies the epilogue.
__global__ __launch_bounds__(256) void splitk_finish_kernel(GemmParams p) {
  const int groups = (p.N + 3) >> 2;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)p.M * groups) return;
  const int m = (int)(idx / groups);
  const int n = (int)(idx % groups) * 4;
  const int64_t mn = (int64_t)p.M * p.N;
  const float *src = p.partial + (int64_t)m * p.N + n;
  float v[4] = {0.f, 0.f, 0.f, 0.f};
  const bool vec = (n + 3 < p.N) && (p.N & 3) == 0;
  for (int s = 0; s < p.splits; ++s) {
    if (vec) {
      f32x4 x = *(const f32x4 *)(src + s * mn);
      v[0] += x[0]; v[1] += x[1]; v[2] += x[2]; v[3] += x[3];
    } else {
      for (int e = 0; e < 4; ++e)
        if (n + e < p.N) v[e] += src[s * mn + e];
    }
  }
  epilogue4(p.ep, m, n, v);
}

// ---- host launcher --------------------------------------------------------------
namespace {

struct Plan {
  int big;  // 1: 128x128 tiles, 0: 64x64 tiles
  int BM, BN, BK;
  int tiles_m, tiles_n, nk, splits, kps;
};

Plan make_plan(int ab_type, int64_t M, int64_t N, int64_t K, int split_k) {
  Plan pl;
  const int bk = ab_type == GE_F32 ? 32 : 64;
  const int64_t t128 = ((M + 127) / 128) * ((N + 127) / 128);
  pl.big = (t128 >= 192) ? 1 : 0;
  pl.BM = pl.BN = pl.big ? 128 : 64;
  pl.BK = bk;
  pl.tiles_m = (int)((M + pl.BM - 1) / pl.BM);
  pl.tiles_n = (int)((N + pl.BN - 1) / pl.BN);
  pl.nk = (int)((K + bk - 1) / bk);
  int s = 1;
  if (split_k >= 1) {
    s = split_k;
  } else {
    const int64_t tiles = (int64_t)pl.tiles_m * pl.tiles_n;
    // split long K loops when the output alone cannot fill the 256 CUs
    if (tiles < 256 && pl.nk >= 16) {
      int64_t want = (512 + tiles - 1) / tiles;
      s = (int)std::min<int64_t>(want, pl.nk / 8);
      s = std::max(1, std::min(s, 64));
    }
  }
  s = std::max(1, std::min(s, std::max(1, pl.nk)));
  pl.kps = (pl.nk + s - 1) / std::max(1, s);
  pl.splits = pl.kps > 0 ? (pl.nk + pl.kps - 1) / pl.kps : 1;
  if (pl.splits < 1) pl.splits = 1;
  return pl;
}

template <typename T, int LAYOUT>
void launch_t(const Plan &pl, const GemmParams &gp, hipStream_t s) {
  dim3 grid(pl.tiles_m * pl.tiles_n, 1, pl.splits);
  constexpr int BK = sizeof(T) == 4 ? 32 : 64;
  if (pl.big)
    hipLaunchKernelGGL((gemm_kernel<T, LAYOUT, 128, 128, BK>), grid, dim3(256), 0, s, gp);
  else
    hipLaunchKernelGGL((gemm_kernel<T, LAYOUT, 64, 64, BK>), grid, dim3(256), 0, s, gp);
}

template <typename T>
void launch_layout(int layout, const Plan &pl, const GemmParams &gp, hipStream_t s) {
  if (layout == GE_NN) launch_t<T, GE_NN>(pl, gp, s);
  else if (layout == GE_NT) launch_t<T, GE_NT>(pl, gp, s);
  else launch_t<T, GE_TN>(pl, gp, s);
}

}  // namespace

int64_t gemm_ws_bytes(int layout, int ab_type, int64_t M, int64_t N, int64_t K, int split_k) {
  (void)layout;
  if (M <= 0 || N <= 0) return 0;
  Plan pl = make_plan(ab_type, M, N, K, split_k);
  if (pl.splits <= 1) return 0;
  return (int64_t)pl.splits * M * N * 4;
}

int gemm_launch(const ge_gemm_args &a, hipStream_t s) {
  if (a.M == 0 || a.N == 0) return GE_OK;
  Plan pl = make_plan(a.ab_type, a.M, a.N, a.K, a.split_k);
  GemmParams gp;
  const int es = dtype_size(a.ab_type);
  gp.A = a.A;
  gp.B = a.B;
  gp.lda = a.lda;
  gp.ldb = a.ldb;
  gp.M = (int)a.M;
  gp.N = (int)a.N;
  gp.K = (int)a.K;
  gp.a_vec = vec_aligned(a.A, a.lda, es, 16);
  gp.b_vec = vec_aligned(a.B, a.ldb, es, 16);
  gp.tiles_m = pl.tiles_m;
  gp.tiles_n = pl.tiles_n;
  gp.ktiles_per_split = pl.kps;
  gp.splits = pl.splits;
  gp.partial = nullptr;
  if (pl.splits > 1) {
    const int64_t need = (int64_t)pl.splits * a.M * a.N * 4;
    if (a.workspace == nullptr || a.workspace_bytes < need || ((uintptr_t)a.workspace % 16) != 0) {
      set_error("gemm_bias_act: split-K over %d splits needs %lld workspace bytes (16-byte aligned)", pl.splits,
                (long long)need);
      return GE_E_WORKSPACE;
    }
    gp.partial = (float *)a.workspace;
  }
  EpiParams &e = gp.ep;
  e.alpha = a.alpha;
  e.bias = a.bias;
  e.act = a.act;
  e.slope = a.act_slope;
  e.aux = a.aux;
  e.ld_aux = a.ld_aux;
  e.aux_type = a.aux_type;
  e.res = a.residual;
  e.ld_res = a.ld_res;
  e.res_type = a.res_type;
  e.C = a.C;
  e.ldc = a.ldc;
  e.c_type = a.c_type;
  e.pre = a.pre;
  e.ld_pre = a.ld_pre;
  e.pre_type = a.pre_type;
  e.M = (int)a.M;
  e.N = (int)a.N;
  e.aux_vec = a.aux ? vec_aligned(a.aux, a.ld_aux, dtype_size(a.aux_type), 4 * dtype_size(a.aux_type)) : 0;
  e.res_vec = a.residual ? vec_aligned(a.residual, a.ld_res, dtype_size(a.res_type), 4 * dtype_size(a.res_type)) : 0;
  e.c_vec = vec_aligned(a.C, a.ldc, dtype_size(a.c_type), 4 * dtype_size(a.c_type));
  e.pre_vec = a.pre ? vec_aligned(a.pre, a.ld_pre, dtype_size(a.pre_type), 4 * dtype_size(a.pre_type)) : 0;
  e.bias_vec = a.bias ? (((uintptr_t)a.bias % 16) == 0) : 0;

  if (a.ab_type == GE_F16) launch_layout<half_t>(a.layout, pl, gp, s);
  else if (a.ab_type == GE_BF16) launch_layout<bf16_t>(a.layout, pl, gp, s);
  else launch_layout<float>(a.layout, pl, gp, s);
  int st = launch_status("gemm_bias_act");
  if (st != GE_OK || pl.splits <= 1) return st;
  const int64_t items = a.M * ((a.N + 3) / 4);
  hipLaunchKernelGGL(splitk_finish_kernel, dim3((unsigned)((items + 255) / 256)), dim3(256), 0, s, gp);
  return launch_status("gemm_bias_act (split-K finish)");
}

}  // namespace ge
