// Host side of gemm_bias_act: launch plan (tile size, split-K), argument
// marshalling into the kernel parameters, and the split-K finishing kernel.
// The MFMA kernel itself is in gemm_kernel.h, instantiated per operand type
// in gemm_f16.hip, gemm_bf16.hip and gemm_f32.hip.
#include <mutex>

#include "gemm_kernel.h"

namespace ge {

// ---- fixed scratch for callers that cannot allocate ------------------------------
// Split-K partials of gemm_bias_act_noalloc live here instead of in a caller
// workspace.  Every GPU the library runs on holds its own copy until the
// process ends; host code must use the per-device address from
// hipGetSymbolAddress, never the array's name.
constexpr int64_t kScratchBytes = (int64_t)64 << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

// Sums split-K partials in split order and applies the epilogue.  The loads
// of eight splits are issued together (the sum is still taken in split
// order), so the pass is bound by bandwidth rather than by one memory round
// trip per split.
__global__ __launch_bounds__(256) void splitk_finish_kernel(GemmParams p) {
  const int groups = (p.N + 3) >> 2;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)p.M * groups) return;
  const int m = (int)(idx / groups);
  const int n = (int)(idx % groups) * 4;
  const int64_t mn = (int64_t)p.M * p.N;
  const float *src = p.partial + (int64_t)m * p.N + n;
  f32x4 v = {0.f, 0.f, 0.f, 0.f};
  constexpr int U = 8;
  if ((n + 3 < p.N) && (p.N & 3) == 0) {
    int s = 0;
    for (; s + U <= p.splits; s += U) {
      f32x4 t[U];
#pragma unroll
      for (int u = 0; u < U; ++u) t[u] = *(const f32x4 *)(src + (int64_t)(s + u) * mn);
#pragma unroll
      for (int u = 0; u < U; ++u) v += t[u];
    }
    for (; s < p.splits; ++s) v += *(const f32x4 *)(src + (int64_t)s * mn);
  } else {
    int s = 0;
    for (; s + U <= p.splits; s += U) {
      float t[U][4];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int q = 0; q < 4; ++q) t[u][q] = (n + q < p.N) ? src[(int64_t)(s + u) * mn + q] : 0.f;
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] += t[u][q];
    }
    for (; s < p.splits; ++s) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (n + q < p.N) v[q] += src[(int64_t)s * mn + q];
    }
  }
  float b[4], a[4] = {0.f, 0.f, 0.f, 0.f}, r[4] = {0.f, 0.f, 0.f, 0.f};
  epi_bias(p.ep, n, false, b);
  epi_fetch(p.ep, m, n, false, a, r);
  epi_apply(p.ep, m, n, v, b, a, r, false);
}

// Many splits over a small output (the narrow weight gradient: 32 splits of
// a 2048 x 10 tile): eight lanes per group of four columns, lane u adding
// splits u, u+8, ... in order, then a fixed butterfly over the eight lanes,
// so the pass takes one or two memory round trips instead of one per split.
__global__ __launch_bounds__(256) void splitk_finish_wide_kernel(GemmParams p) {
  const int groups = (p.N + 3) >> 2;
  const int64_t items = (int64_t)p.M * groups;
  const int64_t g = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 3;
  const int u = threadIdx.x & 7;
  const bool live = g < items;
  const int m = live ? (int)(g / groups) : 0;
  const int n = live ? (int)(g % groups) * 4 : 0;
  const int64_t mn = (int64_t)p.M * p.N;
  const float *src = p.partial + (int64_t)m * p.N + n;
  float v[4] = {0.f, 0.f, 0.f, 0.f};
  if (live) {
    int s = u;
    for (; s + 8 * 3 < p.splits; s += 8 * 4) {
      float t[4][4];
#pragma unroll
      for (int w = 0; w < 4; ++w)
#pragma unroll
        for (int q = 0; q < 4; ++q) t[w][q] = (n + q < p.N) ? src[(int64_t)(s + 8 * w) * mn + q] : 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w)
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] += t[w][q];
    }
    for (; s < p.splits; s += 8) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (n + q < p.N) v[q] += src[(int64_t)s * mn + q];
    }
  }
#pragma unroll
  for (int o = 1; o < 8; o <<= 1) {
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] += __shfl_xor(v[q], o, 64);
  }
  if (!live || u != 0) return;
  const f32x4 acc = {v[0], v[1], v[2], v[3]};
  float b[4], a[4] = {0.f, 0.f, 0.f, 0.f}, r[4] = {0.f, 0.f, 0.f, 0.f};
  epi_bias(p.ep, n, false, b);
  epi_fetch(p.ep, m, n, false, a, r);
  epi_apply(p.ep, m, n, acc, b, a, r, false);
}

// ---- host launcher --------------------------------------------------------------
namespace {

int64_t ntiles(int64_t M, int64_t N, int t) { return ((M + t - 1) / t) * ((N + t - 1) / t); }
int64_t t256_128(int64_t M, int64_t N) { return ((M + 255) / 256) * ((N + 127) / 128); }
// shapes the eight-wave kernel takes: whole 16-byte chunks along every dimension
bool x8_shape(int64_t M, int64_t N, int64_t K) { return M % 8 == 0 && N % 8 == 0 && K % 8 == 0 && M >= 8 && N >= 8; }

Plan make_plan(int ab_type, int64_t M, int64_t N, int64_t K, int split_k) {
  Plan pl;
  pl.x8 = 0;
  const int bk = ab_type == GE_F32 ? 32 : 64;
  const int nk = (int)((K + bk - 1) / bk);
  const int64_t t256 = ntiles(M, N, 256);
  int s = 0;  // 0: chosen below with the tile
  // The 256x256 tile is the most efficient per k-step.  Use it when the
  // output alone gives most of the 256 CUs a tile.  When K is long enough
  // that splitting it (at least 8 k-tiles per split) fills the CUs, split
  // 256x128 tiles: measured on the weight-gradient shapes (K = batch 4096),
  // half the splits' FP32 partial traffic outweighs the larger tile's
  // cheaper k-steps (2048x2048: 51.8 against 53.3 us with the finishing
  // pass; 784x2048: 33.4 against 35.4 us).
  if (N <= 16 && M > 16) {
    // one narrow column of tiles; split-K supplies the parallelism
    pl.bm = 128;
    pl.bn = 16;
  } else if (t256 >= 192) {
    pl.bm = pl.bn = 256;
  } else if (split_k < 1 && nk >= 48 && t256 * std::min<int64_t>(nk / 8, 64) >= 192) {
    pl.bm = 256;
    pl.bn = 128;
    const int64_t t = t256_128(M, N);
    s = (int)std::min<int64_t>({(256 + t - 1) / t, nk / 8, 64});
  } else if (split_k < 1 && t256_128(M, N) >= 192 && (nk >= 24 || (ab_type != GE_F32 && nk >= 12 && x8_shape(M, N, K)))) {
    // 256x128: less operand traffic into LDS per MFMA than 128x128; on four
    // waves measured faster once the k loop is long (slower at 13 k-tiles),
    // on the eight-wave kernel already at 13
    pl.bm = 256;
    pl.bn = 128;
  } else if (ntiles(M, N, 128) >= 160) {
    pl.bm = pl.bn = 128;
  } else {
    pl.bm = pl.bn = 64;
  }
  pl.BK = bk;
  pl.tiles_m = (int)((M + pl.bm - 1) / pl.bm);
  pl.tiles_n = (int)((N + pl.bn - 1) / pl.bn);
  pl.nk = nk;
  if (split_k >= 1) {
    s = split_k;
  } else if (s == 0) {
    s = 1;
    const int64_t tiles = (int64_t)pl.tiles_m * pl.tiles_n;
    // split long K loops when the output alone cannot fill the 256 CUs
    if (tiles < 256 && pl.nk >= 16) {
      // (a narrow tile is bound by reading A, so short splits still pay)
      const int64_t want = (512 + tiles - 1) / tiles;
      s = (int)std::min<int64_t>(want, pl.nk / (pl.bn == 16 ? 2 : 8));
      s = std::max(1, std::min(s, 64));
    } else if (ab_type != GE_F32 && pl.bn == 64 && tiles <= 16 && pl.nk >= 8) {
      // a handful of 64x64 tiles with a short k loop waits on each k-step's
      // loads: runs of three or four k-tiles per split, even with the
      // finishing pass (128x256x784 FP16, eight tiles, GPU time per launch:
      // 12.3 / 9.5 / 14.9 us NN / NT / TN in one launch, 9.0 / 8.1 / 9.8
      // split four ways)
      s = pl.nk / 3;
    }
  }
  s = std::max(1, std::min(s, std::max(1, pl.nk)));
  pl.kps = (pl.nk + s - 1) / s;
  pl.splits = pl.kps > 0 ? (pl.nk + pl.kps - 1) / pl.kps : 1;
  return pl;
}

}  // namespace

int64_t gemm_ws_bytes(int layout, int ab_type, int64_t M, int64_t N, int64_t K, int split_k) {
  (void)layout;
  if (M <= 0 || N <= 0) return 0;
  Plan pl = make_plan(ab_type, M, N, K, split_k);
  if (pl.splits <= 1) return 0;
  return (int64_t)pl.splits * M * N * 4;
}

namespace {
// the epilogue's 4-wide access checks (as store_tile's fast path reads them)
int al4(const void *ptr, int64_t ld, int t) {
  return ptr ? (int)vec_aligned(ptr, ld, dtype_size(t), 4 * dtype_size(t)) : 0;
}
// every tile of the plan takes the fast epilogue, K is not split and the
// tile's kernel carries the column sums (all but the 256x256 tiles), so the
// epilogue can also write per-tile-row column sums of C
bool colsum_fusable(const Plan &pl, const ge_gemm_args &a) {
  const bool bwd = a.act == GE_ACT_RELU_MASK_BWD || a.act == GE_ACT_LRELU_SQ_BWD;
  return pl.splits == 1 && pl.bn < 256 && a.M % pl.bm == 0 && a.N % pl.bn == 0 && al4(a.C, a.ldc, a.c_type) &&
         (!a.aux || al4(a.aux, a.ld_aux, a.aux_type)) && (!a.residual || al4(a.residual, a.ld_res, a.res_type)) &&
         (!a.pre || al4(a.pre, a.ld_pre, a.pre_type)) && (!a.bias || ((uintptr_t)a.bias % 16) == 0) &&
         !(bwd && a.residual);
}
}  // namespace

int64_t gemm_colsum_rows(const ge_gemm_args &a) {
  if (a.M <= 0 || a.N <= 0) return 0;
  Plan pl = make_plan(a.ab_type, a.M, a.N, a.K, a.split_k);
  return colsum_fusable(pl, a) ? pl.tiles_m : 0;
}

int64_t gemm_colsum_bytes(int ab_type, int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0) return 0;
  Plan pl = make_plan(ab_type, M, N, K, 0);
  return pl.splits == 1 && pl.bn < 256 ? (int64_t)pl.tiles_m * N * 4 : 0;
}

int gemm_launch(const ge_gemm_args &a, hipStream_t s, float *colpart, int *deferred) {
  if (deferred) *deferred = 0;
  if (a.M == 0 || a.N == 0) return GE_OK;
  Plan pl = make_plan(a.ab_type, a.M, a.N, a.K, a.split_k);
  if (colpart != nullptr && (!colsum_fusable(pl, a) || ((uintptr_t)colpart % 16) != 0)) {
    set_error("gemm_bias_act: column sums in the epilogue need unsplit, whole, aligned tiles");
    return GE_E_INVALID;
  }
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
  // the fast loads address up to 64 operand rows from one per-thread 32-bit offset
  gp.off32 = (a.lda * es * 64 < ((int64_t)1 << 31)) && (a.ldb * es * 64 < ((int64_t)1 << 31));
  // clamped edge loads: 16-byte vectors must stay whole inside the rows of an
  // operand stored along m / n (A of TN, B of NN and TN)
  {
    const int64_t v = 16 / es;
    const bool a_mc = a.layout == GE_TN, b_mc = a.layout != GE_NT;
    gp.clamp = gp.a_vec && gp.b_vec && a.M >= v && a.N >= v && (!a_mc || a.M % v == 0) && (!b_mc || a.N % v == 0);
  }
  // the eight-wave kernel takes the plan's 256x256 or 256x128 tiles (same
  // tiles and splits, so the same workspace) when M, N and K are multiples of
  // 8 (edge tiles read clamped rows, the last k-tile is zero-padded), the
  // rows are 16-byte aligned and the buffer offsets of one tile stay below
  // 2^31 bytes
  if ((a.ab_type == GE_F16 || a.ab_type == GE_BF16) && pl.bm == 256 && (pl.bn == 256 || pl.bn == 128) &&
      x8_shape(a.M, a.N, a.K) && gp.a_vec && gp.b_vec) {
    auto span = [&](bool kc, int64_t ld, int64_t w) { return kc ? ((w - 1) * ld + a.K) * es : (a.K * ld + w) * es; };
    const bool a_kc = a.layout != GE_TN, b_kc = a.layout == GE_NT;
    if (span(a_kc, a.lda, 256) < ((int64_t)1 << 31) && span(b_kc, a.ldb, pl.bn) < ((int64_t)1 << 31))
      pl.x8 = pl.bn == 256 ? 1 : 2;
  }
  gp.tiles_m = pl.tiles_m;
  gp.tiles_n = pl.tiles_n;
  gp.ktiles_per_split = pl.kps;
  gp.splits = pl.splits;
  gp.partial = nullptr;
  if (pl.splits > 1) {
    const int64_t need = (int64_t)pl.splits * a.M * a.N * 4;
    if (a.workspace == nullptr || a.workspace_bytes < need || ((uintptr_t)a.workspace % 16) != 0) {
      set_error("gemm_bias_act: split-K over %d splits needs %lld workspace bytes (16-byte aligned)",
                pl.splits, (long long)need);
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
  e.colpart = colpart;
  e.aux_vec = al4(a.aux, a.ld_aux, a.aux_type);
  e.res_vec = al4(a.residual, a.ld_res, a.res_type);
  e.c_vec = al4(a.C, a.ldc, a.c_type);
  e.pre_vec = al4(a.pre, a.ld_pre, a.pre_type);
  e.bias_vec = a.bias ? (((uintptr_t)a.bias % 16) == 0) : 0;

  if (a.ab_type == GE_F16) gemm_dispatch_f16(a.layout, pl, gp, s);
  else if (a.ab_type == GE_BF16) gemm_dispatch_bf16(a.layout, pl, gp, s);
  else gemm_dispatch_f32(a.layout, pl, gp, s);
  int st = launch_status("gemm_bias_act");
  if (st != GE_OK || pl.splits <= 1) return st;
  // a plain FP32 result (alpha times the sum, row-major, nothing else in the
  // epilogue) may leave its split partials for the caller to add
  if (deferred && !a.bias && a.act == GE_ACT_NONE && !a.aux && !a.residual && !a.pre && a.c_type == GE_F32 &&
      a.ldc == a.N) {
    *deferred = pl.splits;
    return GE_OK;
  }
  const int64_t items = a.M * ((a.N + 3) / 4);
  if (items < (64 << 10) && pl.splits >= 8)
    hipLaunchKernelGGL(splitk_finish_wide_kernel, dim3((unsigned)((items * 8 + 255) / 256)), dim3(256), 0, s, gp);
  else
    hipLaunchKernelGGL(splitk_finish_kernel, dim3((unsigned)((items + 255) / 256)), dim3(256), 0, s, gp);
  return launch_status("gemm_bias_act (split-K finish)");
}

namespace {
std::mutex g_scratch_mu;
void *g_scratch_ptr[64] = {nullptr};
}  // namespace

// device address of this device's scratch array (looked up once per device)
int scratch_address(void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= 64) {
    set_error("gemm_bias_act_noalloc: no usable current device (%s)", hipGetErrorString(e));
    return GE_E_LAUNCH;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      set_error("gemm_bias_act_noalloc: hipGetSymbolAddress failed (%s)", hipGetErrorString(e));
      return GE_E_LAUNCH;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return GE_OK;
}

int64_t scratch_bytes() { return kScratchBytes; }

}  // namespace ge
