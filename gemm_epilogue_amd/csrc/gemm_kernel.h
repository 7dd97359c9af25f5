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
// Design (ours, not the pages'): a block computes a BM x BN tile (256x256 on
// 8 wavefronts, 128x128 or 64x64 on 4, by problem size); A and B tiles of BK
// along k are staged through LDS, double-buffered, always stored k-contiguous
// ([row][k], 128-byte rows whose 16-byte chunks are XOR-swizzled by row) so
// each MFMA fragment is one 16-byte LDS read per lane and the 16 lanes that
// read one fragment hit 16 different bank groups.  Operands contiguous along
// m/n in memory (B of NN, both of TN) are transposed in registers on their way
// into LDS.  The 256x256 tile runs a ping-pong schedule: its two wave groups
// alternate between MFMA work on one buffer and staging the next k-tile into
// the other.  Tiles entirely inside the matrix use unconditional 16-byte
// loads and stores (a block-uniform branch); tiles on the M/N edge and the
// partial last k-tile use checked element loads.  MFMA 16x16 tiles are issued
// with the B tile in the instruction's first operand slot, so each lane owns
// four consecutive columns of one output row.  FP16/BF16 use
// v_mfma_f32_16x16x32_{f16,bf16}; FP32 uses v_mfma_f32_16x16x4_f32.  Split-K
// writes FP32 partials to a workspace and a finishing kernel sums them in
// split order, then applies the same epilogue.
#pragma once
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
  // optional: per-tile-row column sums of the stored C ([tiles_m x N] FP32),
  // for the bias gradient of a layer whose dZ this GEMM writes; the host sets
  // it only when every tile takes the fast epilogue and K is not split
  float *colpart;
};

struct GemmParams {
  const void *A;
  const void *B;
  int64_t lda, ldb;
  int M, N, K;
  int a_vec, b_vec;
  int off32;  // per-thread operand offsets of the fast loads fit in 31 bits
  int clamp;  // edge tiles may use vector loads with clamped rows / columns
  int tiles_m, tiles_n;
  int ktiles_per_split;
  int splits;
  float *partial;  // [splits][M][N] when splits > 1
  EpiParams ep;
};

// Epilogue for four consecutive columns n..n+3 of row m, in three steps so a
// caller can batch the memory accesses of several rows: the bias of the
// column group (loaded once per thread), the per-element inputs (aux for the
// derivative epilogues, residual), then the arithmetic and the store.
// `fast`: the four columns are inside the matrix and every access is aligned.
__device__ __forceinline__ void epi_bias(const EpiParams &e, int n, bool fast, float b[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) b[j] = 0.f;
  if (!e.bias || n >= e.N) return;
  if ((fast || n + 3 < e.N) && e.bias_vec) {
    const f32x4 x = *(const f32x4 *)(e.bias + n);
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = x[j];
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = (n + j < e.N) ? e.bias[n + j] : 0.f;
  }
}

__device__ __forceinline__ void epi_fetch(const EpiParams &e, int m, int n, bool fast, float a[4], float r[4]) {
  if (!fast && (m >= e.M || n >= e.N)) return;
  const bool full = fast || (n + 3) < e.N;
  if (e.act == GE_ACT_RELU_MASK_BWD || e.act == GE_ACT_LRELU_SQ_BWD) {
    if (full) {
      load4_any(e.aux, (int64_t)m * e.ld_aux + n, e.aux_type, e.aux_vec, a);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        a[j] = (n + j < e.N) ? load_any(e.aux, (int64_t)m * e.ld_aux + n + j, e.aux_type) : 0.f;
    }
  }
  if (e.res) {
    if (full) {
      load4_any(e.res, (int64_t)m * e.ld_res + n, e.res_type, e.res_vec, r);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        r[j] = (n + j < e.N) ? load_any(e.res, (int64_t)m * e.ld_res + n + j, e.res_type) : 0.f;
    }
  }
}

__device__ __forceinline__ void epi_apply(const EpiParams &e, int m, int n, f32x4 acc, const float b[4],
                                          const float a[4], const float r[4], bool fast) {
  if (!fast && (m >= e.M || n >= e.N)) return;
  const bool full = fast || (n + 3) < e.N;
  float v[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) v[j] = e.alpha * acc[j] + b[j];
  if (e.pre) {
    if (full) {
      store4_any(e.pre, (int64_t)m * e.ld_pre + n, e.pre_type, e.pre_vec, v);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (n + j < e.N) store_any(e.pre, (int64_t)m * e.ld_pre + n + j, e.pre_type, v[j]);
    }
  }
  if (e.act == GE_ACT_RELU) {
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = fmaxf(v[j], 0.f);
  } else if (e.act == GE_ACT_LRELU_SQ) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float t = v[j] > 0.f ? v[j] : e.slope * v[j];
      v[j] = t * t;
    }
  } else if (e.act == GE_ACT_RELU_MASK_BWD) {
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = a[j] > 0.f ? v[j] : 0.f;
  } else if (e.act == GE_ACT_LRELU_SQ_BWD) {
    const float s2 = 2.f * e.slope * e.slope;
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] *= (a[j] > 0.f ? 2.f * a[j] : s2 * a[j]);
  }
  if (e.res) {
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] += r[j];
  }
  if (full) {
    store4_any(e.C, (int64_t)m * e.ldc + n, e.c_type, e.c_vec, v);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (n + j < e.N) store_any(e.C, (int64_t)m * e.ldc + n + j, e.c_type, v[j]);
  }
}

// ---- epilogue fast path for interior tiles ------------------------------------
// The output element size CS (2 or 4 bytes) and the element size XS of at
// most one extra per-element input (0: none; otherwise the aux of a
// derivative epilogue or the residual) are template parameters, so the row
// loop is straight-line code.  The extra input of the next batch of rows is
// loaded before the stores of the current batch: the vector-memory counter of
// this GPU counts stores as well as loads, and a wait for a load issued after
// a store would also wait for the store.
template <int XS> struct RawOf { typedef uint32_t __attribute__((ext_vector_type(2))) T; };
template <> struct RawOf<4> { typedef uint32_t __attribute__((ext_vector_type(4))) T; };

template <typename R> __device__ __forceinline__ void raw_to_f4(const R &w, int t, float v[4]) {
  if constexpr (sizeof(R) == 16) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // element copied to a scalar first: a bit cast of the vector element
      // itself compiles to a read of element 0
      const uint32_t u = w[j];
      v[j] = __builtin_bit_cast(float, u);
    }
  } else if (t == GE_F16) {
    const f16x4 h = __builtin_bit_cast(f16x4, w);
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = (float)h[j];
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t u = (j & 1) ? (w[j >> 1] & 0xffff0000u) : (w[j >> 1] << 16);
      v[j] = __builtin_bit_cast(float, u);
    }
  }
}

template <int CS> __device__ __forceinline__ void store_c4(void *C, int64_t i, int ct, const float v[4]) {
  if constexpr (CS == 4) {
    *(f32x4 *)((float *)C + i) = f32x4{v[0], v[1], v[2], v[3]};
  } else if (ct == GE_F16) {
    *(f16x4 *)((half_t *)C + i) = f16x4{(half_t)v[0], (half_t)v[1], (half_t)v[2], (half_t)v[3]};
  } else {
    *(bf16x4 *)((bf16_t *)C + i) = bf16x4{(bf16_t)v[0], (bf16_t)v[1], (bf16_t)v[2], (bf16_t)v[3]};
  }
}

// the value a store of v in the output type leaves in memory
template <int CS> __device__ __forceinline__ float stored_value(float v, int ct) {
  if constexpr (CS == 4) return v;
  else return ct == GE_F16 ? (float)(half_t)v : (float)(bf16_t)v;
}

// Rows m_base + r0 + q*RS (q < RPT) of the staged tile, columns n..n+3,
// in batches of EU rows; with CSUM and e.colpart, csum gathers the stored
// values.
template <int CS, int XS, int RPT, int EU, int RS, int CSTRIDE, bool CSUM>
__device__ __forceinline__ void epi_rows_fast(const EpiParams &e, const float *cs, int m_base, int r0, int cg,
                                              int n, const float b[4], float (&csum)[4]) {
  const bool bwd = e.act == GE_ACT_RELU_MASK_BWD || e.act == GE_ACT_LRELU_SQ_BWD;
  const char *xp = (const char *)(bwd ? e.aux : e.res);
  const int64_t ldx = bwd ? e.ld_aux : e.ld_res;
  const int xt = bwd ? e.aux_type : e.res_type;
  typedef typename RawOf<XS>::T X;
  constexpr int NB = RPT / EU;
  X xr[NB][EU];
  auto fetch = [&](int bb) {
#pragma unroll
    for (int u = 0; u < EU; ++u) {
      const int64_t m = m_base + r0 + (bb * EU + u) * RS;
      xr[bb][u] = *(const X *)(xp + (m * ldx + n) * XS);
    }
  };
  if constexpr (XS > 0) fetch(0);
#pragma unroll
  for (int bb = 0; bb < NB; ++bb) {
    if constexpr (XS > 0) {
      if (bb + 1 < NB) fetch(bb + 1);
    }
#pragma unroll
    for (int u = 0; u < EU; ++u) {
      const int rr = r0 + (bb * EU + u) * RS;
      const f32x4 acc = *(const f32x4 *)(cs + rr * CSTRIDE + cg * 4);
      const int64_t m = m_base + rr;
      float v[4], x[4] = {0.f, 0.f, 0.f, 0.f};
      if constexpr (XS > 0) raw_to_f4(xr[bb][u], xt, x);
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = e.alpha * acc[j] + b[j];
      if (e.pre) store4_any(e.pre, m * e.ld_pre + n, e.pre_type, true, v);
      if (e.act == GE_ACT_RELU) {
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = fmaxf(v[j], 0.f);
      } else if (e.act == GE_ACT_LRELU_SQ) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float t = v[j] > 0.f ? v[j] : e.slope * v[j];
          v[j] = t * t;
        }
      } else if (e.act == GE_ACT_RELU_MASK_BWD) {
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = x[j] > 0.f ? v[j] : 0.f;
      } else if (e.act == GE_ACT_LRELU_SQ_BWD) {
        const float s2 = 2.f * e.slope * e.slope;
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] *= (x[j] > 0.f ? 2.f * x[j] : s2 * x[j]);
      }
      if (XS > 0 && !bwd) {
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] += x[j];
      }
      store_c4<CS>(e.C, m * e.ldc + n, e.c_type, v);
      if constexpr (CSUM) {
        if (e.colpart) {
#pragma unroll
          for (int j = 0; j < 4; ++j) csum[j] += stored_value<CS>(v[j], e.c_type);
        }
      }
    }
  }
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

// The same products with the accumulator pinned to the accumulation
// registers (AGPRs), for the kernel whose 256 accumulator registers per lane
// fill that file: with the builtin the register allocator moves accumulators
// between the two register files inside the k loop.
template <typename T> struct FragA;
template <> struct FragA<half_t> {
  static __device__ __forceinline__ void mma(const f16x8 &a, const f16x8 &b, f32x4 &c) {
    asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
  }
};
template <> struct FragA<bf16_t> {
  static __device__ __forceinline__ void mma(const bf16x8 &a, const bf16x8 &b, f32x4 &c) {
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
  }
};
template <> struct FragA<float> {
  static __device__ __forceinline__ void mma(const f32x4 &a, const f32x4 &b, f32x4 &c) {
    asm volatile("v_mfma_f32_16x16x4_f32 %0, %1, %2, %0\n\t"
                 "v_mfma_f32_16x16x4_f32 %0, %3, %4, %0\n\t"
                 "v_mfma_f32_16x16x4_f32 %0, %5, %6, %0\n\t"
                 "v_mfma_f32_16x16x4_f32 %0, %7, %8, %0"
                 : "+a"(c)
                 : "v"(a[0]), "v"(b[0]), "v"(a[1]), "v"(b[1]), "v"(a[2]), "v"(b[2]), "v"(a[3]), "v"(b[3]));
  }
};

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// element e of a 16-byte vector holding T values, as raw bits
template <typename T> __device__ __forceinline__ uint32_t elem_bits(const u32x4 &v, int e) {
  if constexpr (sizeof(T) == 4) return v[e];
  else return (e & 1) ? (v[e >> 1] >> 16) : (v[e >> 1] & 0xffffu);
}
template <typename T> __device__ __forceinline__ uint32_t bits_of(T x) {
  if constexpr (sizeof(T) == 4) return __builtin_bit_cast(uint32_t, x);
  else return (uint32_t)__builtin_bit_cast(uint16_t, x);
}

// ---- LDS tile layout ---------------------------------------------------------
// Tile rows are 128 bytes (eight 16-byte chunks) with no padding; chunk q of
// row r is stored at chunk q ^ s(r >> 1), s(p) = 4 (p & 1) + ((p >> 1) & 3).
// s takes all eight values over eight consecutive row pairs, so the MFMA
// fragment read (16 consecutive rows, one chunk) hits 16 distinct bank
// groups; consecutive row pairs differ in bit 2 of s, so a write of half a
// row (one 32-wide k-chunk) by 16 lanes covering four rows does as well.
// (A 16-byte row pad costs two-way conflicts on the fragment reads.)
__device__ __forceinline__ int lds_chunk(int row, int q) {
  const int p = row >> 1;
  return q ^ (((p & 1) << 2) | ((p >> 1) & 3));
}

// ---- tile loaders ------------------------------------------------------------
// k-contiguous source: R rows (m or n) x BK, each row contiguous along k.
// Thread t moves vectors v = t + i*NT: row v / VPR, 16-byte chunk v % VPR.
template <typename T, int R, int BK, int NT> struct LoaderKC {
  static constexpr int VEC = 16 / sizeof(T);
  static constexpr int VPR = BK / VEC;  // vectors per row
  static constexpr int NVEC = R * VPR;  // vectors in the tile
  static constexpr int NV = (NVEC + NT - 1) / NT;
  // a tile with fewer vectors than threads leaves the upper threads idle
  static constexpr bool PART = NVEC < NT;
  static_assert(PART || NVEC % NT == 0, "tile / thread mismatch");
  u32x4 r[NV];

  // vector i of thread t sits at tile row t / VPR + i * (NT / VPR): a
  // block-uniform row base plus one 32-bit per-thread byte offset (the host
  // only takes this path when NT / VPR rows of the operand span < 2 GiB)
  __device__ __forceinline__ void load_fast(const T *__restrict__ p, int64_t ld, int r0, int k0, int tid) {
    if constexpr (PART) {
      if (tid < NVEC) r[0] = *(const u32x4 *)(p + (int64_t)(r0 + tid / VPR) * ld + k0 + (tid % VPR) * VEC);
    } else {
      static_assert(NT % VPR == 0, "whole rows per round");
      const uint32_t off = (uint32_t)(((tid / VPR) * ld + (tid % VPR) * VEC) * (int64_t)sizeof(T));
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const char *base = (const char *)(p + (int64_t)(r0 + i * (NT / VPR)) * ld + k0);
        r[i] = *(const u32x4 *)(base + off);
      }
    }
  }
  // edge tiles of an aligned operand, full k-tile: rows past rmax re-read row
  // rmax - 1; they only feed accumulator rows that are never stored
  __device__ __forceinline__ void load_clamped(const T *__restrict__ p, int64_t ld, int r0, int rmax, int k0,
                                               int tid) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int v = tid + i * NT;
      if (PART && v >= NVEC) continue;
      const int row = min(r0 + v / VPR, rmax - 1);
      r[i] = *(const u32x4 *)(p + (int64_t)row * ld + k0 + (v % VPR) * VEC);
    }
  }
  // single fast loads / LDS writes, for spreading them over MFMA work
  static constexpr int NLOAD = NV, NSTORE = NV;
  __device__ __forceinline__ void load_piece(const T *__restrict__ p, int64_t ld, int r0, int k0, int tid, int i) {
    const uint32_t off = (uint32_t)(((tid / VPR) * ld + (tid % VPR) * VEC) * (int64_t)sizeof(T));
    const char *base = (const char *)(p + (int64_t)(r0 + i * (NT / VPR)) * ld + k0);
    r[i] = *(const u32x4 *)(base + off);
  }
  // qoff: 16-byte chunk offset of this k-slice within the LDS row
  __device__ __forceinline__ void store_piece(T *s, int stride, int tid, int i, int qoff = 0) const {
    const int v = tid + i * NT;
    const int row = v / VPR;
    *(u32x4 *)(s + row * stride + lds_chunk(row, v % VPR + qoff) * VEC) = r[i];
  }
  // quarters of the same
  __device__ __forceinline__ void load_fast_q(const T *__restrict__ p, int64_t ld, int r0, int k0, int tid, int q) {
    static_assert(!PART && NV % 4 == 0, "quarters of whole rounds");
    const uint32_t off = (uint32_t)(((tid / VPR) * ld + (tid % VPR) * VEC) * (int64_t)sizeof(T));
#pragma unroll
    for (int i = q * NV / 4; i < (q + 1) * NV / 4; ++i) {
      const char *base = (const char *)(p + (int64_t)(r0 + i * (NT / VPR)) * ld + k0);
      r[i] = *(const u32x4 *)(base + off);
    }
  }
  __device__ __forceinline__ void store_q(T *s, int stride, int tid, int q) const {
#pragma unroll
    for (int i = q * NV / 4; i < (q + 1) * NV / 4; ++i) {
      const int v = tid + i * NT;
      const int row = v / VPR;
      *(u32x4 *)(s + row * stride + lds_chunk(row, v % VPR) * VEC) = r[i];
    }
  }
  __device__ __forceinline__ void load_checked(const T *__restrict__ p, int64_t ld, int r0, int rmax, int k0,
                                               int kmax, bool vec, int tid) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int v = tid + i * NT;
      if (PART && v >= NVEC) continue;
      const int gr = r0 + v / VPR, gk = k0 + (v % VPR) * VEC;
      if (vec && gr < rmax && gk + VEC <= kmax) {
        r[i] = *(const u32x4 *)(p + (int64_t)gr * ld + gk);
      } else {
        uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const uint32_t b = (gr < rmax && gk + e < kmax) ? bits_of<T>(p[(int64_t)gr * ld + gk + e]) : 0u;
          if constexpr (sizeof(T) == 4) w[e] = b;
          else w[e >> 1] |= b << (16 * (e & 1));
        }
        r[i] = u32x4{w[0], w[1], w[2], w[3]};
      }
    }
  }
  __device__ __forceinline__ void store(T *s, int stride, int tid) const {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int v = tid + i * NT;
      if (PART && v >= NVEC) continue;
      const int row = v / VPR;
      *(u32x4 *)(s + row * stride + lds_chunk(row, v % VPR) * VEC) = r[i];
    }
  }
};

// m/n-contiguous source: BK k-rows, each contiguous along the R dimension.
// Thread t owns k-group kg = t % NKG (KB consecutive k-rows) and vector
// rv = t / NKG (VEC consecutive rows of the tile); it writes VEC LDS rows of
// KB k-values.  Consecutive lanes take consecutive k-groups, so one LDS write
// instruction spreads over distinct 16-byte bank groups.
template <typename T, int R, int BK, int NT> struct LoaderMC {
  static constexpr int VEC = 16 / sizeof(T);
  static constexpr int RV = R / VEC;  // vectors per k-row
  // k-rows per thread; a narrow tile gives each active thread two k-rows and
  // leaves threads ACTIVE.. idle
  static constexpr int KB = BK * RV / NT >= 2 ? BK * RV / NT : 2;
  static constexpr int NKG = BK / KB;
  static constexpr int ACTIVE = NKG * RV;
  static constexpr bool PART = ACTIVE < NT;
  static constexpr int W = KB * sizeof(T) / 4;  // dwords per transposed row piece
  static_assert(RV >= 1 && BK % KB == 0 && ACTIVE <= NT && (PART || BK * RV == KB * NT), "tile / thread mismatch");
  static_assert(W == 1 || W == 2 || W % 4 == 0, "transposed piece must be 4, 8 or 16n bytes");
  u32x4 x[KB];

  // k-row j of thread t: a block-uniform row base plus one 32-bit per-thread
  // byte offset
  __device__ __forceinline__ void load_fast(const T *__restrict__ p, int64_t ld, int r0, int k0, int tid) {
    if (PART && tid >= ACTIVE) return;
    const int kg = tid % NKG, rv = tid / NKG;
    const uint32_t off = (uint32_t)(((int64_t)(kg * KB) * ld + rv * VEC) * (int64_t)sizeof(T));
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      const char *base = (const char *)(p + (int64_t)(k0 + j) * ld + r0);
      x[j] = *(const u32x4 *)(base + off);
    }
  }
  __device__ __forceinline__ void load_checked(const T *__restrict__ p, int64_t ld, int r0, int rmax, int k0,
                                               int kmax, bool vec, int tid) {
    if (PART && tid >= ACTIVE) return;
    const int kg = tid % NKG, rv = tid / NKG;
    const int gr = r0 + rv * VEC;
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      const int gk = k0 + kg * KB + j;
      if (vec && gk < kmax && gr + VEC <= rmax) {
        x[j] = *(const u32x4 *)(p + (int64_t)gk * ld + gr);
      } else {
        uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const uint32_t b = (gk < kmax && gr + e < rmax) ? bits_of<T>(p[(int64_t)gk * ld + gr + e]) : 0u;
          if constexpr (sizeof(T) == 4) w[e] = b;
          else w[e >> 1] |= b << (16 * (e & 1));
        }
        x[j] = u32x4{w[0], w[1], w[2], w[3]};
      }
    }
  }
  // transposed write of column e of the KB x VEC block: KB k-values of tile
  // row rv*VEC + e
  __device__ __forceinline__ void store_e(T *s, int stride, int kg, int rv, int e, int qoff = 0) const {
    uint32_t w[W];
#pragma unroll
    for (int q = 0; q < W; ++q) {
      if constexpr (sizeof(T) == 4) w[q] = elem_bits<T>(x[q], e);
      else w[q] = elem_bits<T>(x[2 * q], e) | (elem_bits<T>(x[2 * q + 1], e) << 16);
    }
    // bytes [b, b + 4W) of tile row `row`; pieces of at most 16 bytes never
    // straddle a 16-byte chunk, so each is placed by its chunk's swizzle
    const int row = rv * VEC + e;
    const int b = kg * KB * (int)sizeof(T) + qoff * 16;
    char *rbase = (char *)(s + row * stride);
    if constexpr (W == 1) {
      *(uint32_t *)(rbase + lds_chunk(row, b >> 4) * 16 + (b & 15)) = w[0];
    } else if constexpr (W == 2) {
      *(u32x2 *)(rbase + lds_chunk(row, b >> 4) * 16 + (b & 15)) = u32x2{w[0], w[1]};
    } else {
#pragma unroll
      for (int q = 0; q < W; q += 4)
        *(u32x4 *)(rbase + lds_chunk(row, (b >> 4) + q / 4) * 16) = u32x4{w[q], w[q + 1], w[q + 2], w[q + 3]};
    }
  }
  __device__ __forceinline__ void store(T *s, int stride, int tid) const {
    if (PART && tid >= ACTIVE) return;
    const int kg = tid % NKG, rv = tid / NKG;
#pragma unroll
    for (int e = 0; e < VEC; ++e) store_e(s, stride, kg, rv, e);
  }
  // edge tiles (rmax a multiple of VEC), full k-tile: vectors past rmax
  // re-read the last one; they only feed accumulators that are never stored
  __device__ __forceinline__ void load_clamped(const T *__restrict__ p, int64_t ld, int r0, int rmax, int k0,
                                               int tid) {
    if (PART && tid >= ACTIVE) return;
    const int kg = tid % NKG, rv = tid / NKG;
    const int col = min(r0 + rv * VEC, rmax - VEC);
#pragma unroll
    for (int j = 0; j < KB; ++j) x[j] = *(const u32x4 *)(p + (int64_t)(k0 + kg * KB + j) * ld + col);
  }
  // single fast loads (k-row j) and transposed LDS writes (column e); every
  // write reads all KB loaded vectors, so a step's writes precede its loads
  static constexpr int NLOAD = KB, NSTORE = VEC;
  __device__ __forceinline__ void load_piece(const T *__restrict__ p, int64_t ld, int r0, int k0, int tid, int j) {
    const int kg = tid % NKG, rv = tid / NKG;
    const uint32_t off = (uint32_t)(((int64_t)(kg * KB) * ld + rv * VEC) * (int64_t)sizeof(T));
    const char *base = (const char *)(p + (int64_t)(k0 + j) * ld + r0);
    x[j] = *(const u32x4 *)(base + off);
  }
  __device__ __forceinline__ void store_piece(T *s, int stride, int tid, int e, int qoff = 0) const {
    store_e(s, stride, tid % NKG, tid / NKG, e, qoff);
  }
  // quarters of the fast loads and of the LDS writes
  __device__ __forceinline__ void load_fast_q(const T *__restrict__ p, int64_t ld, int r0, int k0, int tid, int q) {
    static_assert(!PART && KB % 4 == 0, "quarters of whole rounds");
    const int kg = tid % NKG, rv = tid / NKG;
    const uint32_t off = (uint32_t)(((int64_t)(kg * KB) * ld + rv * VEC) * (int64_t)sizeof(T));
#pragma unroll
    for (int j = q * KB / 4; j < (q + 1) * KB / 4; ++j) {
      const char *base = (const char *)(p + (int64_t)(k0 + j) * ld + r0);
      x[j] = *(const u32x4 *)(base + off);
    }
  }
  __device__ __forceinline__ void store_q(T *s, int stride, int tid, int q) const {
    static_assert(VEC % 4 == 0, "quarters of the transposed writes");
    const int kg = tid % NKG, rv = tid / NKG;
#pragma unroll
    for (int e = q * VEC / 4; e < (q + 1) * VEC / 4; ++e) store_e(s, stride, kg, rv, e);
  }
};

template <typename T, bool KC, int R, int BK, int NT> struct Loader;
template <typename T, int R, int BK, int NT> struct Loader<T, true, R, BK, NT> : LoaderKC<T, R, BK, NT> {};
template <typename T, int R, int BK, int NT> struct Loader<T, false, R, BK, NT> : LoaderMC<T, R, BK, NT> {};

// ---- block -> (split, output tile) ---------------------------------------------
// Blocks are dealt round-robin over the 8 XCDs in dispatch order (x fastest,
// then the split index z).  The remap gives each XCD a contiguous run of the
// split-major work list -- so with split-K an XCD works on one split -- and
// tiles are ordered in groups of 8 tile-rows, so the A and B panels that an
// XCD's blocks share stay in its L2.
__device__ __forceinline__ void block_work(const GemmParams &p, int BM, int BN, int &bm0, int &bn0, int &split) {
  const int tiles = p.tiles_m * p.tiles_n;
  const int total = tiles * p.splits;
  int lin = blockIdx.x + tiles * blockIdx.z;
  if ((total & 7) == 0) lin = (lin & 7) * (total >> 3) + (lin >> 3);
  split = lin / tiles;
  const int bid = lin - split * tiles;
  constexpr int GROUP = 8;
  const int per_group = GROUP * p.tiles_n;
  const int first_m = (bid / per_group) * GROUP;
  const int gsize = min(p.tiles_m - first_m, GROUP);
  const int tm = first_m + (bid % per_group) % gsize;
  const int tn = (bid % per_group) / gsize;
  bm0 = tm * BM;
  bn0 = tn * BN;
}

// ---- epilogue of one BM x BN tile ---------------------------------------------------
// The FP32 tile is staged in LDS in NPASS passes of BM / NPASS rows; `stage`
// (pass, cs) writes the accumulators of that pass's rows into cs (row-major,
// CSTRIDE floats per row).  Then all threads walk the staged rows, four
// consecutive columns per thread, so global stores are whole-row coalesced.
template <int BM, int BN, int NT, int NPASS, int EUQ, bool CSUM, typename Stage>
__device__ __forceinline__ void store_tile_staged(const GemmParams &p, char *smem, int tid, int bm0, int bn0,
                                                  int split, Stage &&stage) {
  constexpr int RP = BM / NPASS;
  constexpr int CSTRIDE = BN + 4;  // floats per staged row (16-byte pad)
  const EpiParams &e = p.ep;
  const bool fast = (bm0 + BM <= p.M) && (bn0 + BN <= p.N) && e.c_vec && (!e.aux || e.aux_vec) &&
                    (!e.res || e.res_vec) && (!e.pre || e.pre_vec) && (!e.bias || e.bias_vec);
  float *cs = (float *)smem;
  float *part = p.splits > 1 ? p.partial + (int64_t)split * p.M * p.N : nullptr;
  const bool pvec = (p.N & 3) == 0;
  // each thread owns one group of four columns and rows r0, r0 + RS, ...
  constexpr int CG = BN / 4;
  static_assert(NT % CG == 0, "threads must tile whole staged rows");
  constexpr int RS = NT / CG;
  constexpr int RPT = RP / RS;
  // rows whose loads are issued together (fewer while a second pass still
  // holds its accumulators in registers)
  constexpr int EU = EUQ > 0 ? EUQ : (NPASS > 1 ? 2 : (RPT >= 4 ? 4 : RPT));
  static_assert(RPT % EU == 0, "rows per thread must split into batches");
  const int cg = tid % CG, r0 = tid / CG;
  const int n = bn0 + cg * 4;
  float bias[4];
  epi_bias(e, n, fast, bias);
  const bool bwd = e.act == GE_ACT_RELU_MASK_BWD || e.act == GE_ACT_LRELU_SQ_BWD;
  const void *xin = bwd ? e.aux : e.res;
  const int xin_type = bwd ? e.aux_type : e.res_type;
  float csum[4] = {0.f, 0.f, 0.f, 0.f};
  for (int pass = 0; pass < NPASS; ++pass) {
    stage(pass, cs);
    __syncthreads();
    const int m_base = bm0 + pass * RP;
    if (part != nullptr) {
      // split-K: raw FP32 partial sums, stores only
#pragma unroll
      for (int q = 0; q < RPT; ++q) {
        const int m = m_base + r0 + q * RS;
        const f32x4 v = *(const f32x4 *)(cs + (r0 + q * RS) * CSTRIDE + cg * 4);
        if (m < p.M && n < p.N) {
          float *dst = part + (int64_t)m * p.N + n;
          if (pvec && n + 3 < p.N) {
            *(f32x4 *)dst = v;
          } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
              if (n + j < p.N) dst[j] = v[j];
          }
        }
      }
    } else if (fast && !(bwd && e.res)) {
      const int xs = xin == nullptr ? 0 : (xin_type == GE_F32 ? 4 : 2);
      if (e.c_type == GE_F32) {
        if (xs == 0) epi_rows_fast<4, 0, RPT, EU, RS, CSTRIDE, CSUM>(e, cs, m_base, r0, cg, n, bias, csum);
        else if (xs == 2) epi_rows_fast<4, 2, RPT, EU, RS, CSTRIDE, CSUM>(e, cs, m_base, r0, cg, n, bias, csum);
        else epi_rows_fast<4, 4, RPT, EU, RS, CSTRIDE, CSUM>(e, cs, m_base, r0, cg, n, bias, csum);
      } else {
        if (xs == 0) epi_rows_fast<2, 0, RPT, EU, RS, CSTRIDE, CSUM>(e, cs, m_base, r0, cg, n, bias, csum);
        else if (xs == 2) epi_rows_fast<2, 2, RPT, EU, RS, CSTRIDE, CSUM>(e, cs, m_base, r0, cg, n, bias, csum);
        else epi_rows_fast<2, 4, RPT, EU, RS, CSTRIDE, CSUM>(e, cs, m_base, r0, cg, n, bias, csum);
      }
    } else {
      // edge tiles and unaligned operands: checked element access
#pragma unroll
      for (int q0 = 0; q0 < RPT; q0 += EU) {
        f32x4 v[EU];
        float a[EU][4], r[EU][4];
#pragma unroll
        for (int u = 0; u < EU; ++u) {
          const int rr = r0 + (q0 + u) * RS;
          v[u] = *(const f32x4 *)(cs + rr * CSTRIDE + cg * 4);
          epi_fetch(e, m_base + rr, n, false, a[u], r[u]);
        }
#pragma unroll
        for (int u = 0; u < EU; ++u) epi_apply(e, m_base + r0 + (q0 + u) * RS, n, v[u], bias, a[u], r[u], false);
      }
    }
    __syncthreads();
  }
  if (CSUM && e.colpart != nullptr) {
    // column sums of the tile: thread (cg, r0) holds rows r0, r0 + RS, ... of
    // every pass; the RS row groups are added in order through LDS
    float *red = (float *)smem;
    *(f32x4 *)(red + r0 * BN + cg * 4) = f32x4{csum[0], csum[1], csum[2], csum[3]};
    __syncthreads();
    if (tid < CG) {
      f32x4 t = *(const f32x4 *)(red + tid * 4);
#pragma unroll
      for (int r = 1; r < RS; ++r) t += *(const f32x4 *)(red + r * BN + tid * 4);
      *(f32x4 *)(e.colpart + (int64_t)(bm0 / BM) * p.N + bn0 + tid * 4) = t;
    }
  }
}

// acc[i][j] holds the 16x16 block (wm0 + 16i, wn0 + 16j) of the tile, lane l
// owning row l % 16, columns 4(l / 16) .. +3; the lane writes its four values
// to the staged tile.  CSUM: the kernel has the registers to also gather
// column sums for e.colpart (the 256x256 tiles do not: the four accumulators
// spill there).
template <int BM, int BN, int NT, int FM, int FN, int NPASS, int EUQ = 0, bool CSUM = false>
__device__ __forceinline__ void store_tile(const GemmParams &p, char *smem, f32x4 (&acc)[FM][FN], int tid, int wm0,
                                           int wn0, int bm0, int bn0, int split) {
  const int lane = tid & 63;
  constexpr int RP = BM / NPASS;
  constexpr int CSTRIDE = BN + 4;
  store_tile_staged<BM, BN, NT, NPASS, EUQ, CSUM>(p, smem, tid, bm0, bn0, split, [&](int pass, float *cs) {
    if (wm0 / RP == pass) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int row = wm0 - pass * RP + i * 16 + (lane & 15);
          const int col = wn0 + j * 16 + (lane >> 4) * 4;
          *(f32x4 *)(cs + row * CSTRIDE + col) = acc[i][j];
        }
    }
  });
}

// ---- the kernel ---------------------------------------------------------------
template <typename T, int LAYOUT, int BM, int BN, int BK, int WGM, int WGN>
__global__ __launch_bounds__(64 * WGM * WGN, (WGM * WGN >= 8 ? 1 : 2)) void gemm_kernel(GemmParams p) {
  constexpr int NT = 64 * WGM * WGN;
  constexpr int VEC = 16 / sizeof(T);
  constexpr int KCH = 4 * VEC;  // k covered by one 16-byte-per-lane fragment
  constexpr int STRIDE = BK;  // 128-byte rows, 16-byte chunks XOR-swizzled by row
  static_assert(BK * sizeof(T) == 128, "the LDS swizzle assumes 128-byte tile rows");
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int FM = WTM / 16, FN = WTN / 16;
  constexpr bool A_KC = (LAYOUT != GE_TN);
  constexpr bool B_KC = (LAYOUT == GE_NT);
  constexpr bool PING_PONG = (WGM == 2 && WGN * WGM == 8);
  static_assert(BK % KCH == 0, "BK must hold whole fragments");
  typedef typename Frag<T>::V V;

  // operand tiles (double-buffered); after the k loop the same memory stages
  // the FP32 accumulator tile for the epilogue
  constexpr int OPER_BYTES = 2 * (BM + BN) * STRIDE * (int)sizeof(T);
  constexpr int NPASS = BM >= 256 ? 2 : 1;  // row passes of the staged epilogue
  constexpr int RP = BM / NPASS;
  constexpr int CSTRIDE = BN + 4;  // floats per staged row (16-byte pad)
  constexpr int STAGE_BYTES = RP * CSTRIDE * 4;
  constexpr int SMEM_BYTES = OPER_BYTES > STAGE_BYTES ? OPER_BYTES : STAGE_BYTES;
  static_assert(SMEM_BYTES <= 160 * 1024, "LDS budget of one CU");
  static_assert(BM / WGM <= RP && RP % (BM / WGM) == 0, "a wave's rows must fall in one pass");
  __shared__ __attribute__((aligned(16))) char smem[SMEM_BYTES];
  T(*sA)[BM * STRIDE] = (T(*)[BM * STRIDE])smem;
  T(*sB)[BN * STRIDE] = (T(*)[BN * STRIDE])(smem + 2 * BM * STRIDE * sizeof(T));

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm0 = (wave / WGN) * WTM, wn0 = (wave % WGN) * WTN;

  int bm0, bn0, split;
  block_work(p, BM, BN, bm0, bn0, split);

  const int nk_total = (p.K + BK - 1) / BK;
  const int nk_full = p.K / BK;
  const int kt0 = split * p.ktiles_per_split;
  const int kt1 = min(nk_total, kt0 + p.ktiles_per_split);
  const bool interior = (bm0 + BM <= p.M) && (bn0 + BN <= p.N) && p.a_vec && p.b_vec && p.off32;

  const T *__restrict__ Ap = (const T *)p.A;
  const T *__restrict__ Bp = (const T *)p.B;

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // lane reads tile row (block + lane % 16) at 16-byte chunk 4c + lane / 16;
  // rows of a fragment start at multiples of 16, so the swizzle depends on
  // the lane only
  constexpr int NCH = BK / KCH;
  const int arow = (wm0 + (lane & 15)) * STRIDE;
  const int brow = (wn0 + (lane & 15)) * STRIDE;
  int koff[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) koff[c] = lds_chunk(lane & 15, 4 * c + (lane >> 4)) * VEC;

  // MFMAs over one LDS buffer.  Software-pipelined fragment reads: the k-tile
  // is a sequence of S = NC*FM A fragments (chunk c, row block i); the read of
  // fragment s+2 is issued before the MFMAs of fragment s, and the B fragments
  // of chunk c+1 halfway through chunk c, so each LDS read has MFMA work in
  // flight to hide its latency.  Scheduling barriers keep that order.
  auto compute = [&](int buf) {
    const T *a_s = sA[buf] + arow;
    const T *b_s = sB[buf] + brow;
    constexpr int NC = BK / KCH;
    constexpr int S = NC * FM;
    V af[S], bf[NC][FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) bf[0][j] = *(const V *)(b_s + j * 16 * STRIDE + koff[0]);
#pragma unroll
    for (int s = 0; s < 2 && s < S; ++s)
      af[s] = *(const V *)(a_s + (s % FM) * 16 * STRIDE + koff[s / FM]);
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int c = s / FM, i = s % FM;
      if (s + 2 < S) af[s + 2] = *(const V *)(a_s + ((s + 2) % FM) * 16 * STRIDE + koff[(s + 2) / FM]);
      if (i == FM / 2 && c + 1 < NC) {
#pragma unroll
        for (int j = 0; j < FN; ++j) bf[c + 1][j] = *(const V *)(b_s + j * 16 * STRIDE + koff[c + 1]);
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = Frag<T>::mma(bf[c][j], af[s], acc[i][j]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  if constexpr (PING_PONG) {
    // Two wave groups (rows 0..BM/2 and BM/2..BM of the tile; one wave of
    // each group per SIMD) alternate: while one group multiplies tile k the
    // other stores its half of tile k+1 (loaded one iteration earlier) into
    // the other LDS buffer and issues the global loads of its half of tile
    // k+2.  So every SIMD always has one wave issuing MFMAs, and each global
    // load has a whole iteration to arrive.
    const int g = wave / WGN;
    const int gt = tid % (NT / 2);
    Loader<T, A_KC, BM / 2, BK, NT / 2> la;
    Loader<T, B_KC, BN / 2, BK, NT / 2> lb;
    const int ar0 = bm0 + g * (BM / 2), br0 = bn0 + g * (BN / 2);
    auto load_half = [&](int kt) {
      if (interior && kt < nk_full) {
        la.load_fast(Ap, p.lda, ar0, kt * BK, gt);
        lb.load_fast(Bp, p.ldb, br0, kt * BK, gt);
      } else if (LAYOUT == GE_TN && p.clamp && kt < nk_full) {
        // (NN and NT instances of this kernel have no registers to spare)
        la.load_clamped(Ap, p.lda, ar0, p.M, kt * BK, gt);
        lb.load_clamped(Bp, p.ldb, br0, p.N, kt * BK, gt);
      } else {
        la.load_checked(Ap, p.lda, ar0, p.M, kt * BK, p.K, p.a_vec, gt);
        lb.load_checked(Bp, p.ldb, br0, p.N, kt * BK, p.K, p.b_vec, gt);
      }
    };
    auto store_half = [&](int buf) {
      la.store(sA[buf] + g * (BM / 2) * STRIDE, STRIDE, gt);
      lb.store(sB[buf] + g * (BN / 2) * STRIDE, STRIDE, gt);
    };
    auto memory_phase = [&](int kt, int buf) {
      if (kt + 1 < kt1) {
        store_half(buf ^ 1);
        if (kt + 2 < kt1) load_half(kt + 2);
      }
    };
    if (kt0 < kt1) {
      load_half(kt0);
      store_half(0);
      if (kt0 + 1 < kt1) load_half(kt0 + 1);
      __syncthreads();
    }
    for (int kt = kt0; kt < kt1; ++kt) {
      const int buf = (kt - kt0) & 1;
      if (g == 0) {
        __builtin_amdgcn_s_setprio(1);
        compute(buf);
        __builtin_amdgcn_s_setprio(0);
      } else {
        memory_phase(kt, buf);
      }
      __syncthreads();
      if (g == 1) {
        __builtin_amdgcn_s_setprio(1);
        compute(buf);
        __builtin_amdgcn_s_setprio(0);
      } else {
        memory_phase(kt, buf);
      }
      __syncthreads();
    }
  } else {
    Loader<T, A_KC, BM, BK, NT> la;
    Loader<T, B_KC, BN, BK, NT> lb;
    auto load_tile = [&](int kt) {
      if (interior && kt < nk_full) {
        la.load_fast(Ap, p.lda, bm0, kt * BK, tid);
        lb.load_fast(Bp, p.ldb, bn0, kt * BK, tid);
      } else if (p.clamp && kt < nk_full) {
        la.load_clamped(Ap, p.lda, bm0, p.M, kt * BK, tid);
        lb.load_clamped(Bp, p.ldb, bn0, p.N, kt * BK, tid);
      } else {
        la.load_checked(Ap, p.lda, bm0, p.M, kt * BK, p.K, p.a_vec, tid);
        lb.load_checked(Bp, p.ldb, bn0, p.N, kt * BK, p.K, p.b_vec, tid);
      }
    };
    if (kt0 < kt1) {
      load_tile(kt0);
      la.store(sA[0], STRIDE, tid);
      lb.store(sB[0], STRIDE, tid);
      __syncthreads();
    }
    for (int kt = kt0; kt < kt1; ++kt) {
      const int cur = (kt - kt0) & 1;
      const bool more = kt + 1 < kt1;
      if (more) load_tile(kt + 1);
      compute(cur);
      if (more) {
        la.store(sA[cur ^ 1], STRIDE, tid);
        lb.store(sB[cur ^ 1], STRIDE, tid);
      }
      __syncthreads();
    }
  }

  store_tile<BM, BN, NT, FM, FN, NPASS, 0, (BM < 256)>(p, smem, acc, tid, wm0, wn0, bm0, bn0, split);
}

// ---- 256 x BN tile on four waves (BN = 256 or 128) ------------------------------------
// One wave per SIMD, each owning a 128 x BN/2 quarter of the tile, so every A
// fragment read from LDS feeds BN/32 MFMAs (eight for BN = 256, where the
// 8-wave kernel's 64- or 128-wide quarters feed four).  A k-tile of BK is two k-chunks.  While the
// MFMAs of chunk 0 run, the wave reads the fragments of chunk 1, writes the
// next k-tile (fetched into registers one step earlier) into the other LDS
// buffer and fetches the k-tile after it; one barrier then separates those
// writes from the reads of the next k-tile, whose chunk-0 fragments are read
// while the MFMAs of chunk 1 run.  The steady-state step is straight-line
// code with scheduling groups that interleave memory instructions with the
// MFMAs, since a single wave per SIMD has no other wave to fill its gaps.
template <typename T, int LAYOUT, int BN>
__global__ __launch_bounds__(256, 1) void gemm_w4_kernel(GemmParams p) {
  constexpr int BM = 256, NT = 256;
  static_assert(BN == 256 || BN == 128, "tile width");
  constexpr int VEC = 16 / sizeof(T);
  constexpr int KCH = 4 * VEC;
  constexpr int BK = 128 / (int)sizeof(T);  // 128-byte LDS rows
  constexpr int STRIDE = BK;
  constexpr int NC = BK / KCH;
  static_assert(NC == 2, "two k-chunks per k-tile");
  constexpr int FM = 8, FN = BN / 32;
  constexpr bool A_KC = (LAYOUT != GE_TN);
  constexpr bool B_KC = (LAYOUT == GE_NT);
  constexpr int NPASS = 2;
  constexpr int OPER_BYTES = 2 * (BM + BN) * STRIDE * (int)sizeof(T);
  constexpr int STAGE_BYTES = (BM / NPASS) * (BN + 4) * 4;
  constexpr int SMEM_BYTES = OPER_BYTES > STAGE_BYTES ? OPER_BYTES : STAGE_BYTES;
  static_assert(SMEM_BYTES <= 160 * 1024, "LDS budget of one CU");
  typedef typename Frag<T>::V V;
  __shared__ __attribute__((aligned(16))) char smem[SMEM_BYTES];
  T(*sA)[BM * STRIDE] = (T(*)[BM * STRIDE])smem;
  T(*sB)[BN * STRIDE] = (T(*)[BN * STRIDE])(smem + 2 * BM * STRIDE * sizeof(T));

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm0 = (wave >> 1) * 128, wn0 = (wave & 1) * (BN / 2);
  int bm0, bn0, split;
  block_work(p, BM, BN, bm0, bn0, split);
  const int nk_total = (p.K + BK - 1) / BK;
  const int nk_full = p.K / BK;
  const int kt0 = split * p.ktiles_per_split;
  const int kt1 = min(nk_total, kt0 + p.ktiles_per_split);
  const bool interior = (bm0 + BM <= p.M) && (bn0 + BN <= p.N) && p.a_vec && p.b_vec && p.off32;
  const T *__restrict__ Ap = (const T *)p.A;
  const T *__restrict__ Bp = (const T *)p.B;

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  int koff[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) koff[c] = lds_chunk(lane & 15, 4 * c + (lane >> 4)) * VEC;
  const int arow = (wm0 + (lane & 15)) * STRIDE;
  const int brow = (wn0 + (lane & 15)) * STRIDE;

  // Operands are staged one k-chunk (KCH) at a time: chunk c of k-tile t
  // occupies the 64-byte half c of the rows of LDS buffer t % 2, so the two
  // buffers form a ring of four chunk slots.  Phase q multiplies chunk q,
  // reads the fragments of chunk q+1, writes chunk q+2 (fetched two phases
  // earlier into register set q % 2) and fetches chunk q+4 into that set; a
  // barrier ends every phase.  Chunk q+2's slot last held chunk q-2, whose
  // fragments were read in phase q-3, and chunk q+1 was written in phase q-1,
  // so one barrier per phase orders every LDS write against its readers, and
  // each phase writes half a k-tile instead of one phase writing all of it.
  typedef Loader<T, A_KC, BM, KCH, NT> LA;
  typedef Loader<T, B_KC, BN, KCH, NT> LB;
  LA la0, la1;
  LB lb0, lb1;
  constexpr int QH = KCH * (int)sizeof(T) / 16;  // 16-byte chunks per k-chunk (4)
  auto ld_any = [&](LA &la, LB &lb, int q) {  // chunk q = 2 * k-tile + c
    const int k0 = q * KCH;
    if (interior && (q >> 1) < nk_full) {
      la.load_fast(Ap, p.lda, bm0, k0, tid);
      lb.load_fast(Bp, p.ldb, bn0, k0, tid);
    } else if (p.clamp && (q >> 1) < nk_full) {
      la.load_clamped(Ap, p.lda, bm0, p.M, k0, tid);
      lb.load_clamped(Bp, p.ldb, bn0, p.N, k0, tid);
    } else {
      la.load_checked(Ap, p.lda, bm0, p.M, k0, p.K, p.a_vec, tid);
      lb.load_checked(Bp, p.ldb, bn0, p.N, k0, p.K, p.b_vec, tid);
    }
  };
  auto st_all = [&](const LA &la, const LB &lb, int q) {
#pragma unroll
    for (int i = 0; i < LA::NSTORE; ++i) la.store_piece(sA[(q >> 1) & 1], STRIDE, tid, i, (q & 1) * QH);
#pragma unroll
    for (int i = 0; i < LB::NSTORE; ++i) lb.store_piece(sB[(q >> 1) & 1], STRIDE, tid, i, (q & 1) * QH);
  };
  // fa: A fragments of the chunk being multiplied; row i's fragment of the
  // next chunk replaces it as soon as row i's MFMAs are issued.  fb0 / fb1:
  // B fragments of even / odd chunks.
  V fa[FM], fb0[FN], fb1[FN];
  auto read_a = [&](int q, int i) {
    fa[i] = *(const V *)(sA[(q >> 1) & 1] + arow + i * 16 * STRIDE + koff[q & 1]);
  };
  auto read_b = [&](int q, V(&fb)[FN]) {
#pragma unroll
    for (int j = 0; j < FN; ++j) fb[j] = *(const V *)(sB[(q >> 1) & 1] + brow + j * 16 * STRIDE + koff[q & 1]);
  };
  // generic phase: MFMAs of chunk q with fb, then (when there is one) the
  // fragments of chunk q+1
  auto phase_any = [&](V(&fb)[FN], V(&fb_next)[FN], int q, bool next) {
    if (next) read_b(q + 1, fb_next);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int j = 0; j < FN; ++j) FragA<T>::mma(fb[j], fa[i], acc[i][j]);
      if (next) read_a(q + 1, i);
    }
  };
  // steady phase q: every MFMA is its own scheduling region carrying at most
  // one memory instruction -- B reads of chunk q+1 in row 0, then the loads
  // of chunk q+3 into the other register set (written in phase q-1), one per
  // slot from slot 0 (A first), then the LDS writes of chunk q+2 spread over
  // the second part of the phase, and each row's A read right after its last
  // MFMA.  A load thus precedes its LDS write by more than one phase.
  constexpr int NSLOT = FM * FN;
  constexpr int NLD = LA::NLOAD + LB::NLOAD, NST = LA::NSTORE + LB::NSTORE;
  constexpr int W0 = NSLOT * 3 / 8;
  constexpr int WS = (NSLOT - W0) / NST > 0 ? (NSLOT - W0) / NST : 1;
  static_assert(NLD <= W0 && W0 + WS * (NST - 1) < NSLOT, "memory slots must fit the phase");
  auto phase_fast = [&](V(&fb)[FN], V(&fb_next)[FN], const LA &law, const LB &lbw, LA &lal, LB &lbl, int q) {
    const int wb = ((q + 2) >> 1) & 1, wq = ((q + 2) & 1) * QH;
    const int k3 = (q + 3) * KCH;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        FragA<T>::mma(fb[j], fa[i], acc[i][j]);
        const int slot = i * FN + j;
        if (i == 0) fb_next[j] = *(const V *)(sB[((q + 1) >> 1) & 1] + brow + j * 16 * STRIDE + koff[(q + 1) & 1]);
        if (slot < LA::NLOAD) lal.load_piece(Ap, p.lda, bm0, k3, tid, slot);
        else if (slot < NLD) lbl.load_piece(Bp, p.ldb, bn0, k3, tid, slot - LA::NLOAD);
        if (slot >= W0 && (slot - W0) % WS == 0) {
          const int w = (slot - W0) / WS;
          if (w < LA::NSTORE) law.store_piece(sA[wb], STRIDE, tid, w, wq);
          else if (w < NST) lbw.store_piece(sB[wb], STRIDE, tid, w - LA::NSTORE, wq);
        }
        if (j == FN - 1) read_a(q + 1, i);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  const int q0 = 2 * kt0, q1 = 2 * kt1;  // chunk range of this block
  int q = q0;
  // steady state: chunks q+4 and q+5 exist and are full interior ones.  Its
  // prologue issues the same unconditional loads as a loop step, so the
  // loop entry carries the same outstanding-load pattern as the back edge
  // and the compiler's waits before the LDS writes stay partial.
  const int q_end = 2 * min(kt1, nk_full) - 5;
  if (interior && q0 + 1 < q_end) {
    la0.load_fast(Ap, p.lda, bm0, q0 * KCH, tid);
    lb0.load_fast(Bp, p.ldb, bn0, q0 * KCH, tid);
    la1.load_fast(Ap, p.lda, bm0, (q0 + 1) * KCH, tid);
    lb1.load_fast(Bp, p.ldb, bn0, (q0 + 1) * KCH, tid);
    st_all(la0, lb0, q0);
    la0.load_fast(Ap, p.lda, bm0, (q0 + 2) * KCH, tid);
    lb0.load_fast(Bp, p.ldb, bn0, (q0 + 2) * KCH, tid);
    st_all(la1, lb1, q0 + 1);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < FM; ++i) read_a(q0, i);
    read_b(q0, fb0);
    for (; q < q_end; q += 2) {
      phase_fast(fb0, fb1, la0, lb0, la1, lb1, q);
      __syncthreads();
      phase_fast(fb1, fb0, la1, lb1, la0, lb0, q + 1);
      __syncthreads();
    }
    // the steady loop leaves chunk q+2 in set 0; the remaining phases also
    // expect chunk q+3 in set 1
    if (q + 3 < q1) ld_any(la1, lb1, q + 3);
  } else if (q0 < q1) {
    ld_any(la0, lb0, q0);
    st_all(la0, lb0, q0);
    ld_any(la1, lb1, q0 + 1);
    st_all(la1, lb1, q0 + 1);
    if (q0 + 2 < q1) ld_any(la0, lb0, q0 + 2);
    if (q0 + 3 < q1) ld_any(la1, lb1, q0 + 3);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < FM; ++i) read_a(q0, i);
    read_b(q0, fb0);
  }
  // remaining phases (edge tiles, the last chunks, a partial k-tile)
  for (; q < q1; q += 2) {
    phase_any(fb0, fb1, q, q + 1 < q1);
    if (q + 2 < q1) {
      st_all(la0, lb0, q + 2);
      if (q + 4 < q1) ld_any(la0, lb0, q + 4);
    }
    __syncthreads();
    phase_any(fb1, fb0, q + 1, q + 2 < q1);
    if (q + 3 < q1) {
      st_all(la1, lb1, q + 3);
      if (q + 5 < q1) ld_any(la1, lb1, q + 5);
    }
    __syncthreads();
  }
  store_tile<BM, BN, NT, FM, FN, NPASS, 4, (BN < 256)>(p, smem, acc, tid, wm0, wn0, bm0, bn0, split);
}

// ---- 256 x 256 tile on eight waves, 32x32x16 MFMA, LDS filled by DMA ------------------
// Measured on this GPU: a 16x16x32 MFMA issued back to back from one wave
// per SIMD reaches about half the matrix rate (about 25 cycles each), the
// 32x32x16 form about nine tenths; and one wave per SIMD pulls about half the
// LDS bandwidth that two waves do.  So this kernel runs two waves per SIMD,
// each owning a 128 x 64 block of the tile (4 x 2 blocks of 32 x 32, 128
// accumulator registers), on the 32x32x16 MFMA.
//
// Operands move from memory to LDS without registers: one buffer load with
// the LDS flag moves 16 bytes per lane into 1 KB of consecutive LDS, so the
// tile layout is chosen through the global address each lane loads (the
// buffer form, not the flat one, so the compiler's LDS-read counters stay
// exact).  k-tiles are 64 wide (whole 128-byte lines of k-contiguous rows),
// in two LDS stages of 64 KB: the loads of stage t+1 are issued right after
// the barrier that opens stage t, so they have one stage of MFMA work to land.
//   k-contiguous operand: 256 rows x 128 bytes; 16-byte chunk c of row r is
//     stored at chunk c ^ ((r >> 1) & 7) (a 16-lane fragment read -- 16 rows,
//     one chunk -- hits 16 distinct bank groups).
//   m/n-contiguous operand: 64 k-rows x 512 bytes; 32-byte slot s of k-row k
//     is stored at slot s ^ 2 (k & 3).  Its fragments are read with the
//     transposing LDS read (ds_read_b64_tr_b16): within each 16-lane group,
//     lane j receives element j & 3 of the 4 elements read by lanes
//     (j >> 2) + 4 r, r = 0..3, so lanes reading 4 k-rows x 16 consecutive m
//     hand each lane 4 k-values of one m (two reads make the 8 of a fragment).
// Within a stage the fragment reads of the next 16-wide k block are spread
// between the MFMAs of the current one.
template <typename T> struct Mfma32;
template <> struct Mfma32<half_t> {
  typedef f16x8 V;
  static __device__ __forceinline__ f32x16 mma(V a, V b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mfma32<bf16_t> {
  typedef bf16x8 V;
  static __device__ __forceinline__ f32x16 mma(V a, V b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

constexpr int X8_BK = 64;  // k per stage
template <bool B> struct BoolC { static constexpr bool value = B; };

// LDS bytes of one stage (A tile 256 x 64, B tile BN x 64) and of the kernel
// (two stages, or the FP32 staging of half the tile for the epilogue)
template <int BN> constexpr int x8_stage() { return (256 + BN) * X8_BK * 2; }
// stages in the LDS ring: three of 48 KB for 256x128 tiles, two of 64 KB for
// 256x256; NT (both operands k-contiguous) measured faster on two
template <int BN, int LAYOUT> constexpr int x8_nstage() { return BN == 128 && LAYOUT != GE_NT ? 3 : 2; }
template <int BN, int LAYOUT> constexpr int x8_smem() {
  return x8_nstage<BN, LAYOUT>() * x8_stage<BN>() > 128 * (BN + 4) * 4 ? x8_nstage<BN, LAYOUT>() * x8_stage<BN>()
                                                                       : 128 * (BN + 4) * 4;
}

__device__ __forceinline__ int x8_kc_swz(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int x8_mc_swz(int k) { return 2 * (k & 3); }

// Per-lane byte offsets of the two instruction parities of one operand tile.
// A k-contiguous tile: instruction ins covers rows 8 ins .. +7.  An
// m/n-contiguous tile W wide: its k-rows are 2 W bytes, so instruction ins
// covers k-rows (1024 / 2W) ins .. + 1024 / 2W - 1 (two k-rows at W = 256,
// four at W = 128).  The rest of the address is uniform and goes in the
// scalar offset.  wv (a multiple of 8) is how many of the tile's W rows or
// columns lie inside the operand: on an edge tile an m/n-contiguous lane past
// it reads the last valid 8 columns instead (those outputs are never stored).
template <bool KC, int W>
__device__ __forceinline__ void x8_lane_offsets(int64_t ld, int es, int lane, int wv, uint32_t (&vo)[2]) {
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    if constexpr (KC) {
      const int row = par * 8 + (lane >> 3);
      const int c = (lane & 7) ^ x8_kc_swz(row);
      vo[par] = (uint32_t)(((lane >> 3) * ld + 8 * c) * es);
    } else if constexpr (W == 256) {
      const int k = par * 2 + (lane >> 5);
      const int sl = ((lane & 31) >> 1) ^ x8_mc_swz(k);
      const int col = min(16 * sl + 8 * (lane & 1), wv - 8);
      vo[par] = (uint32_t)(((lane >> 5) * ld + col) * es);
    } else {
      // four k-rows per instruction: k & 3 = lane >> 4 for every instruction
      const int kl = lane >> 4;
      const int sl = ((lane & 15) >> 1) ^ x8_mc_swz(kl);
      const int col = min(16 * sl + 8 * (lane & 1), wv - 8);
      vo[par] = (uint32_t)((kl * ld + col) * es);
    }
  }
}

// The uniform part of instruction ins's address at k-tile offset k0; on an
// edge tile the rows of a k-contiguous operand past wv are read from its last
// eight valid rows instead (uniform, as wv is a multiple of 8).
template <bool KC, int W>
__device__ __forceinline__ uint32_t x8_soff(int64_t ld, int es, int k0, int ins, int wv) {
  constexpr int KPI = 1024 / (2 * W);  // k-rows per instruction of an m/n-contiguous tile
  const int r0 = ins * 8 < wv - 8 ? ins * 8 : wv - 8;
  return KC ? (uint32_t)(((int64_t)r0 * ld + k0) * es) : (uint32_t)((int64_t)(k0 + ins * KPI) * ld * es);
}

// The last, partial k-tile (K % 64 != 0) goes through ordinary loads and LDS
// stores, zero where the lane's k (its 8-wide chunk of a k-contiguous row,
// or its k-row) is at or past K, so the padded products add exact zeros; the
// LDS slot is the lane's, as the direct load writes it.  This gives the
// lane's byte offset from the tile base and sets ok = (k < K); a lane at or
// past K gets an in-bounds offset of the same tile (chunk 0 of its row, or
// k-row K - 1 of its columns), so every load is issued before any is used.
template <bool KC, int W>
__device__ __forceinline__ uint32_t x8_tail_off(int64_t ld, int es, int k0, int K, int ins, int wv,
                                                const uint32_t (&vo)[2], int lane, bool &ok) {
  constexpr int KPI = 1024 / (2 * W);
  const uint32_t off = vo[ins & 1] + x8_soff<KC, W>(ld, es, k0, ins, wv);
  if constexpr (KC) {
    const int c = (lane & 7) ^ x8_kc_swz((ins & 1) * 8 + (lane >> 3));
    ok = k0 + 8 * c < K;
    return ok ? off : off - (uint32_t)(8 * c * es);
  } else {
    const int k = k0 + ins * KPI + (W == 256 ? (lane >> 5) : (lane >> 4));
    ok = k < K;
    return ok ? off : off - (uint32_t)((int64_t)(k - (K - 1)) * ld * es);
  }
}

// fragment of the 32x32x16 MFMA: rows r .. r+31 of the operand, k block kb
// (16 k) of the stage; lane l gets row r + l % 32, k = 16 kb + 8 (l / 32) .. +7
template <typename V, bool KC, int W>
__device__ __forceinline__ V x8_frag(const char *tile, int r, int kb, int lane) {
  if constexpr (KC) {
    const int row = r + (lane & 31);
    const int c = (2 * kb + (lane >> 5)) ^ x8_kc_swz(row);
    return __builtin_bit_cast(V, *(const lds_u32x4 *)(tile + row * 128 + c * 16));
  } else {
    constexpr int ROWB = 2 * W;  // bytes of one k-row
    const int G = lane >> 4, j = lane & 15;
    const int k = 16 * kb + 8 * (G >> 1) + (j >> 2);
    const int slot = (r >> 4) + (G & 1);
    const char *p0 = tile + k * ROWB + ((slot ^ x8_mc_swz(k)) * 32) + 8 * (j & 3);
    const char *p1 = tile + (k + 4) * ROWB + ((slot ^ x8_mc_swz(k + 4)) * 32) + 8 * (j & 3);
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p0);
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p1);
    return __builtin_bit_cast(V, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  }
}

// BN = 256: wave tile 128 x 64 (waves 2 x 4); BN = 128: 64 x 64 (waves 4 x 2),
// which fills the 256 CUs at 4096 x 2048 and carries the dgrad's column sums
template <typename T, int LAYOUT, int BN>
__global__ __launch_bounds__(512, 1) void gemm_x8_kernel(GemmParams p) {
  constexpr int BM = 256, NT = 512;
  constexpr int WTM = BN == 256 ? 128 : 64;
  constexpr int FA = WTM / 32;  // A fragments (32-row blocks) per wave
  constexpr bool A_KC = (LAYOUT != GE_TN);
  constexpr bool B_KC = (LAYOUT == GE_NT);
  constexpr int TILE_A = BM * X8_BK * 2;
  constexpr int STAGE = x8_stage<BN>();
  constexpr int NS = x8_nstage<BN, LAYOUT>();
  constexpr int BPW = BN / 64;  // B tile load instructions per wave
  typedef typename Mfma32<T>::V V;
  __shared__ __attribute__((aligned(1024))) char smem[x8_smem<BN, LAYOUT>()];
  // the wave index is uniform; saying so keeps the loads' scalar offsets in
  // SGPRs (otherwise each direct load sits in a loop over distinct values)
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm0 = BN == 256 ? (wave >> 2) * 128 : (wave >> 1) * 64;
  const int wn0 = BN == 256 ? (wave & 3) * 64 : (wave & 1) * 64;
  int bm0, bn0, split;
  block_work(p, BM, BN, bm0, bn0, split);
  const int nk = (p.K + X8_BK - 1) / X8_BK;
  const bool ktail = (p.K % X8_BK) != 0;  // the last k-tile is partial
  const int mv = min(BM, p.M - bm0), nv = min(BN, p.N - bn0);  // valid rows / columns of the tile
  const int kt0 = split * p.ktiles_per_split;
  const int kt1 = min(nk, kt0 + p.ktiles_per_split);
  constexpr int es = (int)sizeof(T);
  // buffer resources based at this tile's rows / columns (offsets stay far below 2^31)
  const T *Ab = (const T *)p.A + (A_KC ? (int64_t)bm0 * p.lda : (int64_t)bm0);
  const T *Bb = (const T *)p.B + (B_KC ? (int64_t)bn0 * p.ldb : (int64_t)bn0);
  const u32x4 ra = raw_buffer_rsrc(Ab), rb = raw_buffer_rsrc(Bb);
  uint32_t voa[2], vob[2];
  x8_lane_offsets<A_KC, BM>(p.lda, es, lane, mv, voa);
  x8_lane_offsets<B_KC, BN>(p.ldb, es, lane, nv, vob);
  // the loads' LDS and scalar addresses at k-tile 0, and their step per k-tile
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void *)smem);
  uint32_t soa[4], sob[BPW];
#pragma unroll
  for (int u = 0; u < 4; ++u) soa[u] = x8_soff<A_KC, BM>(p.lda, es, 0, wave * 4 + u, mv);
#pragma unroll
  for (int u = 0; u < BPW; ++u) sob[u] = x8_soff<B_KC, BN>(p.ldb, es, 0, wave * BPW + u, nv);
  const uint32_t dka = (uint32_t)(A_KC ? X8_BK * es : (int64_t)X8_BK * p.lda * es);
  const uint32_t dkb = (uint32_t)(B_KC ? X8_BK * es : (int64_t)X8_BK * p.ldb * es);
  // a stage: 32 instructions for the A tile (4 per wave), BN / 8 for the B tile
  auto issue = [&](int t) {
    char *st = smem + (t % NS) * STAGE;
    if (ktail && t == nk - 1) {
      u32x4 va[4], vb[BPW];
      bool oa[4], ob[BPW];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        va[u] = *(const u32x4 *)((const char *)Ab +
                                 x8_tail_off<A_KC, BM>(p.lda, es, t * X8_BK, p.K, wave * 4 + u, mv, voa, lane, oa[u]));
#pragma unroll
      for (int u = 0; u < BPW; ++u)
        vb[u] = *(const u32x4 *)((const char *)Bb +
                                 x8_tail_off<B_KC, BN>(p.ldb, es, t * X8_BK, p.K, wave * BPW + u, nv, vob, lane, ob[u]));
      const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int u = 0; u < 4; ++u) *(lds_u32x4 *)(st + (wave * 4 + u) * 1024 + lane * 16) = oa[u] ? va[u] : zero;
#pragma unroll
      for (int u = 0; u < BPW; ++u)
        *(lds_u32x4 *)(st + TILE_A + (wave * BPW + u) * 1024 + lane * 16) = ob[u] ? vb[u] : zero;
      return;
    }
    const uint32_t sl = lds0 + (uint32_t)((t % NS) * STAGE);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int ins = wave * 4 + u;
      lds_dma16_at(ra, voa[ins & 1], soa[u] + (uint32_t)t * dka, sl + ins * 1024);
    }
#pragma unroll
    for (int u = 0; u < BPW; ++u) {
      const int ins = wave * BPW + u;
      lds_dma16_at(rb, vob[ins & 1], sob[u] + (uint32_t)t * dkb, sl + TILE_A + ins * 1024);
    }
  };

  f32x16 acc[FA][2];
#pragma unroll
  for (int i = 0; i < FA; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  V fa0[FA], fb0[2], fa1[FA], fb1[2];
  auto rd = [&](const char *st, int kb, V(&fa)[FA], V(&fb)[2]) {
#pragma unroll
    for (int j = 0; j < 2; ++j) fb[j] = x8_frag<V, B_KC, BN>(st + TILE_A, wn0 + 32 * j, kb, lane);
#pragma unroll
    for (int i = 0; i < FA; ++i) fa[i] = x8_frag<V, A_KC, BM>(st, wm0 + 32 * i, kb, lane);
  };
  // the B fragment goes first, so lane l owns C[m = l % 32][n = 8 (e / 4) + 4 (l / 32) + e % 4]
  auto mma = [&](const V(&fa)[FA], const V(&fb)[2]) {
#pragma unroll
    for (int i = 0; i < FA; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = Mfma32<T>::mma(fb[j], fa[i], acc[i][j]);
  };
  constexpr int NM = 2 * FA;                                // MFMAs per k block
  constexpr int NR = (A_KC ? FA : 2 * FA) + (B_KC ? 2 : 4);  // LDS read instructions per k block
  auto phase = [&](const char *st, int kb, V(&fan)[FA], V(&fbn)[2], const V(&fac)[FA], const V(&fbc)[2],
                   bool do_mma) {
    rd(st, kb, fan, fbn);
    if (do_mma) {
      mma(fac, fbc);
#pragma unroll
      for (int u = 0; u < NM; ++u) {
        __builtin_amdgcn_sched_group_barrier(0x100, (NR + NM - 1) / NM, 0);  // LDS reads
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                 // one MFMA
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // one k-step; `first` (a compile-time flag, so the steady-state loop has no
  // branch between its LDS reads and MFMAs) skips the previous step's MFMAs
  auto step = [&](int t, auto first) {
    // stage t's loads and the previous stage's LDS reads are done; in a
    // three-stage ring stage t + 1's loads (the wave's last 4 + BPW
    // instructions) may stay in flight
    if (NS == 3 && t + 1 < kt1) __builtin_amdgcn_s_waitcnt(0x0070 | (4 + BPW));
    else __builtin_amdgcn_s_waitcnt(0x0070);
    // a bare barrier: the waits above are the ordering this needs, and a
    // fenced barrier would also wait for the loads still in flight
    asm volatile("s_barrier" ::: "memory");
    if (t + NS - 1 < kt1) issue(t + NS - 1);
    __builtin_amdgcn_sched_barrier(0);
    const char *st = smem + (t % NS) * STAGE;
    phase(st, 0, fa0, fb0, fa1, fb1, !decltype(first)::value);  // with the previous stage's last MFMAs
    phase(st, 1, fa1, fb1, fa0, fb0, true);
    phase(st, 2, fa0, fb0, fa1, fb1, true);
    phase(st, 3, fa1, fb1, fa0, fb0, true);
  };
  if (kt0 < kt1) issue(kt0);
  if (NS == 3 && kt0 + 1 < kt1) issue(kt0 + 1);
  if (kt0 < kt1) step(kt0, BoolC<true>{});
  for (int t = kt0 + 1; t < kt1; ++t) step(t, BoolC<false>{});
  if (kt0 < kt1) mma(fa1, fb1);
  __builtin_amdgcn_s_waitcnt(0x0070);
  __syncthreads();
  // the staged epilogue in two passes of 128 rows: waves 0-3 hold rows 0..127
  store_tile_staged<BM, BN, NT, 2, 0, (BN < 256)>(p, smem, tid, bm0, bn0, split, [&](int pass, float *cs) {
    if ((wave >> 2) == pass) {
#pragma unroll
      for (int i = 0; i < FA; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int r = (wm0 - 128 * pass) + 32 * i + (lane & 31);
            const int c = wn0 + 32 * j + 8 * q + 4 * (lane >> 5);
            const f32x16 &v = acc[i][j];
            *(f32x4 *)(cs + r * (BN + 4) + c) = f32x4{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
          }
    }
  });
}

// ---- launch plan and per-type launchers ---------------------------------------
struct Plan {
  int x8;      // the eight-wave kernel (k-tiles of 64): 1 for 256x256 tiles, 2 for 256x128
  int bm, bn;  // tile: 256x256, 256x128, 128x128, 64x64, or 128x16 for N <= 16
  int BK;
  int tiles_m, tiles_n, nk, splits, kps;
};

template <typename T, int LAYOUT>
void launch_t(const Plan &pl, const GemmParams &gp, hipStream_t s) {
  dim3 grid(pl.tiles_m * pl.tiles_n, 1, pl.splits);
  constexpr int BK = sizeof(T) == 4 ? 32 : 64;
  // 256x256: measured on 4096^3, the four-wave kernel is faster when an
  // operand is transposed on its way into LDS (NN, TN), the eight-wave
  // ping-pong kernel when both are k-contiguous (NT) and for short k ranges
  // (split-K blocks of fewer than 16 k-tiles)
  if constexpr (sizeof(T) == 2) {
    if (pl.x8 == 1) {
      hipLaunchKernelGGL((gemm_x8_kernel<T, LAYOUT, 256>), grid, dim3(512), 0, s, gp);
      return;
    }
    if (pl.x8 == 2) {
      hipLaunchKernelGGL((gemm_x8_kernel<T, LAYOUT, 128>), grid, dim3(512), 0, s, gp);
      return;
    }
  }
  if (pl.bm == 256 && pl.bn == 128)
    hipLaunchKernelGGL((gemm_w4_kernel<T, LAYOUT, 128>), grid, dim3(256), 0, s, gp);
  else if (pl.bm == 256 && (LAYOUT == GE_NT || pl.kps < 16))
    hipLaunchKernelGGL((gemm_kernel<T, LAYOUT, 256, 256, BK, 2, 4>), grid, dim3(512), 0, s, gp);
  else if (pl.bm == 256)
    hipLaunchKernelGGL((gemm_w4_kernel<T, LAYOUT, 256>), grid, dim3(256), 0, s, gp);
  else if (pl.bn == 16)
    hipLaunchKernelGGL((gemm_kernel<T, LAYOUT, 128, 16, BK, 4, 1>), grid, dim3(256), 0, s, gp);
  else if (pl.bm == 128)
    hipLaunchKernelGGL((gemm_kernel<T, LAYOUT, 128, 128, BK, 2, 2>), grid, dim3(256), 0, s, gp);
  else
    hipLaunchKernelGGL((gemm_kernel<T, LAYOUT, 64, 64, BK, 2, 2>), grid, dim3(256), 0, s, gp);
}

template <typename T>
void launch_layout(int layout, const Plan &pl, const GemmParams &gp, hipStream_t s) {
  if (layout == GE_NN) launch_t<T, GE_NN>(pl, gp, s);
  else if (layout == GE_NT) launch_t<T, GE_NT>(pl, gp, s);
  else launch_t<T, GE_TN>(pl, gp, s);
}

// one translation unit per operand type instantiates the kernels
void gemm_dispatch_f16(int layout, const Plan &pl, const GemmParams &gp, hipStream_t s);
void gemm_dispatch_bf16(int layout, const Plan &pl, const GemmParams &gp, hipStream_t s);
void gemm_dispatch_f32(int layout, const Plan &pl, const GemmParams &gp, hipStream_t s);

}  // namespace ge
