// Shared device/host helpers of the gfx950 GEMM-epilogue library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_epilogue.h"

namespace ge {

typedef _Float16 half_t;
typedef __bf16 bf16_t;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef half_t f16x8 __attribute__((ext_vector_type(8)));
typedef bf16_t bf16x8 __attribute__((ext_vector_type(8)));
typedef half_t f16x4 __attribute__((ext_vector_type(4)));
typedef bf16_t bf16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

// ---- loads from global memory straight into LDS -------------------------------
// Buffer resource of a raw 32-bit buffer at base: no stride, the largest record
// count and the data-format word of a raw buffer.
__device__ __forceinline__ u32x4 raw_buffer_rsrc(const void *base) {
  const uint64_t b = (uint64_t)base;
  return u32x4{(uint32_t)b, (uint32_t)(b >> 32), 0x7fffffffu, 0x00020000u};
}

// 16 bytes per lane from rs + voff (per lane) + soff (uniform) into LDS, lane
// l's bytes at dst + 16 l (dst uniform).  Written as inline asm because the
// compiler, seeing a load that writes LDS, waits for every such load before
// the next LDS read, so a prefetch could never overlap the work on the data
// already there; callers order these loads with explicit s_waitcnt vmcnt and
// barriers.  The asm has no outputs.  The compiler does not look inside it
// for hazards, so it opens with five wait states: the most a buffer load
// needs after a VALU write of an SGPR it reads (the readfirstlane below) and
// after the SALU write of M0.
// The same with the LDS byte address given as a 32-bit value (uniform).
__device__ __forceinline__ void lds_dma16_at(const u32x4 &rs, uint32_t voff, uint32_t soff, uint32_t lds_addr) {
  const u32x4 r = {(uint32_t)__builtin_amdgcn_readfirstlane(rs[0]), (uint32_t)__builtin_amdgcn_readfirstlane(rs[1]),
                   (uint32_t)__builtin_amdgcn_readfirstlane(rs[2]), (uint32_t)__builtin_amdgcn_readfirstlane(rs[3])};
  const uint32_t so = __builtin_amdgcn_readfirstlane(soff);
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_addr);
  asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff), "s"(r), "s"(so), "{m0}"(m0v)
               : "memory");
}

__device__ __forceinline__ void lds_dma16(const u32x4 &rs, uint32_t voff, uint32_t soff, char *dst) {
  // all uniform; readfirstlane keeps them in SGPRs where the compiler would
  // otherwise leave a copy in VGPRs
  const u32x4 r = {(uint32_t)__builtin_amdgcn_readfirstlane(rs[0]), (uint32_t)__builtin_amdgcn_readfirstlane(rs[1]),
                   (uint32_t)__builtin_amdgcn_readfirstlane(rs[2]), (uint32_t)__builtin_amdgcn_readfirstlane(rs[3])};
  const uint32_t so = __builtin_amdgcn_readfirstlane(soff);
  const uint32_t m0v = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void *)dst);
  asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff), "s"(r), "s"(so), "{m0}"(m0v)
               : "memory");
}

inline int dtype_size(int t) { return t == GE_F32 ? 4 : 2; }
inline bool dtype_ok(int t) { return t == GE_F32 || t == GE_F16 || t == GE_BF16; }

// ---- conversions (hardware conversions round to nearest even) -------------
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(half_t x) { return (float)x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ half_t from_f32<half_t>(float x) { return (half_t)x; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) { return (bf16_t)x; }

// element of a runtime-typed array
__device__ __forceinline__ float load_any(const void *p, int64_t i, int t) {
  if (t == GE_F32) return ((const float *)p)[i];
  if (t == GE_F16) return (float)((const half_t *)p)[i];
  return (float)((const bf16_t *)p)[i];
}
__device__ __forceinline__ void store_any(void *p, int64_t i, int t, float v) {
  if (t == GE_F32) ((float *)p)[i] = v;
  else if (t == GE_F16) ((half_t *)p)[i] = (half_t)v;
  else ((bf16_t *)p)[i] = (bf16_t)v;
}

// four consecutive elements; `vec` says the address is aligned for one access
__device__ __forceinline__ void load4_any(const void *p, int64_t i, int t, bool vec, float v[4]) {
  if (vec) {
    if (t == GE_F32) {
      f32x4 x = *(const f32x4 *)((const float *)p + i);
      v[0] = x[0]; v[1] = x[1]; v[2] = x[2]; v[3] = x[3];
    } else if (t == GE_F16) {
      f16x4 x = *(const f16x4 *)((const half_t *)p + i);
      v[0] = (float)x[0]; v[1] = (float)x[1]; v[2] = (float)x[2]; v[3] = (float)x[3];
    } else {
      bf16x4 x = *(const bf16x4 *)((const bf16_t *)p + i);
      v[0] = (float)x[0]; v[1] = (float)x[1]; v[2] = (float)x[2]; v[3] = (float)x[3];
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = load_any(p, i + j, t);
  }
}
__device__ __forceinline__ void store4_any(void *p, int64_t i, int t, bool vec, const float v[4]) {
  if (vec) {
    if (t == GE_F32) {
      f32x4 x = {v[0], v[1], v[2], v[3]};
      *(f32x4 *)((float *)p + i) = x;
    } else if (t == GE_F16) {
      f16x4 x = {(half_t)v[0], (half_t)v[1], (half_t)v[2], (half_t)v[3]};
      *(f16x4 *)((half_t *)p + i) = x;
    } else {
      bf16x4 x = {(bf16_t)v[0], (bf16_t)v[1], (bf16_t)v[2], (bf16_t)v[3]};
      *(bf16x4 *)((bf16_t *)p + i) = x;
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) store_any(p, i + j, t, v[j]);
  }
}

// wave64 reductions (butterfly over all 64 lanes)
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// ---- host side -------------------------------------------------------------
void set_error(const char *fmt, ...);
int launch_status(const char *what);  // GE_OK or GE_E_LAUNCH after hipGetLastError

// aligned for a `bytes`-wide vector access at every row start
inline bool vec_aligned(const void *p, int64_t ld, int esize, int bytes) {
  return p != nullptr && ((uintptr_t)p % bytes) == 0 && ((ld * esize) % bytes) == 0;
}

// internal launchers (validated arguments)
// colpart (optional, 16-byte aligned): per-tile-row FP32 column sums of the
// stored C, [gemm_colsum_rows(a) x N]; allowed when gemm_colsum_rows(a) > 0
// deferred (optional): a split-K GEMM whose epilogue is alpha times the sum
// into row-major FP32 C skips its finishing pass, leaves splits x M x N
// partials in the workspace (split-major) and sets *deferred to the split
// count (0 when the result was written)
int gemm_launch(const ge_gemm_args &a, hipStream_t s, float *colpart = nullptr, int *deferred = nullptr);
int64_t gemm_colsum_rows(const ge_gemm_args &a);
int64_t gemm_colsum_bytes(int ab_type, int64_t M, int64_t N, int64_t K);
// out[n] = alpha * sum over r < rows of part[r][n], rows added in order
int colsum_rows_launch(const float *part, int64_t rows, int64_t N, float alpha, float *out, hipStream_t st);
int64_t gemm_ws_bytes(int layout, int ab_type, int64_t M, int64_t N, int64_t K, int split_k);
// the library's fixed device scratch (gemm_bias_act_noalloc): its address on
// the current device and its size
int scratch_address(void **out);
int64_t scratch_bytes();
int colsum_launch(const void *X, int64_t M, int64_t N, int64_t ldx, int x_type, float alpha,
                  float *out, void *ws, int64_t ws_bytes, hipStream_t s, int accumulate = 0);
int64_t colsum_ws_bytes(int64_t M, int64_t N);
// fused narrow output layer of the MLP step (head.hip)
bool head_supported(int64_t B, int64_t D, int64_t C);
int64_t head_ws_bytes(int64_t B, int64_t D);
int head_launch(const half_t *H, int64_t B, int64_t D, const half_t *W, const float *bias, int64_t C,
                const int32_t *labels, float gscale, float alpha, float *Z, half_t *G, float *row_loss,
                half_t *dH, float *db, float *db_below, float *loss, void *ws, hipStream_t st);
int xent_launch(const float *logits, int64_t B, int64_t C, int64_t ld, const int32_t *labels,
                float grad_scale, float *loss_mean, float *row_loss, void *dl, int64_t ld_d,
                int d_type, int32_t *argmax, hipStream_t s, int32_t *bad_label_count = nullptr);
// persistent one-launch step of a one-hidden-layer FP32 MLP (step_persist.hip)
struct MlpPersistArgs {
  const float *X;         // [B x D0]
  const int32_t *labels;  // [B]
  float *P, *Gr, *V;      // flat params, grads, velocity: [W1, b1, W2, b2]
  float *H;               // [B x D1]
  float *Zl;              // [B x C] logits
  float *Gz;              // [B x C] dZ, scaled by 1/B
  float *row_loss;        // [B]
  float *dH;              // [B x D1]
  float *loss;            // [1]
  unsigned *sync;         // [2]: barrier counter, error word (zero at launch)
  int B, D0, D1, C;
  float lr, mu;
};
bool mlp_persist_supported(int64_t B, int64_t D0, int64_t D1, int64_t C);
int mlp_persist_launch(const MlpPersistArgs &args, hipStream_t s);
// bit-exact mode (exact.hip): the primitives as fixed sequences of rounded
// binary32 operations with linear-order sums
bool bit_exact_on();
int gemm_exact_launch(const ge_gemm_args &a, hipStream_t s);
int colsum_exact_launch(const void *X, int64_t M, int64_t N, int64_t ldx, int xt, float alpha, float *out,
                        int accumulate, hipStream_t s);
int sgd_exact_launch(float *w, const float *g, float *v, float lr, float mu, int64_t n, void *wl, int lt,
                     hipStream_t s);
int rmsnorm_exact_launch(const ge_rmsnorm_args &a, hipStream_t s);
// the block's forward as one kernel (megakernel.hip)
int64_t block_fused_ws_bytes(int64_t D, int64_t F);
int block_fused_launch(const ge_block_fused_args &a, hipStream_t s);
int to_lowp_launch(const float *w, int64_t n, void *w_lowp, int lowp_type, hipStream_t s);
int rmsnorm_launch(const ge_rmsnorm_args &a, hipStream_t s);
int64_t rmsnorm_ws_bytes(int64_t rows, int64_t D);
// A gradient segment the update forms first: g[g0 .. g0 + len) = alpha
// times the sum of `rows` partial rows [rows x len], added in row order.
struct SgdSegmentDesc {
  const float *part;
  int64_t g0, len;
  int rows;
  float alpha;
};
constexpr int kSgdMaxSegments = 4;
// segs (optional, up to kSgdMaxSegments, not overlapping): the segments of g
// formed (and written to g) before the update reads them
int sgd_launch(float *w, float *g, float *v, float lr, float mu, int64_t n, void *wl, int lt, hipStream_t s,
               const SgdSegmentDesc *segs = nullptr, int nseg = 0);

}  // namespace ge
