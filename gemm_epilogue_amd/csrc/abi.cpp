// extern "C" entry points: host-side validation, then the internal launchers.
// Nothing is enqueued unless every argument checks out.
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "common.h"

namespace ge {

static thread_local char g_err[512] = "";
static thread_local int64_t g_launches = 0;
static std::atomic<int> g_bit_exact{0};

bool bit_exact_on() { return g_bit_exact.load(std::memory_order_relaxed) != 0; }

void set_error(const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
}

// called after every kernel launch of the library
int launch_status(const char *what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("%s: launch failed: %s", what, hipGetErrorString(e));
    return GE_E_LAUNCH;
  }
  ++g_launches;
  return GE_OK;
}

}  // namespace ge

using namespace ge;

#define CHECK(cond, ...)          \
  do {                            \
    if (!(cond)) {                \
      set_error(__VA_ARGS__);     \
      return GE_E_INVALID;        \
    }                             \
  } while (0)

static const int64_t kMaxDim = (int64_t)1 << 30;

extern "C" {

int ge_abi_version(void) { return 1; }
const char *ge_last_error(void) { return g_err; }
int64_t ge_launch_count(void) { return g_launches; }
int32_t ge_set_bit_exact(int32_t on) { return g_bit_exact.exchange(on != 0 ? 1 : 0); }
int32_t ge_bit_exact(void) { return g_bit_exact.load() ? 1 : 0; }

int64_t gemm_workspace_bytes(int32_t layout, int32_t ab_type, int64_t M, int64_t N, int64_t K,
                             int32_t split_k) {
  if (layout < GE_NN || layout > GE_TN || !dtype_ok(ab_type) || M < 0 || N < 0 || K < 0 || split_k < 0)
    return -1;
  return gemm_ws_bytes(layout, ab_type, M, N, K, split_k);
}

int gemm_bias_act(const ge_gemm_args *a, ge_stream_t stream) {
  CHECK(a != nullptr, "gemm_bias_act: args is NULL");
  CHECK(a->layout >= GE_NN && a->layout <= GE_TN, "gemm_bias_act: unknown layout %d", a->layout);
  CHECK(dtype_ok(a->ab_type), "gemm_bias_act: unknown ab_type %d", a->ab_type);
  CHECK(dtype_ok(a->c_type), "gemm_bias_act: unknown c_type %d", a->c_type);
  CHECK(a->M >= 0 && a->N >= 0 && a->K >= 0, "gemm_bias_act: negative size");
  CHECK(a->M < kMaxDim && a->N < kMaxDim && a->K < kMaxDim, "gemm_bias_act: size too large");
  CHECK(a->act >= GE_ACT_NONE && a->act <= GE_ACT_LRELU_SQ_BWD, "gemm_bias_act: unknown act %d", a->act);
  CHECK(a->split_k >= 0 && a->split_k <= 1024, "gemm_bias_act: split_k out of range");
  if (a->M == 0 || a->N == 0) return GE_OK;
  const bool nn = a->layout == GE_NN, nt = a->layout == GE_NT;
  const int64_t rowsA = (nn || nt) ? a->M : a->K, colsA = (nn || nt) ? a->K : a->M;
  const int64_t colsB = nt ? a->K : a->N;
  (void)rowsA;
  if (a->K > 0) {
    CHECK(a->A != nullptr && a->B != nullptr, "gemm_bias_act: A or B is NULL");
    CHECK(a->lda >= colsA && a->lda >= 1, "gemm_bias_act: lda %lld < %lld", (long long)a->lda, (long long)colsA);
    CHECK(a->ldb >= colsB && a->ldb >= 1, "gemm_bias_act: ldb %lld < %lld", (long long)a->ldb, (long long)colsB);
  }
  CHECK(a->C != nullptr, "gemm_bias_act: C is NULL");
  CHECK(a->ldc >= a->N, "gemm_bias_act: ldc < N");
  if (a->act == GE_ACT_RELU_MASK_BWD || a->act == GE_ACT_LRELU_SQ_BWD) {
    CHECK(a->aux != nullptr, "gemm_bias_act: backward activation needs aux");
    CHECK(dtype_ok(a->aux_type) && a->ld_aux >= a->N, "gemm_bias_act: bad aux type / ld");
  }
  if (a->residual) CHECK(dtype_ok(a->res_type) && a->ld_res >= a->N, "gemm_bias_act: bad residual type / ld");
  if (a->pre) CHECK(dtype_ok(a->pre_type) && a->ld_pre >= a->N, "gemm_bias_act: bad pre type / ld");
  CHECK(a->C != a->A && a->C != a->B, "gemm_bias_act: C aliases an input");
  if (bit_exact_on()) return gemm_exact_launch(*a, (hipStream_t)stream);
  return gemm_launch(*a, (hipStream_t)stream);
}

int gemm_bias_act_noalloc(const ge_gemm_args *a, ge_stream_t stream) {
  CHECK(a != nullptr, "gemm_bias_act_noalloc: args is NULL");
  CHECK(a->layout >= GE_NN && a->layout <= GE_TN && dtype_ok(a->ab_type) && a->M >= 0 && a->N >= 0 && a->K >= 0 &&
            a->split_k >= 0 && a->split_k <= 1024,
        "gemm_bias_act_noalloc: bad layout, type, size or split_k");
  // the bit-exact kernels keep no partials
  const int64_t need = bit_exact_on() ? 0 : gemm_ws_bytes(a->layout, a->ab_type, a->M, a->N, a->K, a->split_k);
  if (need > scratch_bytes()) {
    set_error("gemm_bias_act_noalloc: split-K partials need %lld bytes, more than the %lld-byte scratch",
              (long long)need, (long long)scratch_bytes());
    return GE_E_WORKSPACE;
  }
  ge_gemm_args b = *a;
  b.workspace = nullptr;
  b.workspace_bytes = 0;
  if (need > 0) {
    void *p = nullptr;
    const int st = scratch_address(&p);
    if (st != GE_OK) return st;
    b.workspace = p;
    b.workspace_bytes = scratch_bytes();
  }
  return gemm_bias_act(&b, stream);
}

int64_t colsum_workspace_bytes(int64_t M, int64_t N) {
  if (M < 0 || N < 0) return -1;
  return colsum_ws_bytes(M, N);
}

int colsum(const void *X, int64_t M, int64_t N, int64_t ldx, int32_t x_type, float alpha, float *out,
           int32_t accumulate, void *workspace, int64_t workspace_bytes, ge_stream_t stream) {
  CHECK(M >= 0 && N >= 0 && M < kMaxDim && N < kMaxDim, "colsum: bad size");
  CHECK(dtype_ok(x_type), "colsum: unknown x_type %d", x_type);
  if (N == 0) return GE_OK;
  CHECK(out != nullptr, "colsum: out is NULL");
  if (M > 0) CHECK(X != nullptr && ldx >= N, "colsum: X is NULL or ldx < N");
  if (bit_exact_on())
    return colsum_exact_launch(X, M, N, ldx, x_type, alpha, out, accumulate != 0, (hipStream_t)stream);
  return colsum_launch(X, M, N, ldx, x_type, alpha, out, workspace, workspace_bytes, (hipStream_t)stream,
                       accumulate != 0);
}

int softmax_xent_fwd_bwd(const float *logits, int64_t B, int64_t C, int64_t ld, const int32_t *labels,
                         float grad_scale, float *loss_mean, float *row_loss, void *dlogits, int64_t ld_d,
                         int32_t d_type, int32_t *argmax, int32_t *bad_label_count, ge_stream_t stream) {
  CHECK(B >= 0 && B < kMaxDim, "softmax_xent_fwd_bwd: bad B");
  CHECK(C >= 1 && C <= 4096, "softmax_xent_fwd_bwd: C must be in [1, 4096]");
  CHECK(loss_mean != nullptr, "softmax_xent_fwd_bwd: loss_mean is NULL");
  if (B > 0) {
    CHECK(logits != nullptr && labels != nullptr && row_loss != nullptr,
          "softmax_xent_fwd_bwd: logits, labels or row_loss is NULL");
    CHECK(ld >= C, "softmax_xent_fwd_bwd: ld < C");
    if (dlogits) CHECK(dtype_ok(d_type) && ld_d >= C, "softmax_xent_fwd_bwd: bad d_type / ld_d");
  }
  return xent_launch(logits, B, C, ld, labels, grad_scale, loss_mean, row_loss, dlogits, ld_d, d_type, argmax,
                     (hipStream_t)stream, bad_label_count);
}

int64_t rmsnorm_workspace_bytes(int64_t rows, int64_t D) {
  if (rows < 0 || D < 0) return -1;
  return rmsnorm_ws_bytes(rows, D);
}

int rmsnorm_fwd_bwd(const ge_rmsnorm_args *a, ge_stream_t stream) {
  CHECK(a != nullptr, "rmsnorm_fwd_bwd: args is NULL");
  CHECK(a->pass == GE_FWD || a->pass == GE_BWD, "rmsnorm_fwd_bwd: unknown pass %d", a->pass);
  CHECK(a->rows >= 0 && a->rows < kMaxDim, "rmsnorm_fwd_bwd: bad rows");
  CHECK(a->D >= 1 && a->D <= 4096, "rmsnorm_fwd_bwd: D must be in [1, 4096]");
  CHECK(a->eps >= 0.f, "rmsnorm_fwd_bwd: eps < 0");
  if (a->rows == 0) return GE_OK;
  CHECK(a->x != nullptr && dtype_ok(a->x_type) && a->ld_x >= a->D, "rmsnorm_fwd_bwd: bad x");
  CHECK(a->r != nullptr, "rmsnorm_fwd_bwd: r is NULL");
  if (a->pass == GE_FWD) {
    CHECK(a->y != nullptr && dtype_ok(a->y_type) && a->ld_y >= a->D, "rmsnorm_fwd_bwd: bad y");
  } else {
    CHECK(a->dy != nullptr && dtype_ok(a->dy_type) && a->ld_dy >= a->D, "rmsnorm_fwd_bwd: bad dy");
    CHECK(a->dx != nullptr && dtype_ok(a->dx_type) && a->ld_dx >= a->D, "rmsnorm_fwd_bwd: bad dx");
    if (a->dres) CHECK(dtype_ok(a->dres_type) && a->ld_dres >= a->D, "rmsnorm_fwd_bwd: bad dres");
  }
  if (bit_exact_on()) return rmsnorm_exact_launch(*a, (hipStream_t)stream);
  return rmsnorm_launch(*a, (hipStream_t)stream);
}

int sgd_momentum(float *w, const float *g, float *v, float lr, float momentum, int64_t n, void *w_lowp,
                 int32_t lowp_type, ge_stream_t stream) {
  CHECK(n >= 0, "sgd_momentum: n < 0");
  if (n == 0) return GE_OK;
  CHECK(w != nullptr && g != nullptr && v != nullptr, "sgd_momentum: w, g or v is NULL");
  if (w_lowp) CHECK(lowp_type == GE_F16 || lowp_type == GE_BF16, "sgd_momentum: lowp_type must be F16 or BF16");
  if (bit_exact_on()) return sgd_exact_launch(w, g, v, lr, momentum, n, w_lowp, lowp_type, (hipStream_t)stream);
  // without a gradient segment the update only reads g
  return sgd_launch(w, const_cast<float *>(g), v, lr, momentum, n, w_lowp, lowp_type, (hipStream_t)stream);
}

int64_t mlp_block_fused_workspace_bytes(int64_t D, int64_t F) {
  if (D < 0 || F < 0) return -1;
  return block_fused_ws_bytes(D, F);
}

int mlp_block_fwd_fused(const ge_block_fused_args *a, ge_stream_t stream) {
  CHECK(a != nullptr, "mlp_block_fwd_fused: args is NULL");
  CHECK(a->type == GE_BF16 || a->type == GE_F16, "mlp_block_fwd_fused: type must be BF16 or F16");
  CHECK(a->rows >= 0 && a->rows < kMaxDim && a->D >= 1 && a->F >= 1 && a->D < kMaxDim && a->F < kMaxDim,
        "mlp_block_fwd_fused: bad sizes");
  CHECK(a->eps >= 0.f, "mlp_block_fwd_fused: eps < 0");
  CHECK(a->w_up != nullptr && a->w_down != nullptr, "mlp_block_fwd_fused: a weight is NULL");
  if (a->rows > 0) CHECK(a->x != nullptr && a->y != nullptr, "mlp_block_fwd_fused: x or y is NULL");
  CHECK(a->workspace != nullptr && a->workspace_bytes >= block_fused_ws_bytes(a->D, a->F),
        "mlp_block_fwd_fused: workspace needs %lld bytes", (long long)block_fused_ws_bytes(a->D, a->F));
  const uintptr_t al = (uintptr_t)a->x | (uintptr_t)a->y | (uintptr_t)a->w_up | (uintptr_t)a->w_down |
                       (uintptr_t)a->n | (uintptr_t)a->u | (uintptr_t)a->a | (uintptr_t)a->workspace;
  CHECK(al % 16 == 0, "mlp_block_fwd_fused: every buffer must be 16-byte aligned");
  return block_fused_launch(*a, (hipStream_t)stream);
}

int params_to_lowp(const float *w, void *w_lowp, int64_t n, int32_t lowp_type, ge_stream_t stream) {
  CHECK(n >= 0, "params_to_lowp: n < 0");
  if (n == 0) return GE_OK;
  CHECK(w != nullptr && w_lowp != nullptr, "params_to_lowp: NULL pointer");
  CHECK(lowp_type == GE_F16 || lowp_type == GE_BF16, "params_to_lowp: lowp_type must be F16 or BF16");
  return to_lowp_launch(w, n, w_lowp, lowp_type, (hipStream_t)stream);
}

}  // extern "C"
