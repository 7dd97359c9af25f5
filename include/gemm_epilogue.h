/*
 * gemm_epilogue.h -- C ABI of the MI355X (gfx950) GEMM-epilogue training path.
 *
 * One training step of a small dense network: mixed-precision GEMMs (FP16 /
 * BF16 / FP32 inputs, FP32 accumulation on MFMA) whose bias and activation are
 * applied to the FP32 accumulator in the epilogue, converted once at the final
 * store, plus the glue around them: stable softmax cross-entropy forward and
 * backward, RMSNorm with FP32 statistics, column-sum bias gradients, the
 * ReLU-mask backward (a dgrad-GEMM epilogue) and one flat SGD-momentum update.
 *
 * Conventions for every entry point
 * ---------------------------------
 *  - Memory: the caller allocates and owns all device memory (inputs,
 *    outputs, parameters, gradients, velocity, workspace).  The library never
 *    allocates or frees device memory and never synchronises; pointers named
 *    "device" must point to device memory (or be NULL where allowed).  Host
 *    structs passed by pointer are read during the call only.
 *  - Streams: every call enqueues asynchronously on `stream` (a hipStream_t;
 *    NULL = the null stream) and returns before the work finishes.
 *  - Layout: all matrices are row-major with an explicit leading dimension
 *    (elements between consecutive rows, >= the row length).
 *  - Errors: every call returns GE_OK or a negative status.  Arguments are
 *    validated on the host before anything is enqueued; on GE_E_INVALID,
 *    GE_E_UNSUPPORTED or GE_E_WORKSPACE nothing was enqueued.  GE_E_LAUNCH
 *    reports a HIP launch error.  ge_last_error() returns a thread-local
 *    message for the last failing call.  No call aborts or prints.
 *  - Determinism: for identical inputs the results are bitwise identical from
 *    run to run (no floating-point atomics; split-K partials and every
 *    reduction are summed in a fixed order).
 *
 * Sources (web pages; cited by title and section):
 *  [CAP] "Capstone 5: train a network with your CUDA kernels" (Day 100).
 *  [CAT] "The Work Moved Down a Layer" (Cat Chat, Vulkan compute).
 *  [MK]  "Full-Depth MLP Megakernel + Fused Attention Preprocessing".
 *  [HV3] "HIP + Vulkan backends -- Phase 3 (path to 100%)".
 */
#ifndef GEMM_EPILOGUE_H
#define GEMM_EPILOGUE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void *ge_stream_t; /* hipStream_t */

/* status codes */
#define GE_OK 0
#define GE_E_INVALID (-1)     /* bad argument; nothing enqueued */
#define GE_E_UNSUPPORTED (-2) /* valid but not supported combination */
#define GE_E_LAUNCH (-3)      /* HIP launch error */
#define GE_E_WORKSPACE (-4)   /* workspace missing or too small */

/* storage types */
#define GE_F32 0
#define GE_F16 1  /* IEEE binary16 */
#define GE_BF16 2 /* bfloat16 */

/* operand layouts (see gemm_bias_act) */
#define GE_NN 0
#define GE_NT 1
#define GE_TN 2

/* epilogue activations */
#define GE_ACT_NONE 0
#define GE_ACT_RELU 1          /* max(v, 0)                      [CAP] Read the worked reference */
#define GE_ACT_LRELU_SQ 2      /* (v > 0 ? v : s*v)^2            [MK] What Worked */
#define GE_ACT_RELU_MASK_BWD 3 /* v * [aux > 0]                  [CAP] Work through the backward pass */
#define GE_ACT_LRELU_SQ_BWD 4  /* v * (aux > 0 ? 2aux : 2s^2 aux) [MK] Credits (backward epilogue) */

int ge_abi_version(void); /* returns 1 */
const char *ge_last_error(void);
/* Number of kernels the calling thread has enqueued through the library so
 * far (every entry point counts its launches); the difference around a call
 * is that call's launch count. */
int64_t ge_launch_count(void);
/* Shader clock under matrix-core load, for reading measured rates against
 * the nominal peak: `blocks` blocks of 256 threads each run `iters` rounds of
 * eight 32x32x16 MFMAs; block b writes ticks[3b] = shader-clock cycles and
 * ticks[3b + 1] = 100 MHz reference ticks over its chain (ticks[3b + 2] is
 * 0).  ticks: device int64 [3 * blocks], caller-owned.  GE_E_INVALID for a
 * NULL buffer or blocks outside [1, 65536]. */
int ge_clock_probe(int64_t *ticks, int32_t blocks, int32_t iters, ge_stream_t stream);

/* ------------------------------------------------------------------------
 * Bit-exact mode -- [HV3] "Phase-3 bug hunt" (linear-order subgroup sum,
 * correctly rounded divide, refined rsqrt): with the mode on, gemm_bias_act
 * (and its _noalloc form), colsum, rmsnorm_fwd_bwd and sgd_momentum compute
 * their outputs as the fixed sequences of IEEE binary32 operations below,
 * every operation rounded to nearest even, none fused, so a CPU running the
 * same sequence reproduces every output bit.  Stores convert once with RNE.
 *   gemm:    acc = +0; for k = 0 .. K-1: acc = acc + a_k * b_k;
 *            v = alpha * acc; v = v + bias[n]; pre = convert(v);
 *            RELU: v = v > 0 ? v : +0;  LRELU_SQ: t = v > 0 ? v : s * v, v = t * t;
 *            RELU_MASK_BWD: v = v * (aux > 0 ? 1 : 0);
 *            LRELU_SQ_BWD: v = v * (aux > 0 ? 2 * aux : ((2 * s) * s) * aux);
 *            v = v + residual;  C = convert(v)
 *   colsum:  t = alpha * (x_0 + x_1 + ... in row order); out = t or out + t
 *   rmsnorm: FWD ss = sum_j x_j * x_j in j order; r = 1 / sqrt(ss / D + eps);
 *            y = (x * r) * gamma.  BWD xh = x * r; g = dy * gamma;
 *            c = (sum_j g * xh in j order) / D; dx = r * (g - xh * c) + dres;
 *            dgamma[j] = sum over rows in row order of dy * xh (no workspace)
 *   sgd:     vel = momentum * v - lr * g; v = vel; w = w + vel
 * Divide and square root are correctly rounded ([HV3] refines the hardware
 * rsqrt to within one ulp; a correctly rounded sqrt and reciprocal is the
 * reading a CPU reproduces exactly).  softmax_xent_fwd_bwd and the composite
 * steps (mlp_train_step, mlp_block_fwd_bwd, gru_lm_train_step) are not
 * affected: exp and log keep their library rounding.  The mode is one
 * process-wide switch; one thread per output walks its sum, so it is slow.
 * ge_set_bit_exact returns the previous setting.
 * ---------------------------------------------------------------------- */
int32_t ge_set_bit_exact(int32_t on);
int32_t ge_bit_exact(void);

/* ------------------------------------------------------------------------
 * gemm_bias_act -- C = act(alpha * op(A) op(B) + bias) [+ residual]
 *
 * [CAP] "Read the worked reference": the forward multiply keeps bias and ReLU
 * in its epilogue; "Work through the backward pass": dW = X^T dH and
 * dX = dH W^T are multiplies with one transposed input, dH applies the ReLU
 * mask.  [CAT] "The Debugging Lesson Was Numerical": accumulate in FP32, apply
 * bias and activation in FP32, convert once at the final store.
 *
 * Layouts (row-major storage):
 *   GE_NN: A [M x K] (lda >= K), B [K x N] (ldb >= N):  C = A   B
 *   GE_NT: A [M x K] (lda >= K), B [N x K] (ldb >= K):  C = A   B^T
 *   GE_TN: A [K x M] (lda >= M), B [K x N] (ldb >= N):  C = A^T B
 * A and B share ab_type (F32, F16 or BF16); products accumulate in FP32.
 * Epilogue, per element (m, n), all in FP32:
 *   v = alpha * acc + (bias ? bias[n] : 0)          bias: device f32 [N] or NULL
 *   pre[m, n] = convert(v)                          optional pre-activation store
 *   forward acts (NONE, RELU, LRELU_SQ): v = act(v)
 *   backward acts (*_BWD): v = v * f(aux[m, n])     aux required, aux_type, ld_aux
 *   v += residual[m, n]                             optional (res_type, ld_res)
 *   C[m, n] = convert(v)                            c_type, ldc; one RNE rounding
 * act_slope is the leaky slope s of the LRELU_SQ pair (0.5 in the MLP block).
 * M, N, K >= 0 (M or N == 0: no-op; K == 0: acc = 0).  C must not alias A, B.
 * Split-K: large-K, small-output problems split the K loop; FP32 partials go
 * to `workspace` and are summed in fixed order by a finishing pass that
 * applies the epilogue.  gemm_workspace_bytes() gives the size needed
 * (0 if none); split_k = 0 picks automatically, >= 1 forces that count.
 * ---------------------------------------------------------------------- */
typedef struct ge_gemm_args {
  int32_t layout;  /* GE_NN / GE_NT / GE_TN */
  int32_t ab_type; /* GE_F32 / GE_F16 / GE_BF16 */
  int64_t M, N, K;
  const void *A; /* device */
  int64_t lda;
  const void *B; /* device */
  int64_t ldb;
  float alpha;
  const float *bias; /* device f32 [N] or NULL */
  int32_t act;       /* GE_ACT_* */
  float act_slope;
  const void *aux; /* device [M x N] or NULL (required by *_BWD acts) */
  int64_t ld_aux;
  int32_t aux_type;
  const void *residual; /* device [M x N] or NULL */
  int64_t ld_res;
  int32_t res_type;
  void *C; /* device [M x N] */
  int64_t ldc;
  int32_t c_type;
  void *pre; /* device [M x N] or NULL */
  int64_t ld_pre;
  int32_t pre_type;
  void *workspace; /* device or NULL */
  int64_t workspace_bytes;
  int32_t split_k; /* 0 = auto */
} ge_gemm_args;

int gemm_bias_act(const ge_gemm_args *args, ge_stream_t stream);
/* gemm_bias_act for callers that cannot allocate (code under stream capture,
 * serving loops, harnesses that forbid hipMalloc): the same operation and
 * result bits as gemm_bias_act, but args->workspace is ignored and the split-K
 * partials live in the library's own fixed device scratch of 64 MiB (one per
 * GPU, held until the process ends).  No allocation happens in the call.
 * Returns GE_E_WORKSPACE when the partials would exceed 64 MiB
 * (gemm_workspace_bytes(...) > 67108864); nothing is enqueued then.  Every
 * element of the partials is written before it is read, so nothing needs
 * clearing between calls.  All calls on one GPU share the scratch: calls that
 * may overlap on one GPU (different streams without ordering, or several
 * threads) race and must be serialized by the caller. */
int gemm_bias_act_noalloc(const ge_gemm_args *args, ge_stream_t stream);
/* bytes of workspace gemm_bias_act needs for this problem with split_k
 * (0 = the automatic choice); 0 when no split is used. */
int64_t gemm_workspace_bytes(int32_t layout, int32_t ab_type, int64_t M, int64_t N,
                             int64_t K, int32_t split_k);

/* ------------------------------------------------------------------------
 * colsum -- out[n] = alpha * sum_m X[m, n]            (accumulate == 0)
 *           out[n] = out[n] + alpha * sum_m X[m, n]   (accumulate != 0)
 * [CAP] "Work through the backward pass" / "Check your mapping": each db is
 * a column reduction over the batch.  X: device [M x N] (x_type, ldx >= N);
 * out: device f32 [N].  Sums in FP32 in a fixed order.  Problems with many
 * rows use a two-pass reduction whose partials live in `workspace`
 * (colsum_workspace_bytes(M, N) bytes; 0 means none needed).
 * ---------------------------------------------------------------------- */
int colsum(const void *X, int64_t M, int64_t N, int64_t ldx, int32_t x_type, float alpha,
           float *out, int32_t accumulate, void *workspace, int64_t workspace_bytes,
           ge_stream_t stream);
int64_t colsum_workspace_bytes(int64_t M, int64_t N);

/* ------------------------------------------------------------------------
 * softmax_xent_fwd_bwd -- stable softmax cross-entropy, loss and dlogits
 * [CAP] "The minimum model" and "Read the worked reference": subtract each
 * row's maximum before exponentiating; the loss kernel yields loss and dZ.
 * [CAT] "The Debugging Lesson Was Numerical": reductions in FP32.
 *   per row b:  m = max_c z;  lse = m + log(sum_c exp(z - m));
 *               row_loss[b] = lse - z[label[b]];
 *               dlogits[b, c] = grad_scale * (exp(z - lse) - [c == label[b]])
 *   loss_mean[0] = (1/B) sum_b row_loss[b]      (fixed-order sum)
 *   argmax[b] = lowest index of the row maximum  (optional)
 * logits: device f32 [B x C] (ld >= C); labels: device int32 [B] in [0, C)
 * (a label outside that range reads nothing and gives a NaN row loss, so the
 * mean is NaN too); row_loss: device f32 [B] (required: it is also the
 * scratch of the mean); loss_mean: device f32 [1]; dlogits: device [B x C]
 * (d_type, ld_d) or NULL; argmax: device int32 [B] or NULL;
 * bad_label_count: device int32 [1] or NULL, receives the number of labels
 * outside [0, C) (written, not accumulated; labels are device data, so this
 * is how a caller learns of them without a host check).  C <= 4096.
 * ---------------------------------------------------------------------- */
int softmax_xent_fwd_bwd(const float *logits, int64_t B, int64_t C, int64_t ld,
                         const int32_t *labels, float grad_scale, float *loss_mean,
                         float *row_loss, void *dlogits, int64_t ld_d, int32_t d_type,
                         int32_t *argmax, int32_t *bad_label_count, ge_stream_t stream);

/* ------------------------------------------------------------------------
 * rmsnorm_fwd_bwd -- RMSNorm over rows of width D, FP32 statistics
 * [CAT] "The Debugging Lesson Was Numerical": normalisation statistics stay
 * FP32; [MK] "What Worked": RMSNorm opens the MLP block.
 *   GE_FWD: r[i] = 1/sqrt(mean_j x[i,j]^2 + eps);  y = x * r (* gamma[j])
 *   GE_BWD: xh = x * r;  g = dy (* gamma);  c = mean_j g xh;
 *           dx = r * (g - xh * c) (+ dres);  dgamma[j] = sum_i dy xh (optional)
 * x: device [rows x D] (x_type, ld_x); y: (y_type, ld_y); r: device f32 [rows];
 * dy: (dy_type, ld_dy); dres: (dres_type, ld_dres) or NULL; dx: (dx_type,
 * ld_dx); gamma: device f32 [D] or NULL; dgamma: device f32 [D] or NULL (needs
 * workspace of rmsnorm_workspace_bytes(rows, D) bytes).  1 <= D <= 4096.
 * ---------------------------------------------------------------------- */
#define GE_FWD 0
#define GE_BWD 1
typedef struct ge_rmsnorm_args {
  int32_t pass; /* GE_FWD or GE_BWD */
  int64_t rows, D;
  float eps;
  const void *x;
  int64_t ld_x;
  int32_t x_type;
  const float *gamma; /* or NULL */
  void *y;            /* FWD output */
  int64_t ld_y;
  int32_t y_type;
  float *r;       /* FWD output / BWD input, f32 [rows] */
  const void *dy; /* BWD input */
  int64_t ld_dy;
  int32_t dy_type;
  const void *dres; /* BWD optional residual gradient added to dx */
  int64_t ld_dres;
  int32_t dres_type;
  void *dx; /* BWD output */
  int64_t ld_dx;
  int32_t dx_type;
  float *dgamma; /* BWD optional */
  void *workspace;
  int64_t workspace_bytes;
} ge_rmsnorm_args;

int rmsnorm_fwd_bwd(const ge_rmsnorm_args *args, ge_stream_t stream);
int64_t rmsnorm_workspace_bytes(int64_t rows, int64_t D);

/* ------------------------------------------------------------------------
 * sgd_momentum -- one update over a flat parameter buffer
 * [CAP] "Read the worked reference": all parameter tensors live in one flat
 * buffer; vel = momentum * v - lr * g; v = vel; w += vel, for every element.
 * w, g, v: device f32 [n] (w, v updated in place); w_lowp: device [n] of
 * lowp_type (F16 or BF16) receiving convert(w_new), or NULL.
 * ---------------------------------------------------------------------- */
int sgd_momentum(float *w, const float *g, float *v, float lr, float momentum, int64_t n,
                 void *w_lowp, int32_t lowp_type, ge_stream_t stream);

/* params_to_lowp -- w_lowp[i] = convert(w[i]), round to nearest even: the
 * low-precision working copy of a flat parameter buffer that the GEMMs read
 * ([CAT] "The Debugging Lesson Was Numerical": FP16 only as GEMM input), as
 * sgd_momentum keeps it after each update; used to form it from the initial
 * FP32 parameters.  w: device f32 [n]; w_lowp: device [n] of lowp_type
 * (F16 or BF16). */
int params_to_lowp(const float *w, void *w_lowp, int64_t n, int32_t lowp_type, ge_stream_t stream);

/* ------------------------------------------------------------------------
 * mlp_train_step -- one SGD-momentum step of a dense ReLU MLP
 * [CAP] "The minimum model", "Work through the backward pass", "Read the
 * worked reference":  H_l = ReLU(H_{l-1} W_l + b_l), Z = H_{L-1} W_L + b_L,
 * stable softmax CE (mean over the batch), dW_l = H_{l-1}^T G_l,
 * db_l = colsum(G_l), G_{l-1} = (G_l W_l^T) * (H_{l-1} > 0), then one
 * momentum update over the flat buffer.
 *
 * Flat parameter layout: [W1, b1, W2, b2, ...], W_l row-major
 * [dims[l-1] x dims[l]], biases f32; params / grads / velocity are device f32
 * [mlp_param_count].  storage = GE_F32: X f32, everything stored in FP32,
 * G = (p - onehot)/B.  storage = GE_F16: X f16, GEMMs read the FP16 working
 * copy `params_lowp` (device f16 [mlp_param_count], kept in step by the
 * update), hidden activations, G = p - onehot (unscaled) and dH are FP16,
 * logits FP32, and 1/B is applied in the weight/bias gradient epilogues.
 * labels: device int32 [B]; loss_out: device f32 [1] (mean loss).
 * Workspace: mlp_workspace_bytes(desc, B) bytes; its layout is reported by
 * mlp_workspace_offsets.  The masked hidden gradients alternate between two
 * buffers, starting with the first for dH_{L-1} (so after the step dH_{L-1-2k}
 * is in the first and dH_{L-2-2k} in the second).
 * ---------------------------------------------------------------------- */
/* plan: GE_MLP_AUTO takes the persistent step where it applies, else the
 * launch chain; GE_MLP_CHAIN enqueues the step as the fixed sequence of
 * library kernels (any shape); GE_MLP_PERSISTENT runs the whole step as one
 * launch of 128 resident blocks with two grid-wide barriers ([CAP] "Explain
 * a different result": the small step is bound by launches) after a tiny
 * clear of its barrier words, and returns GE_E_UNSUPPORTED unless L = 2,
 * storage = GE_F32, 1 <= B <= 128, dims[0] % 4 == 0 and <= 1024,
 * dims[1] % 64 == 0 and <= 512, dims[2] <= 16, and the device holds 128 of
 * its blocks at once.  X must then be 16-byte aligned (else GE_E_INVALID).
 * Both plans compute the same step and fill the same workspace slots; their
 * summation orders differ.  A persistent step whose barrier gave up (it
 * waits a bounded time) writes a NaN mean loss. */
#define GE_MLP_AUTO 0
#define GE_MLP_CHAIN 1
#define GE_MLP_PERSISTENT 2

typedef struct ge_mlp_desc {
  int32_t n_layers;     /* number of weight layers L >= 1 */
  const int64_t *dims;  /* host [L + 1] widths, dims[0] = input, dims[L] = classes */
  int32_t storage;      /* GE_F32 or GE_F16 */
  int32_t plan;         /* GE_MLP_AUTO, GE_MLP_CHAIN or GE_MLP_PERSISTENT */
} ge_mlp_desc;

typedef struct ge_mlp_buffers {
  float *params;      /* device f32 [P] */
  float *grads;       /* device f32 [P] (written) */
  float *velocity;    /* device f32 [P] */
  void *params_lowp;  /* device f16 [P] (GE_F16 storage) or NULL */
  void *workspace;    /* device */
  int64_t workspace_bytes;
} ge_mlp_buffers;

int64_t mlp_param_count(int32_t n_layers, const int64_t *dims);
int64_t mlp_workspace_bytes(const ge_mlp_desc *desc, int64_t B);
/* writes n_layers + 4 byte offsets: H_1 .. H_{L-1}, Z (f32), G, row_loss (f32),
 * and the two hidden-gradient buffers */
int mlp_workspace_offsets(const ge_mlp_desc *desc, int64_t B, int64_t *offsets, int32_t n);
int mlp_train_step(const ge_mlp_desc *desc, const ge_mlp_buffers *buf, const void *X,
                   const int32_t *labels, int64_t B, float lr, float momentum,
                   float *loss_out, ge_stream_t stream);

/* ------------------------------------------------------------------------
 * mlp_block_fwd_bwd -- transformer MLP block, forward and backward
 * [MK] "What Worked": RMSNorm -> up projection -> LeakyReLU^2 -> down
 * projection -> residual; "Credits": the activation derivative as a
 * backward GEMM epilogue.  [CAT] "The Debugging Lesson Was Numerical": FP32
 * normalisation statistics.  Enqueues, on `stream`:
 *   r = 1/sqrt(mean_j x^2 + eps);  n = x r                      (RMSNorm)
 *   u = n W_up (stored), a = (u > 0 ? u : slope u)^2            (NN, from FP32 u)
 *   y = x + a W_down                                            (NN, residual)
 *   du = (dy W_down^T) * (u > 0 ? 2u : 2 slope^2 u)             (NT, stored u)
 *   dW_down = a^T dy;  dn = du W_up^T;  dW_up = n^T du          (TN, NT, TN)
 *   dx = dy + r (dn - xh mean_j(dn xh)),  xh = x r              (RMSNorm bwd)
 * type (GE_BF16 or GE_F16) is the storage of x, W_up [D x F], W_down [F x D],
 * dy, and of the outputs y, n, u, a, du, dx (all row-major, contiguous);
 * r (f32 [rows]), dn (f32 [rows x D]), dw_up (f32 [D x F]) and dw_down (f32
 * [F x D]) are FP32.  All pointers are device memory owned by the caller;
 * the weight gradients need mlp_block_workspace_bytes() of workspace.
 * 1 <= D <= 4096.
 * ---------------------------------------------------------------------- */
typedef struct ge_block_args {
  int64_t rows, D, F;
  float eps, slope;
  int32_t type;
  const void *x, *w_up, *w_down, *dy;
  void *y;
  float *r;
  void *n, *u, *a, *du;
  float *dn;
  void *dx;
  float *dw_up, *dw_down;
  void *workspace;
  int64_t workspace_bytes;
} ge_block_args;

int64_t mlp_block_workspace_bytes(int64_t rows, int64_t D, int64_t F, int32_t type);
int mlp_block_fwd_bwd(const ge_block_args *args, ge_stream_t stream);

/* ------------------------------------------------------------------------
 * mlp_block_fwd_fused -- the block's forward pass as one kernel
 * [MK] "What Worked": RMSNorm -> up projection -> LeakyReLU^2 -> down
 * projection -> residual in one kernel, the F-wide intermediate accumulated
 * in 64-wide chunks on chip and never written to HBM; "What Didn't Work":
 * that kernel lost to library GEMMs on its GPU, so this is the variant to
 * measure against the GEMM chain of mlp_block_fwd_bwd, not a replacement.
 * Same arithmetic and storage as the forward half of mlp_block_fwd_bwd:
 *   r = 1/sqrt(mean_j x^2 + eps);  n = convert(x r);  u = n W_up (FP32);
 *   a = convert((u > 0 ? u : slope u)^2);  y = convert(x + a W_down).
 * type: GE_BF16 or GE_F16, the storage of x, w_up [D x F], w_down [F x D],
 * y and the optional n, u, a (all device, row-major, contiguous); r: device
 * f32 [rows] or NULL; n [rows x D] and u [rows x F] are written when not NULL
 * (what the backward pass consumes), and a [rows x F] too (for checking; the
 * point of the kernel is that a need not reach HBM).  D must be 512 and F
 * a positive multiple of 64 (else GE_E_UNSUPPORTED).  workspace: device,
 * mlp_block_fused_workspace_bytes(D, F) bytes, receives transposed copies of
 * the two weights (written by a first small kernel of the same call).
 * ---------------------------------------------------------------------- */
typedef struct ge_block_fused_args {
  int64_t rows, D, F;
  float eps, slope;
  int32_t type;
  const void *x, *w_up, *w_down;
  void *y;
  float *r;
  void *n, *u, *a;
  void *workspace;
  int64_t workspace_bytes;
} ge_block_fused_args;

int64_t mlp_block_fused_workspace_bytes(int64_t D, int64_t F);
int mlp_block_fwd_fused(const ge_block_fused_args *args, ge_stream_t stream);

/* ------------------------------------------------------------------------
 * Embedding rows and their gradient (the byte-level recurrent LM).
 * embedding_gather: out[i, :] = table[idx[i], :] for i < n; table [V x H]
 * (type, ld_table), out [n x H] (out_type, ld_out); an index outside [0, V)
 * yields a zero row (nothing is read for it).
 * embedding_grad: dE[v, :] = alpha * sum over i with idx[i] == v of dX[i, :];
 * every row of dE [V x H] (f32, ld_de) is written, rows with no occurrence
 * get zeros; an index outside [0, V) contributes nothing.  The positions are
 * first ordered by index value (a stable counting sort into `workspace`,
 * embedding_grad_workspace_bytes(n, V) bytes), then each row of dE is the sum
 * of its run, taken in 16 contiguous pieces of increasing i added in order:
 * a fixed order, so the result is deterministic, and dX is read once
 * (O(n H + V H) work).  V <= 16384.
 * ---------------------------------------------------------------------- */
int embedding_gather(const void *table, int64_t V, int64_t H, int64_t ld_table, int32_t type,
                     const int32_t *idx, int64_t n, void *out, int64_t ld_out, int32_t out_type,
                     ge_stream_t stream);
int embedding_grad(const void *dX, int64_t ld_dx, int32_t dx_type, const int32_t *idx, int64_t n,
                   int64_t V, int64_t H, float alpha, float *dE, int64_t ld_de, void *workspace,
                   int64_t workspace_bytes, ge_stream_t stream);
int64_t embedding_grad_workspace_bytes(int64_t n, int64_t V);

/* ------------------------------------------------------------------------
 * GRU gate arithmetic of one timestep, forward and backward
 * [CAT] "The Work Moved Down a Layer" (the GRU gate shader of the recurrent
 * trainer), "The Debugging Lesson Was Numerical" (recurrent state and gate
 * math in FP32, FP16 only for GEMM inputs).  The pages print no equations;
 * the cell is the standard one (gate blocks r, z, n along 3H, the hidden
 * bias inside the reset product, which the caller's GH already holds):
 * gru_gates_fwd, per batch row b and unit j:
 *   r = sigmoid(GI_r + GH_r);  z = sigmoid(GI_z + GH_z);
 *   n = tanh(GI_n + r GH_n);   h = (1 - z) n + z h_prev
 * GI, GH: device f32 [B x 3H] (row b = [r | z | n] blocks, GI = x W_i + b_i,
 * GH = h_prev W_h + b_h); h_prev: device f32 [B x H] or NULL (h_0 = 0);
 * outputs r, z, n, h: device f32 [B x H] (r, z, n are kept for the
 * backward); h_f16: device f16 [B x H] copy of h for the next recurrent
 * GEMM, or NULL.
 * gru_gates_bwd, with dh = dh_out + carry (carry: gradient reaching h from
 * the next timestep, NULL = 0) and the same r, z, n, GH, h_prev:
 *   dn = dh (1 - z);  dz = dh (h_prev - n);  dh_dir = dh z;
 *   dnh = dn (1 - n^2);  dGr = dnh GH_n r (1 - r);  dGz = dz z (1 - z);
 *   dGH = [dGr | dGz | dnh r],  dGI = [dGr | dGz | dnh]
 * dGH, dGI: device f16 [B x 3H] (GEMM inputs of the carry and weight
 * gradients); dh_dir: device f32 [B x H] (the part of dh_prev that bypasses
 * W_h).  All rows contiguous; H % 4 == 0; f32 pointers 16-byte aligned,
 * f16 pointers 8-byte aligned (GE_E_INVALID otherwise).
 * ---------------------------------------------------------------------- */
int gru_gates_fwd(const float *GI, const float *GH, const float *h_prev, int64_t B, int64_t H,
                  float *r, float *z, float *n, float *h, void *h_f16, ge_stream_t stream);
int gru_gates_bwd(const float *dh_out, const float *carry, const float *r, const float *z,
                  const float *n, const float *GH, const float *h_prev, int64_t B, int64_t H,
                  void *dGH, void *dGI, float *dh_dir, ge_stream_t stream);

/* ------------------------------------------------------------------------
 * gru_lm_train_step -- one training step of a byte-level GRU language model
 * [CAT] "The Work Moved Down a Layer": GEMM, GRU gates, RMSNorm, softmax
 * cross-entropy, gradient reduction and optimizer shaders; "Keep state
 * resident"; "The Debugging Lesson Was Numerical": recurrent state and
 * normalisation statistics in FP32, FP16 for GEMM inputs.  The pages print no
 * GRU equations; the cell is the standard one, gate blocks (r, z, n) along
 * 3H, hidden bias inside the reset product, h_0 = 0:
 *   GI = x_t W_i + b_i;  GH = h_{t-1} W_h + b_h;  r = sigmoid(GI_r + GH_r);
 *   z = sigmoid(GI_z + GH_z);  n = tanh(GI_n + r GH_n);  h_t = (1-z) n + z h_{t-1}
 * then hn = RMSNorm(h_t) (eps, no gain), logits = hn W_c + b_c, mean softmax
 * cross-entropy against the next byte over all B*T positions, full
 * backpropagation through time and one momentum update over the flat buffer
 * [E (V x H), W_i (H x 3H), b_i (3H), W_h (H x 3H), b_h (3H), W_c (H x V),
 * b_c (V)] (gru_param_count(V, H) floats).
 * tokens: device int32 [B x (T+1)] (inputs t0..t_{T-1}, targets t1..t_T).
 * params / grads / velocity: device f32; params_lowp: device f16 working
 * copy of params, kept in step by the update (GEMMs read it).  FP16 storage:
 * embedded inputs, the FP16 copy of h_{t-1}, hn, dZ (unscaled p - onehot),
 * the gate gradients; everything else FP32; alpha = 1/(B*T) is applied in
 * the weight, bias and embedding gradients.  loss_out: device f32 [1].
 * Workspace: gru_workspace_bytes(desc); gru_workspace_offsets reports where
 * each stored tensor lives (GE_GRU_WS_* order; rows time-major, t*B + b).
 * Constraints: V <= 4096, 4 <= H <= 4096, H % 4 == 0.
 * ---------------------------------------------------------------------- */
/* recurrence: GE_GRU_AUTO picks the persistent kernels when they apply,
 * GE_GRU_STEPWISE launches a GEMM and a gate kernel per timestep (any size),
 * GE_GRU_PERSISTENT runs each direction of the recurrence as one cooperative
 * launch with the block's slice of W_h resident in LDS ([CAT] "Keep state
 * resident"); it needs B % 16 == 0, B <= 64, H % 256 == 0, H <= 1024,
 * room for all (H / 16) x (B / 16) blocks at once and cooperative launch
 * support, and returns GE_E_UNSUPPORTED otherwise.  Both
 * compute the same quantities; only the recurrent GEMMs' summation order
 * differs. */
#define GE_GRU_AUTO 0
#define GE_GRU_STEPWISE 1
#define GE_GRU_PERSISTENT 2
typedef struct ge_gru_desc {
  int64_t V, H, B, T;
  float eps;
  int32_t recurrence; /* GE_GRU_AUTO / GE_GRU_STEPWISE / GE_GRU_PERSISTENT */
} ge_gru_desc;

typedef struct ge_gru_buffers {
  float *params, *grads, *velocity;
  void *params_lowp;
  void *workspace;
  int64_t workspace_bytes;
} ge_gru_buffers;

enum {
  GE_GRU_WS_INP, GE_GRU_WS_TGT, GE_GRU_WS_X16, GE_GRU_WS_GI, GE_GRU_WS_GH, GE_GRU_WS_H16,
  GE_GRU_WS_HS, GE_GRU_WS_R, GE_GRU_WS_Z, GE_GRU_WS_N, GE_GRU_WS_HN, GE_GRU_WS_RSTD,
  GE_GRU_WS_LOGITS, GE_GRU_WS_G, GE_GRU_WS_ROW_LOSS, GE_GRU_WS_DHN, GE_GRU_WS_DH_OUT,
  GE_GRU_WS_DGH, GE_GRU_WS_DGI, GE_GRU_WS_DX, GE_GRU_WS_ZERO_H, GE_GRU_WS_CARRY,
  GE_GRU_WS_DH_DIR, GE_GRU_WS_COUNT
};

int64_t gru_param_count(int64_t V, int64_t H);
int64_t gru_workspace_bytes(const ge_gru_desc *desc);
int gru_workspace_offsets(const ge_gru_desc *desc, int64_t *offsets, int32_t n);
int gru_lm_train_step(const ge_gru_desc *desc, const ge_gru_buffers *buf, const int32_t *tokens,
                      float lr, float momentum, float *loss_out, ge_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* GEMM_EPILOGUE_H */
