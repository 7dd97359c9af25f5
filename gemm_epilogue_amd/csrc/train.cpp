// mlp_train_step: one SGD-momentum step of a dense ReLU MLP, enqueued as a
// fixed sequence of library kernels on one stream (no host synchronisation).
//
// Equations from "Capstone 5: train a network with your CUDA kernels":
// "The minimum model" (H = ReLU(X W1 + b1), Z = H W2 + b2, stable softmax
// cross-entropy), "Work through the backward pass" (dW = H^T dZ, db =
// sum_rows(dZ), dH = (dZ W^T) * (H > 0)), "Read the worked reference" (bias and
// ReLU in the GEMM epilogue, one flat buffer, one momentum update).  The
// input gradient of the first layer has no consumer and is not formed.
//
// Launches per step for L weight layers: L forward GEMMs, 2 for the loss,
// per layer a TN weight-gradient GEMM and a column sum, L-1 masked NT dgrad
// GEMMs, one update (plus a finishing pass for each split-K GEMM).
#include <cstring>
#include <mutex>
#include <vector>

#include "common.h"

using namespace ge;

namespace {

const int64_t kAlign = 256;
inline int64_t align_up(int64_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct MlpLayout {
  std::vector<int64_t> h_off;  // H_1..H_{L-1}
  int64_t z_off, g_off, dh_off[2], loss_off, gemm_ws_off, gemm_ws, gemm_ws2_off, cs_ws_off, cs_ws, sync_off, total;
  bool head;  // the last layer runs as one fused kernel (mlp_head_kernel)
  int64_t head_off;
};

// The fused output layer applies to FP16 storage, at least one hidden layer
// and a narrow last layer (C <= 16) whose input width fits its LDS copy of W.
bool use_head(const ge_mlp_desc *d, int64_t B) {
  const int nl = d->n_layers;
  return d->storage == GE_F16 && nl >= 2 && head_supported(B, d->dims[nl - 1], d->dims[nl]);
}

bool desc_ok(const ge_mlp_desc *d) {
  if (!d || d->n_layers < 1 || d->n_layers > 64 || !d->dims) return false;
  for (int i = 0; i <= d->n_layers; ++i)
    if (d->dims[i] < 1 || d->dims[i] > (1 << 20)) return false;
  if (d->plan < GE_MLP_AUTO || d->plan > GE_MLP_PERSISTENT) return false;
  return d->storage == GE_F32 || d->storage == GE_F16;
}

// the one-launch step applies to one hidden layer in FP32 of bounded widths
bool persist_shape(const ge_mlp_desc *d, int64_t B) {
  return d->n_layers == 2 && d->storage == GE_F32 && mlp_persist_supported(B, d->dims[0], d->dims[1], d->dims[2]);
}

MlpLayout layout_of(const ge_mlp_desc *d, int64_t B) {
  MlpLayout L;
  const int nl = d->n_layers;
  const int64_t es = d->storage == GE_F32 ? 4 : 2;
  const int64_t C = d->dims[nl];
  int64_t off = 0, maxh = 1;
  for (int l = 1; l < nl; ++l) {
    L.h_off.push_back(off);
    off = align_up(off + B * d->dims[l] * es);
    maxh = std::max<int64_t>(maxh, d->dims[l]);
  }
  L.z_off = off;
  off = align_up(off + B * C * 4);
  L.g_off = off;
  off = align_up(off + B * C * es);
  for (int k = 0; k < 2; ++k) {
    L.dh_off[k] = off;
    off = align_up(off + B * maxh * es);
  }
  L.loss_off = off;
  off = align_up(off + std::max<int64_t>(B, 1) * 4);
  int64_t gws = 0, cws = 0;
  for (int l = 1; l <= nl; ++l) {
    const int64_t din = d->dims[l - 1], dout = d->dims[l];
    const int t = d->storage == GE_F32 ? GE_F32 : GE_F16;
    gws = std::max(gws, gemm_ws_bytes(GE_NN, t, B, dout, din, 0));
    gws = std::max(gws, gemm_ws_bytes(GE_TN, t, din, dout, B, 0));
    if (l > 1) gws = std::max(gws, gemm_ws_bytes(GE_NT, t, B, din, dout, 0));
    cws = std::max(cws, colsum_ws_bytes(B, dout));
    // or the column partials the masked dgrad GEMM's epilogue writes
    if (l > 1) cws = std::max(cws, gemm_colsum_bytes(t, B, din, dout));
  }
  L.gemm_ws_off = off;
  L.gemm_ws = gws;
  off = align_up(off + gws);
  // the weight-gradient GEMMs that run beside the dgrad chain (with the fused
  // output layer and up to three layers) need split-K scratch of their own
  L.head = use_head(d, B);
  L.gemm_ws2_off = off;
  if (L.head && nl <= 3) off = align_up(off + gws);
  L.cs_ws_off = off;
  L.cs_ws = cws;
  off = align_up(off + cws);
  L.head_off = off;
  if (L.head) off = align_up(off + head_ws_bytes(B, d->dims[d->n_layers - 1]));
  L.sync_off = off;  // barrier counter and error word of the persistent step
  off = align_up(off + 8);
  L.total = off;
  return L;
}

// A second stream of the current device (default priority, non-blocking) and
// two events for forking work onto it and joining back, created once per
// device and kept for the process.
int side_stream(hipStream_t *s2, hipEvent_t *fork, hipEvent_t *join) {
  static std::mutex mu;
  static hipStream_t streams[64];
  static hipEvent_t forks[64], joins[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    set_error("mlp_train_step: no current device for the side stream");
    return GE_E_LAUNCH;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!streams[dev]) {
    hipStream_t st = nullptr;
    hipEvent_t ef = nullptr, ej = nullptr;
    if (hipStreamCreateWithFlags(&st, hipStreamNonBlocking) != hipSuccess ||
        hipEventCreateWithFlags(&ef, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&ej, hipEventDisableTiming) != hipSuccess) {
      (void)hipGetLastError();
      set_error("mlp_train_step: cannot create the side stream or its events");
      return GE_E_LAUNCH;
    }
    streams[dev] = st;
    forks[dev] = ef;
    joins[dev] = ej;
  }
  *s2 = streams[dev];
  *fork = forks[dev];
  *join = joins[dev];
  return GE_OK;
}

ge_gemm_args gemm_args(int layout, int t, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda,
                       const void *B, int64_t ldb, void *C, int64_t ldc, int ct) {
  ge_gemm_args a;
  std::memset(&a, 0, sizeof a);
  a.layout = layout;
  a.ab_type = t;
  a.M = M;
  a.N = N;
  a.K = K;
  a.A = A;
  a.lda = lda;
  a.B = B;
  a.ldb = ldb;
  a.alpha = 1.f;
  a.act = GE_ACT_NONE;
  a.act_slope = 0.f;
  a.C = C;
  a.ldc = ldc;
  a.c_type = ct;
  a.aux_type = a.res_type = a.pre_type = GE_F32;
  return a;
}

}  // namespace

#define CHECK(cond, ...)      \
  do {                        \
    if (!(cond)) {            \
      set_error(__VA_ARGS__); \
      return GE_E_INVALID;    \
    }                         \
  } while (0)

#define RUN(call)                 \
  do {                            \
    int _s = (call);              \
    if (_s != GE_OK) return _s;   \
  } while (0)

extern "C" {

int64_t mlp_param_count(int32_t n_layers, const int64_t *dims) {
  if (n_layers < 1 || !dims) return -1;
  int64_t p = 0;
  for (int l = 1; l <= n_layers; ++l) {
    if (dims[l - 1] < 1 || dims[l] < 1) return -1;
    p += dims[l - 1] * dims[l] + dims[l];
  }
  return p;
}

int64_t mlp_workspace_bytes(const ge_mlp_desc *desc, int64_t B) {
  if (!desc_ok(desc) || B < 0) return -1;
  return layout_of(desc, B).total;
}

int mlp_workspace_offsets(const ge_mlp_desc *desc, int64_t B, int64_t *offsets, int32_t n) {
  CHECK(desc_ok(desc) && B >= 0, "mlp_workspace_offsets: bad descriptor or batch");
  CHECK(offsets != nullptr && n >= desc->n_layers + 4, "mlp_workspace_offsets: need n_layers + 4 slots");
  MlpLayout L = layout_of(desc, B);
  int i = 0;
  for (int64_t o : L.h_off) offsets[i++] = o;
  offsets[i++] = L.z_off;
  offsets[i++] = L.g_off;
  offsets[i++] = L.loss_off;
  offsets[i++] = L.dh_off[0];
  offsets[i++] = L.dh_off[1];
  return GE_OK;
}

int mlp_train_step(const ge_mlp_desc *desc, const ge_mlp_buffers *buf, const void *X, const int32_t *labels,
                   int64_t B, float lr, float momentum, float *loss_out, ge_stream_t stream) {
  CHECK(desc_ok(desc), "mlp_train_step: bad descriptor (layers, dims or storage)");
  CHECK(buf != nullptr && buf->params && buf->grads && buf->velocity, "mlp_train_step: missing buffers");
  CHECK(B >= 1 && B < (1 << 24), "mlp_train_step: batch must be >= 1");
  CHECK(X != nullptr && labels != nullptr && loss_out != nullptr, "mlp_train_step: X, labels or loss is NULL");
  const bool f16 = desc->storage == GE_F16;
  CHECK(!f16 || buf->params_lowp != nullptr, "mlp_train_step: FP16 storage needs params_lowp");
  const MlpLayout L = layout_of(desc, B);
  CHECK(buf->workspace != nullptr && buf->workspace_bytes >= L.total,
        "mlp_train_step: workspace needs %lld bytes", (long long)L.total);
  hipStream_t s = (hipStream_t)stream;
  const int nl = desc->n_layers;
  const int64_t *d = desc->dims;
  const int st = f16 ? GE_F16 : GE_F32;
  const int64_t es = f16 ? 2 : 4;
  char *ws = (char *)buf->workspace;
  const int64_t P = mlp_param_count(nl, d);

  const bool fits = persist_shape(desc, B);
  if (desc->plan == GE_MLP_PERSISTENT && !fits) {
    set_error("mlp_train_step: the persistent plan needs one hidden layer in FP32, B <= 128, dims[0] %% 4 == 0 "
              "and <= 1024, dims[1] %% 64 == 0 and <= 512, dims[2] <= 16 and 128 resident blocks");
    return GE_E_UNSUPPORTED;
  }
  if (fits && desc->plan != GE_MLP_CHAIN) {
    MlpPersistArgs a;
    a.X = (const float *)X;
    a.labels = labels;
    a.P = buf->params;
    a.Gr = buf->grads;
    a.V = buf->velocity;
    a.H = (float *)(ws + L.h_off[0]);
    a.Zl = (float *)(ws + L.z_off);
    a.Gz = (float *)(ws + L.g_off);
    a.row_loss = (float *)(ws + L.loss_off);
    a.dH = (float *)(ws + L.dh_off[0]);
    a.loss = loss_out;
    a.sync = (unsigned *)(ws + L.sync_off);
    a.B = (int)B;
    a.D0 = (int)d[0];
    a.D1 = (int)d[1];
    a.C = (int)d[2];
    a.lr = lr;
    a.mu = momentum;
    return mlp_persist_launch(a, s);
  }

  // parameter offsets (elements)
  std::vector<int64_t> w_off(nl + 1), b_off(nl + 1);
  int64_t o = 0;
  for (int l = 1; l <= nl; ++l) {
    w_off[l] = o;
    o += d[l - 1] * d[l];
    b_off[l] = o;
    o += d[l];
  }
  auto wptr = [&](int l) -> const void * {
    return f16 ? (const void *)((const half_t *)buf->params_lowp + w_off[l]) : (const void *)(buf->params + w_off[l]);
  };
  auto hptr = [&](int l) -> void * { return l == 0 ? (void *)X : (void *)(ws + L.h_off[l - 1]); };
  float *Z = (float *)(ws + L.z_off);
  void *G = ws + L.g_off;
  float *row_loss = (float *)(ws + L.loss_off);
  void *gws = L.gemm_ws ? ws + L.gemm_ws_off : nullptr;
  void *cws = L.cs_ws ? ws + L.cs_ws_off : nullptr;

  // forward (with the fused head, the last layer's GEMM is part of it)
  for (int l = 1; l <= (L.head ? nl - 1 : nl); ++l) {
    const bool last = l == nl;
    ge_gemm_args a = gemm_args(GE_NN, st, B, d[l], d[l - 1], hptr(l - 1), d[l - 1], wptr(l), d[l],
                               last ? (void *)Z : hptr(l), d[l], last ? GE_F32 : st);
    a.bias = buf->params + b_off[l];
    a.act = last ? GE_ACT_NONE : GE_ACT_RELU;
    a.workspace = gws;
    a.workspace_bytes = L.gemm_ws;
    RUN(gemm_launch(a, s));
  }
  // loss and dZ ("G"): f32 plan scales by 1/B here, f16 plan in the dW / db epilogues
  const float gscale = f16 ? 1.f : 1.f / (float)B;
  const float alpha = f16 ? 1.f / (float)B : 1.f;
  if (L.head) {
    // logits, loss, dZ, the last bias gradient and the first masked input
    // gradient dH_{L-1} (into the first ping-pong buffer) in one pass
    RUN(head_launch((const half_t *)hptr(nl - 1), B, d[nl - 1], (const half_t *)wptr(nl), buf->params + b_off[nl],
                    d[nl], labels, gscale, alpha, Z, (half_t *)G, row_loss, (half_t *)(ws + L.dh_off[0]),
                    buf->grads + b_off[nl], buf->grads + b_off[nl - 1], loss_out, ws + L.head_off, s));
  } else {
    RUN(xent_launch(Z, B, d[nl], d[nl], labels, gscale, loss_out, row_loss, G, d[nl], st, nullptr, s));
  }
  // backward.  With the fused output layer the weight gradients of layers
  // L .. 2 (and their split-K finishing passes) run on a second stream
  // beside the dgrad chain and the first layer's weight gradient: each waits
  // for the event recorded when its dZ is complete, and the momentum update
  // waits for the second stream.  Both orders compute the same values; the
  // memory-bound passes of one stream fill in beside the other's GEMMs.  Only
  // for up to three layers: with more, the dgrad chain would overwrite a dZ
  // buffer of its ping-pong pair while a weight gradient on the second
  // stream still reads it.  Not under stream capture, where the step stays
  // on the caller's stream.
  hipStream_t s2 = s;
  hipEvent_t ev_fork = nullptr, ev_join = nullptr;
  bool fork = L.head && nl <= 3;
  if (fork) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cs) != hipSuccess) {
      (void)hipGetLastError();
      cs = hipStreamCaptureStatusActive;
    }
    fork = cs == hipStreamCaptureStatusNone;
  }
  if (fork) RUN(side_stream(&s2, &ev_fork, &ev_join));
  void *gws2 = fork && L.gemm_ws ? ws + L.gemm_ws2_off : gws;
  const void *Gl = G;
  int ping = 0;
  int64_t gl_rows = 0;  // > 0: the GEMM that wrote Gl left its column partials in cws
  int seg_rows = 0;     // > 0: db1 still to be formed from cws by the update
  // gradient segments the momentum update forms from partials: db1 from the
  // masked dgrad's column partials, and on two streams the last split-K
  // weight gradient of each stream (its partials stay in that stream's
  // split-K scratch until the update, which replaces the finishing pass)
  SgdSegmentDesc segs[kSgdMaxSegments];
  int nseg = 0;
  for (int l = nl; l >= 1; --l) {
    ge_gemm_args a = gemm_args(GE_TN, st, d[l - 1], d[l], B, hptr(l - 1), d[l - 1], Gl, d[l],
                               buf->grads + w_off[l], d[l], GE_F32);
    a.alpha = alpha;
    const bool side = fork && l >= 2;
    a.workspace = side ? gws2 : gws;
    a.workspace_bytes = L.gemm_ws;
    if (side) {
      if (hipEventRecord(ev_fork, s) != hipSuccess || hipStreamWaitEvent(s2, ev_fork, 0) != hipSuccess) {
        (void)hipGetLastError();
        set_error("mlp_train_step: cannot fork onto the side stream");
        return GE_E_LAUNCH;
      }
    }
    const bool defer = fork && (l == 2 || l == 1);
    int def = 0;
    RUN(gemm_launch(a, side ? s2 : s, nullptr, defer ? &def : nullptr));
    if (def > 0) segs[nseg++] = SgdSegmentDesc{(const float *)a.workspace, w_off[l], d[l - 1] * d[l], def, alpha};
    const bool fused = L.head && l == nl;  // db and dH of this layer came from the head
    // the head also summed the columns of dH_{L-1}, the bias gradient of layer L-1
    if (!(L.head && l >= nl - 1)) {
      if (gl_rows > 0 && l == 1) {
        // no GEMM follows to reuse cws: the momentum update forms db1 itself
        seg_rows = (int)gl_rows;
      } else if (gl_rows > 0)
        RUN(colsum_rows_launch((const float *)cws, gl_rows, d[l], alpha, buf->grads + b_off[l], s));
      else
        RUN(colsum_launch(Gl, B, d[l], d[l], st, alpha, buf->grads + b_off[l], cws, L.cs_ws, s));
    }
    gl_rows = 0;
    if (fused) {
      Gl = ws + L.dh_off[ping];
      ping ^= 1;
    } else if (l > 1) {
      void *dH = ws + L.dh_off[ping];
      ge_gemm_args b = gemm_args(GE_NT, st, B, d[l - 1], d[l], Gl, d[l], wptr(l), d[l], dH, d[l - 1], st);
      b.act = GE_ACT_RELU_MASK_BWD;
      b.aux = hptr(l - 1);
      b.ld_aux = d[l - 1];
      b.aux_type = st;
      b.workspace = gws;
      b.workspace_bytes = L.gemm_ws;
      // the bias gradient of layer l-1 is the column sum of this dZ: let the
      // epilogue sum each tile's columns when the whole output takes its
      // fast path, leaving a few partial rows for the next step
      const int64_t rows = gemm_colsum_rows(b);
      const bool part = rows > 0 && cws != nullptr && rows * d[l - 1] * 4 <= L.cs_ws;
      RUN(gemm_launch(b, s, part ? (float *)cws : nullptr));
      gl_rows = part ? rows : 0;
      Gl = dH;
      ping ^= 1;
    }
  }
  (void)es;
  if (fork) {
    if (hipEventRecord(ev_join, s2) != hipSuccess || hipStreamWaitEvent(s, ev_join, 0) != hipSuccess) {
      (void)hipGetLastError();
      set_error("mlp_train_step: cannot join the side stream");
      return GE_E_LAUNCH;
    }
  }
  if (seg_rows > 0) segs[nseg++] = SgdSegmentDesc{(const float *)cws, b_off[1], d[1], seg_rows, alpha};
  return sgd_launch(buf->params, buf->grads, buf->velocity, lr, momentum, P, f16 ? buf->params_lowp : nullptr,
                    GE_F16, s, segs, nseg);
}

}  // extern "C"
