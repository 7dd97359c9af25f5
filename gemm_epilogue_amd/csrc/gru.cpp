// gru_lm_train_step: one training step of a byte-level GRU language model,
// enqueued on one stream: embedding gather, the input projection for all
// timesteps, the recurrence (one GEMM and one gate kernel per timestep),
// RMSNorm, classifier, softmax cross-entropy, classifier backward, RMSNorm
// backward, backpropagation through time (one gate kernel and one dgrad GEMM
// per timestep), the batched weight/bias/embedding gradients and one momentum
// update over the flat parameter buffer [E, W_i, b_i, W_h, b_h, W_c, b_c].
//
// "The Work Moved Down a Layer": the trainer's shader family (GEMM, GRU gates,
// RMSNorm, softmax cross-entropy, gradient reduction, optimizer; section "The
// Work Moved Down a Layer"), state kept resident across timesteps ("Keep state
// resident"), FP32 recurrent state and normalisation statistics with FP16 only
// for GEMM inputs ("The Debugging Lesson Was Numerical").
//
// Scaling: dZ is stored unscaled (p - onehot) in FP16; the backward chain
// carries that scale and alpha = 1/(B*T) is applied where weight, bias and
// embedding gradients are formed.  Rows of every [B*T x .] matrix are
// time-major (row = t*B + b).
#include <cstring>
#include <vector>

#include "common.h"

namespace ge {
int tokens_time_major_launch(const int32_t *tok, int B, int T, int32_t *inp, int32_t *tgt, hipStream_t s);
int fill_zero_launch(void *p, int64_t bytes, hipStream_t s);
int embedding_gather_launch(const void *table, int64_t V, int64_t H, int64_t ldt, int tt, const int32_t *idx,
                            int64_t n, void *out, int64_t ldo, int ot, hipStream_t s);
int64_t embedding_grad_ws_bytes(int64_t n, int64_t V);
int embedding_grad_launch(const void *dX, int64_t ldx, int xt, const int32_t *idx, int64_t n, int64_t V,
                          int64_t H, float alpha, float *dE, int64_t lde, void *ws, int64_t ws_bytes,
                          hipStream_t s);
int gru_fwd_launch(const float *GI, const float *GH, const float *hp, int B, int H, float *R, float *Z, float *N,
                   float *h, half_t *h16, hipStream_t s);
int gru_bwd_launch(const float *dh_out, const float *carry, const float *R, const float *Z, const float *N,
                   const float *GH, const float *hp, int B, int H, half_t *dGH, half_t *dGI, float *dh_dir,
                   hipStream_t s);
bool gru_persist_supported(int64_t B, int64_t H);
int64_t gru_sync_bytes();
int gru_rec_fwd_launch(const float *GI, const half_t *Wh, const float *bh, int B, int H, int T, float *GH, float *R,
                       float *Z, float *N, float *HS, half_t *H16, unsigned *sync, hipStream_t s);
int gru_rec_bwd_launch(const float *dh_out, const half_t *Wh, const float *R, const float *Z, const float *N,
                       const float *GH, const float *HS, int B, int H, int T, half_t *dGH, half_t *dGI, unsigned *sync,
                       hipStream_t s);
}  // namespace ge

using namespace ge;

#define CHECK(cond, ...)      \
  do {                        \
    if (!(cond)) {            \
      set_error(__VA_ARGS__); \
      return GE_E_INVALID;    \
    }                         \
  } while (0)

#define RUN(call)               \
  do {                          \
    int _s = (call);            \
    if (_s != GE_OK) return _s; \
  } while (0)

namespace {

const int64_t kAlign = 256;
inline int64_t align_up(int64_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool desc_ok(const ge_gru_desc *d) {
  return d && d->V >= 1 && d->V <= 4096 && d->H >= 4 && d->H <= 4096 && d->H % 4 == 0 && d->B >= 1 &&
         d->T >= 1 && d->B * d->T < (1 << 24) && d->eps >= 0.f && d->recurrence >= GE_GRU_AUTO &&
         d->recurrence <= GE_GRU_PERSISTENT;
}

// byte offsets of every workspace region, in GE_GRU_WS_* order
struct GruLayout {
  int64_t off[GE_GRU_WS_COUNT];
  int64_t gemm_off, gemm_ws, cs_off, cs_ws, emb_off, emb_ws, sync_off, total;
};

GruLayout layout_of(const ge_gru_desc *d) {
  const int64_t B = d->B, T = d->T, H = d->H, V = d->V, NT = B * T, H3 = 3 * H;
  const int64_t sz[GE_GRU_WS_COUNT] = {
      NT * 4,            // INP
      NT * 4,            // TGT
      NT * H * 2,        // X16
      NT * H3 * 4,       // GI
      NT * H3 * 4,       // GH
      (NT + B) * H * 2,  // H16 (block 0 = h_0 = 0)
      NT * H * 4,        // HS
      NT * H * 4,        // R
      NT * H * 4,        // Z
      NT * H * 4,        // N
      NT * H * 2,        // HN
      NT * 4,            // RSTD
      NT * V * 4,        // LOGITS
      NT * V * 2,        // G
      NT * 4,            // ROW_LOSS
      NT * H * 4,        // DHN
      NT * H * 4,        // DH_OUT
      NT * H3 * 2,       // DGH
      NT * H3 * 2,       // DGI
      NT * H * 4,        // DX
      B * H * 4,         // ZERO_H
      2 * B * H * 4,     // CARRY (two buffers)
      B * H * 4,         // DH_DIR
  };
  GruLayout L;
  int64_t o = 0;
  for (int i = 0; i < GE_GRU_WS_COUNT; ++i) {
    L.off[i] = o;
    o = align_up(o + sz[i]);
  }
  const int t = GE_F16;
  int64_t g = 0;
  g = std::max(g, gemm_ws_bytes(GE_NN, t, NT, H3, H, 0));  // input projection
  g = std::max(g, gemm_ws_bytes(GE_NN, t, B, H3, H, 0));   // recurrent GEMM
  g = std::max(g, gemm_ws_bytes(GE_NN, t, NT, V, H, 0));   // classifier
  g = std::max(g, gemm_ws_bytes(GE_TN, t, H, V, NT, 0));   // dW_c
  g = std::max(g, gemm_ws_bytes(GE_NT, t, NT, H, V, 0));   // d(hn)
  g = std::max(g, gemm_ws_bytes(GE_NT, t, B, H, H3, 0));   // carry
  g = std::max(g, gemm_ws_bytes(GE_TN, t, H, H3, NT, 0));  // dW_h, dW_i
  g = std::max(g, gemm_ws_bytes(GE_NT, t, NT, H, H3, 0));  // dX
  L.gemm_off = o;
  L.gemm_ws = g;
  o = align_up(o + g);
  L.cs_off = o;
  L.cs_ws = std::max(colsum_ws_bytes(NT, V), colsum_ws_bytes(NT, H3));
  o = align_up(o + L.cs_ws);
  L.emb_off = o;
  L.emb_ws = embedding_grad_ws_bytes(NT, V);
  o = align_up(o + L.emb_ws);
  L.sync_off = o;  // barrier counters and error word of the persistent recurrence
  o = align_up(o + gru_sync_bytes());
  L.total = o;
  return L;
}

ge_gemm_args gargs(int layout, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B,
                   int64_t ldb, void *C, int64_t ldc, int ct, void *ws, int64_t wsb) {
  ge_gemm_args a;
  std::memset(&a, 0, sizeof a);
  a.layout = layout;
  a.ab_type = GE_F16;
  a.M = M;
  a.N = N;
  a.K = K;
  a.A = A;
  a.lda = lda;
  a.B = B;
  a.ldb = ldb;
  a.alpha = 1.f;
  a.C = C;
  a.ldc = ldc;
  a.c_type = ct;
  a.aux_type = a.res_type = a.pre_type = GE_F32;
  a.workspace = ws;
  a.workspace_bytes = wsb;
  return a;
}

}  // namespace

extern "C" {

int embedding_gather(const void *table, int64_t V, int64_t H, int64_t ld_table, int32_t type,
                     const int32_t *idx, int64_t n, void *out, int64_t ld_out, int32_t out_type,
                     ge_stream_t stream) {
  CHECK(V >= 1 && H >= 0 && n >= 0 && V < (1 << 30) && H < (1 << 30) && n < (1 << 30),
        "embedding_gather: bad sizes");
  CHECK(dtype_ok(type) && dtype_ok(out_type), "embedding_gather: unknown type");
  if (n == 0 || H == 0) return GE_OK;
  CHECK(table && idx && out && ld_table >= H && ld_out >= H, "embedding_gather: NULL pointer or ld < H");
  return embedding_gather_launch(table, V, H, ld_table, type, idx, n, out, ld_out, out_type, (hipStream_t)stream);
}

int64_t embedding_grad_workspace_bytes(int64_t n, int64_t V) {
  if (n < 0 || V < 0) return -1;
  return embedding_grad_ws_bytes(n, V);
}

int embedding_grad(const void *dX, int64_t ld_dx, int32_t dx_type, const int32_t *idx, int64_t n, int64_t V,
                   int64_t H, float alpha, float *dE, int64_t ld_de, void *workspace, int64_t workspace_bytes,
                   ge_stream_t stream) {
  CHECK(V >= 0 && H >= 0 && n >= 0 && V <= 16384 && H < (1 << 30) && n < (1 << 30),
        "embedding_grad: bad sizes (V <= 16384)");
  CHECK(dtype_ok(dx_type), "embedding_grad: unknown type");
  if (V == 0 || H == 0) return GE_OK;
  CHECK(dE && ld_de >= H && (n == 0 || (dX && idx && ld_dx >= H)), "embedding_grad: NULL pointer or ld < H");
  return embedding_grad_launch(dX, ld_dx, dx_type, idx, n, V, H, alpha, dE, ld_de, workspace, workspace_bytes,
                               (hipStream_t)stream);
}

int gru_gates_fwd(const float *GI, const float *GH, const float *h_prev, int64_t B, int64_t H, float *r, float *z,
                  float *n, float *h, void *h_f16, ge_stream_t stream) {
  CHECK(B >= 0 && H >= 0 && B * H < ((int64_t)1 << 31) && H % 4 == 0, "gru_gates_fwd: bad sizes (H %% 4 == 0)");
  if (B == 0 || H == 0) return GE_OK;
  CHECK(GI && GH && r && z && n && h, "gru_gates_fwd: NULL pointer");
  const void *ps[] = {GI, GH, h_prev, r, z, n, h};
  for (const void *p : ps) CHECK((uintptr_t)p % 16 == 0, "gru_gates_fwd: pointers must be 16-byte aligned");
  CHECK((uintptr_t)h_f16 % 8 == 0, "gru_gates_fwd: h_f16 must be 8-byte aligned");
  return gru_fwd_launch(GI, GH, h_prev, (int)B, (int)H, r, z, n, h, (half_t *)h_f16, (hipStream_t)stream);
}

int gru_gates_bwd(const float *dh_out, const float *carry, const float *r, const float *z, const float *n,
                  const float *GH, const float *h_prev, int64_t B, int64_t H, void *dGH, void *dGI, float *dh_dir,
                  ge_stream_t stream) {
  CHECK(B >= 0 && H >= 0 && B * H < ((int64_t)1 << 31) && H % 4 == 0, "gru_gates_bwd: bad sizes (H %% 4 == 0)");
  if (B == 0 || H == 0) return GE_OK;
  CHECK(dh_out && r && z && n && GH && dGH && dGI && dh_dir, "gru_gates_bwd: NULL pointer");
  const void *ps[] = {dh_out, carry, r, z, n, GH, h_prev, dh_dir};
  for (const void *p : ps) CHECK((uintptr_t)p % 16 == 0, "gru_gates_bwd: pointers must be 16-byte aligned");
  CHECK((uintptr_t)dGH % 8 == 0 && (uintptr_t)dGI % 8 == 0, "gru_gates_bwd: dGH, dGI must be 8-byte aligned");
  return gru_bwd_launch(dh_out, carry, r, z, n, GH, h_prev, (int)B, (int)H, (half_t *)dGH, (half_t *)dGI, dh_dir,
                        (hipStream_t)stream);
}

int64_t gru_param_count(int64_t V, int64_t H) {
  if (V < 1 || H < 1) return -1;
  return V * H + 2 * (H * 3 * H + 3 * H) + H * V + V;
}

int64_t gru_workspace_bytes(const ge_gru_desc *desc) {
  if (!desc_ok(desc)) return -1;
  return layout_of(desc).total;
}

int gru_workspace_offsets(const ge_gru_desc *desc, int64_t *offsets, int32_t n) {
  CHECK(desc_ok(desc), "gru_workspace_offsets: bad descriptor");
  CHECK(offsets != nullptr && n >= GE_GRU_WS_COUNT, "gru_workspace_offsets: need %d slots", GE_GRU_WS_COUNT);
  GruLayout L = layout_of(desc);
  for (int i = 0; i < GE_GRU_WS_COUNT; ++i) offsets[i] = L.off[i];
  return GE_OK;
}

int gru_lm_train_step(const ge_gru_desc *desc, const ge_gru_buffers *buf, const int32_t *tokens, float lr,
                      float momentum, float *loss_out, ge_stream_t stream) {
  CHECK(desc_ok(desc), "gru_lm_train_step: bad descriptor (V <= 4096, 4 <= H <= 4096 with H %% 4 == 0)");
  CHECK(buf && buf->params && buf->grads && buf->velocity && buf->params_lowp,
        "gru_lm_train_step: missing parameter buffers");
  CHECK(tokens != nullptr && loss_out != nullptr, "gru_lm_train_step: tokens or loss is NULL");
  const GruLayout L = layout_of(desc);
  CHECK(buf->workspace && buf->workspace_bytes >= L.total, "gru_lm_train_step: workspace needs %lld bytes",
        (long long)L.total);
  hipStream_t s = (hipStream_t)stream;
  const int64_t B = desc->B, T = desc->T, H = desc->H, V = desc->V, NT = B * T, H3 = 3 * H;
  const bool persist_ok = gru_persist_supported(B, H);
  if (desc->recurrence == GE_GRU_PERSISTENT && !persist_ok) {
    set_error("gru_lm_train_step: the persistent recurrence needs B %% 16 == 0, B <= 64, H %% 256 == 0, "
              "H <= 1536 and cooperative launch");
    return GE_E_UNSUPPORTED;
  }
  const bool persist = persist_ok && desc->recurrence != GE_GRU_STEPWISE;
  char *ws = (char *)buf->workspace;
  auto W = [&](int i) { return (void *)(ws + L.off[i]); };
  int32_t *inp = (int32_t *)W(GE_GRU_WS_INP), *tgt = (int32_t *)W(GE_GRU_WS_TGT);
  half_t *X16 = (half_t *)W(GE_GRU_WS_X16), *H16 = (half_t *)W(GE_GRU_WS_H16), *HN = (half_t *)W(GE_GRU_WS_HN);
  half_t *G = (half_t *)W(GE_GRU_WS_G), *dGH = (half_t *)W(GE_GRU_WS_DGH), *dGI = (half_t *)W(GE_GRU_WS_DGI);
  float *GI = (float *)W(GE_GRU_WS_GI), *GH = (float *)W(GE_GRU_WS_GH), *HS = (float *)W(GE_GRU_WS_HS);
  float *R = (float *)W(GE_GRU_WS_R), *Z = (float *)W(GE_GRU_WS_Z), *N = (float *)W(GE_GRU_WS_N);
  float *RSTD = (float *)W(GE_GRU_WS_RSTD), *LOG = (float *)W(GE_GRU_WS_LOGITS);
  float *ROWL = (float *)W(GE_GRU_WS_ROW_LOSS), *DHN = (float *)W(GE_GRU_WS_DHN);
  float *DHO = (float *)W(GE_GRU_WS_DH_OUT), *DX = (float *)W(GE_GRU_WS_DX);
  float *ZH = (float *)W(GE_GRU_WS_ZERO_H), *CARRY = (float *)W(GE_GRU_WS_CARRY);
  float *DHD = (float *)W(GE_GRU_WS_DH_DIR);
  void *gws = L.gemm_ws ? ws + L.gemm_off : nullptr;  // split-K partials
  void *cws = L.cs_ws ? ws + L.cs_off : nullptr;      // column-sum partials

  // parameter offsets (elements) in [E, W_i, b_i, W_h, b_h, W_c, b_c]
  const int64_t oE = 0, oWi = V * H, obi = oWi + H * H3, oWh = obi + H3, obh = oWh + H * H3, oWc = obh + H3,
                obc = oWc + H * V, P = obc + V;
  const half_t *lp = (const half_t *)buf->params_lowp;
  const float *pm = buf->params;
  float *gr = buf->grads;
  const float alpha = 1.f / (float)NT;

  RUN(tokens_time_major_launch(tokens, (int)B, (int)T, inp, tgt, s));
  RUN(fill_zero_launch(H16, B * H * 2, s));
  RUN(fill_zero_launch(ZH, B * H * 4, s));
  RUN(fill_zero_launch(CARRY, B * H * 4, s));
  RUN(embedding_gather_launch(lp + oE, V, H, H, GE_F16, inp, NT, X16, H, GE_F16, s));
  // input projection for every timestep: GI = X W_i + b_i
  ge_gemm_args g = gargs(GE_NN, NT, H3, H, X16, H, lp + oWi, H3, GI, H3, GE_F32, gws, L.gemm_ws);
  g.bias = pm + obi;
  RUN(gemm_launch(g, s));
  // recurrence
  unsigned *sync = (unsigned *)(ws + L.sync_off);
  if (persist)
    RUN(gru_rec_fwd_launch(GI, lp + oWh, pm + obh, (int)B, (int)H, (int)T, GH, R, Z, N, HS, H16, sync, s));
  for (int64_t t = 0; !persist && t < T; ++t) {
    float *GHt = GH + t * B * H3;
    g = gargs(GE_NN, B, H3, H, H16 + t * B * H, H, lp + oWh, H3, GHt, H3, GE_F32, gws, L.gemm_ws);
    g.bias = pm + obh;
    RUN(gemm_launch(g, s));
    const float *hp = t == 0 ? ZH : HS + (t - 1) * B * H;
    RUN(gru_fwd_launch(GI + t * B * H3, GHt, hp, (int)B, (int)H, R + t * B * H, Z + t * B * H, N + t * B * H,
                       HS + t * B * H, H16 + (t + 1) * B * H, s));
  }
  // RMSNorm, classifier, loss
  ge_rmsnorm_args rn;
  std::memset(&rn, 0, sizeof rn);
  rn.pass = GE_FWD;
  rn.rows = NT;
  rn.D = H;
  rn.eps = desc->eps;
  rn.x = HS;
  rn.ld_x = H;
  rn.x_type = GE_F32;
  rn.y = HN;
  rn.ld_y = H;
  rn.y_type = GE_F16;
  rn.r = RSTD;
  RUN(rmsnorm_launch(rn, s));
  g = gargs(GE_NN, NT, V, H, HN, H, lp + oWc, V, LOG, V, GE_F32, gws, L.gemm_ws);
  g.bias = pm + obc;
  RUN(gemm_launch(g, s));
  RUN(xent_launch(LOG, NT, V, V, tgt, 1.f, loss_out, ROWL, G, V, GE_F16, nullptr, s));
  // classifier backward
  g = gargs(GE_TN, H, V, NT, HN, H, G, V, gr + oWc, V, GE_F32, gws, L.gemm_ws);
  g.alpha = alpha;
  RUN(gemm_launch(g, s));
  RUN(colsum_launch(G, NT, V, V, GE_F16, alpha, gr + obc, cws, L.cs_ws, s));
  g = gargs(GE_NT, NT, H, V, G, V, lp + oWc, V, DHN, H, GE_F32, gws, L.gemm_ws);
  RUN(gemm_launch(g, s));
  std::memset(&rn, 0, sizeof rn);
  rn.pass = GE_BWD;
  rn.rows = NT;
  rn.D = H;
  rn.eps = desc->eps;
  rn.x = HS;
  rn.ld_x = H;
  rn.x_type = GE_F32;
  rn.r = RSTD;
  rn.dy = DHN;
  rn.ld_dy = H;
  rn.dy_type = GE_F32;
  rn.dx = DHO;
  rn.ld_dx = H;
  rn.dx_type = GE_F32;
  RUN(rmsnorm_launch(rn, s));
  // backpropagation through time
  int cur = 0;  // CARRY[cur] holds the gradient flowing into h_t from t+1
  if (persist)
    RUN(gru_rec_bwd_launch(DHO, lp + oWh, R, Z, N, GH, HS, (int)B, (int)H, (int)T, dGH, dGI, sync, s));
  for (int64_t t = T - 1; !persist && t >= 0; --t) {
    float *carry_in = CARRY + cur * B * H, *carry_out = CARRY + (cur ^ 1) * B * H;
    const float *hp = t == 0 ? ZH : HS + (t - 1) * B * H;
    RUN(gru_bwd_launch(DHO + t * B * H, carry_in, R + t * B * H, Z + t * B * H, N + t * B * H, GH + t * B * H3,
                       hp, (int)B, (int)H, dGH + t * B * H3, dGI + t * B * H3, DHD, s));
    if (t > 0) {
      g = gargs(GE_NT, B, H, H3, dGH + t * B * H3, H3, lp + oWh, H3, carry_out, H, GE_F32, gws, L.gemm_ws);
      g.residual = DHD;
      g.ld_res = H;
      g.res_type = GE_F32;
      RUN(gemm_launch(g, s));
      cur ^= 1;
    }
  }
  // batched weight, bias and embedding gradients
  g = gargs(GE_TN, H, H3, NT, H16, H, dGH, H3, gr + oWh, H3, GE_F32, gws, L.gemm_ws);
  g.alpha = alpha;
  RUN(gemm_launch(g, s));
  g = gargs(GE_TN, H, H3, NT, X16, H, dGI, H3, gr + oWi, H3, GE_F32, gws, L.gemm_ws);
  g.alpha = alpha;
  RUN(gemm_launch(g, s));
  RUN(colsum_launch(dGH, NT, H3, H3, GE_F16, alpha, gr + obh, cws, L.cs_ws, s));
  RUN(colsum_launch(dGI, NT, H3, H3, GE_F16, alpha, gr + obi, cws, L.cs_ws, s));
  g = gargs(GE_NT, NT, H, H3, dGI, H3, lp + oWi, H3, DX, H, GE_F32, gws, L.gemm_ws);
  RUN(gemm_launch(g, s));
  RUN(embedding_grad_launch(DX, H, GE_F32, inp, NT, V, H, alpha, gr + oE, H, ws + L.emb_off, L.emb_ws, s));
  return sgd_launch(buf->params, buf->grads, buf->velocity, lr, momentum, P, buf->params_lowp, GE_F16, s);
}

}  // extern "C"
