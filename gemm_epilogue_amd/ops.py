"""torch-tensor wrappers over the C ABI: argument marshalling only.

Every computation runs in libgemm_epilogue.so on the caller's current HIP
stream.  torch is used for device memory (outputs and workspaces allocated
here when the caller passes none) and for the stream handle.
"""
from __future__ import annotations

import ctypes as C

import torch

from ._lib import (ACT, GE_BF16, GE_BWD, GE_F16, GE_F32, GE_FWD, LAYOUT, GemmArgs,
                   MlpBuffers, MlpDesc, RmsnormArgs, check, lib)

_DT = {torch.float32: GE_F32, torch.float16: GE_F16, torch.bfloat16: GE_BF16}
_TD = {v: k for k, v in _DT.items()}


def dtype_code(t: torch.dtype) -> int:
    try:
        return _DT[t]
    except KeyError:
        raise TypeError(f"unsupported dtype {t}") from None


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _ld(t: torch.Tensor) -> int:
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("expected a row-major 2-D tensor (unit column stride)")
    return max(t.stride(0), t.shape[1], 1)


def _workspace(nbytes: int, device, ws):
    if nbytes <= 0:
        return ws
    if ws is not None and ws.numel() * ws.element_size() >= nbytes:
        return ws
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def gemm_shape(A, B, layout: str):
    if layout == "NN":
        return A.shape[0], B.shape[1], A.shape[1]
    if layout == "NT":
        return A.shape[0], B.shape[0], A.shape[1]
    if layout == "TN":
        return A.shape[1], B.shape[1], A.shape[0]
    raise ValueError(layout)


def gemm_workspace_bytes(layout: str, dtype, M, N, K, split_k=0) -> int:
    return int(lib.gemm_workspace_bytes(LAYOUT[layout], dtype_code(dtype), M, N, K, split_k))


class bit_exact:
    """Context manager: the library's bit-exact mode on (or off) inside the
    block, restored after it.  In the mode gemm_bias_act, colsum, the
    RMSNorm passes and sgd_momentum compute their documented binary32
    operation sequences (linear-order sums, one rounding per operation)."""

    def __init__(self, on: bool = True):
        self.on = on

    def __enter__(self):
        self.prev = lib.ge_set_bit_exact(1 if self.on else 0)
        return self

    def __exit__(self, *exc):
        lib.ge_set_bit_exact(self.prev)
        return False


def gemm_bias_act(A, B, layout: str = "NN", *, out=None, out_dtype=torch.float32, alpha=1.0,
                  bias=None, act: str = "none", slope: float = 0.5, aux=None, residual=None,
                  pre=None, workspace=None, split_k: int = 0):
    """C = act(alpha * op(A) op(B) + bias) [+ residual]  (see gemm_bias_act in the header)."""
    M, N, K = gemm_shape(A, B, layout)
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=A.device)
    ws_need = gemm_workspace_bytes(layout, A.dtype, M, N, K, split_k)
    ws = _workspace(ws_need, A.device, workspace)
    a = GemmArgs()
    a.layout = LAYOUT[layout]
    a.ab_type = dtype_code(A.dtype)
    a.M, a.N, a.K = M, N, K
    a.A, a.lda = A.data_ptr(), _ld(A)
    a.B, a.ldb = B.data_ptr(), _ld(B)
    a.alpha = alpha
    a.bias = None if bias is None else bias.data_ptr()
    a.act = ACT[act]
    a.act_slope = slope
    if aux is not None:
        a.aux, a.ld_aux, a.aux_type = aux.data_ptr(), _ld(aux), dtype_code(aux.dtype)
    if residual is not None:
        a.residual, a.ld_res, a.res_type = residual.data_ptr(), _ld(residual), dtype_code(residual.dtype)
    a.C, a.ldc, a.c_type = out.data_ptr(), _ld(out), dtype_code(out.dtype)
    if pre is not None:
        a.pre, a.ld_pre, a.pre_type = pre.data_ptr(), _ld(pre), dtype_code(pre.dtype)
    if ws is not None:
        a.workspace, a.workspace_bytes = ws.data_ptr(), ws.numel() * ws.element_size()
    a.split_k = split_k
    check(lib.gemm_bias_act(C.byref(a), _stream()), "gemm_bias_act")
    return out


def colsum(X, alpha: float = 1.0, *, out=None, accumulate: bool = False, workspace=None):
    """out[n] = alpha * sum_m X[m, n] (f32); with accumulate, added to out."""
    M, N = X.shape
    if out is None:
        out = torch.empty(N, dtype=torch.float32, device=X.device)
    ws = _workspace(int(lib.colsum_workspace_bytes(M, N)), X.device, workspace)
    if accumulate and (out is None or out.dtype != torch.float32):
        raise ValueError("accumulate needs an f32 out tensor")
    check(lib.colsum(_ptr(X), M, N, _ld(X), dtype_code(X.dtype), alpha, _ptr(out), int(accumulate), _ptr(ws),
                     0 if ws is None else ws.numel() * ws.element_size(), _stream()), "colsum")
    return out


def softmax_xent_fwd_bwd(logits, labels, grad_scale: float, *, d_dtype=torch.float32,
                         want_grad=True, want_argmax=True, loss=None, row_loss=None, dlogits=None,
                         argmax=None, bad_label_count=None):
    """Returns (loss_mean[1], row_loss[B], dlogits or None, argmax or None);
    bad_label_count (device int32 [1]) receives the number of labels outside [0, C)."""
    B, Cn = logits.shape
    dev = logits.device
    loss = torch.empty(1, dtype=torch.float32, device=dev) if loss is None else loss
    row_loss = torch.empty(B, dtype=torch.float32, device=dev) if row_loss is None else row_loss
    if want_grad and dlogits is None:
        dlogits = torch.empty((B, Cn), dtype=d_dtype, device=dev)
    if want_argmax and argmax is None:
        argmax = torch.empty(B, dtype=torch.int32, device=dev)
    check(lib.softmax_xent_fwd_bwd(
        _ptr(logits), B, Cn, _ld(logits), _ptr(labels), grad_scale, _ptr(loss), _ptr(row_loss),
        _ptr(dlogits), 0 if dlogits is None else _ld(dlogits),
        GE_F32 if dlogits is None else dtype_code(dlogits.dtype), _ptr(argmax), _ptr(bad_label_count),
        _stream()),
        "softmax_xent_fwd_bwd")
    return loss, row_loss, dlogits, argmax


def rmsnorm_fwd(x, eps: float, *, y_dtype=None, gamma=None, y=None, r=None):
    """Returns (y, r) with r = 1/sqrt(mean x^2 + eps) per row (f32)."""
    rows, D = x.shape
    y = torch.empty((rows, D), dtype=y_dtype or x.dtype, device=x.device) if y is None else y
    r = torch.empty(rows, dtype=torch.float32, device=x.device) if r is None else r
    a = RmsnormArgs()
    a.pass_, a.rows, a.D, a.eps = GE_FWD, rows, D, eps
    a.x, a.ld_x, a.x_type = x.data_ptr(), _ld(x), dtype_code(x.dtype)
    a.gamma = None if gamma is None else gamma.data_ptr()
    a.y, a.ld_y, a.y_type = y.data_ptr(), _ld(y), dtype_code(y.dtype)
    a.r = r.data_ptr()
    check(lib.rmsnorm_fwd_bwd(C.byref(a), _stream()), "rmsnorm_fwd_bwd(fwd)")
    return y, r


def rmsnorm_bwd(x, r, dy, *, dres=None, gamma=None, dx_dtype=None, dx=None, dgamma=None,
                workspace=None):
    """Returns (dx, dgamma or None)."""
    rows, D = x.shape
    dx = torch.empty((rows, D), dtype=dx_dtype or x.dtype, device=x.device) if dx is None else dx
    a = RmsnormArgs()
    a.pass_, a.rows, a.D = GE_BWD, rows, D
    a.x, a.ld_x, a.x_type = x.data_ptr(), _ld(x), dtype_code(x.dtype)
    a.gamma = None if gamma is None else gamma.data_ptr()
    a.r = r.data_ptr()
    a.dy, a.ld_dy, a.dy_type = dy.data_ptr(), _ld(dy), dtype_code(dy.dtype)
    if dres is not None:
        a.dres, a.ld_dres, a.dres_type = dres.data_ptr(), _ld(dres), dtype_code(dres.dtype)
    a.dx, a.ld_dx, a.dx_type = dx.data_ptr(), _ld(dx), dtype_code(dx.dtype)
    if dgamma is not None:
        ws = _workspace(int(lib.rmsnorm_workspace_bytes(rows, D)), x.device, workspace)
        a.dgamma = dgamma.data_ptr()
        a.workspace, a.workspace_bytes = ws.data_ptr(), ws.numel() * ws.element_size()
    check(lib.rmsnorm_fwd_bwd(C.byref(a), _stream()), "rmsnorm_fwd_bwd(bwd)")
    return dx, dgamma


def sgd_momentum(w, g, v, lr: float, momentum: float, w_lowp=None):
    """In place: v = momentum*v - lr*g; w += v; w_lowp = convert(w)."""
    lt = GE_F16 if w_lowp is None else dtype_code(w_lowp.dtype)
    check(lib.sgd_momentum(_ptr(w), _ptr(g), _ptr(v), lr, momentum, w.numel(), _ptr(w_lowp), lt,
                           _stream()), "sgd_momentum")


# ------------------------------------------------------------------ MLP ------

def mlp_param_count(dims) -> int:
    arr = (C.c_int64 * len(dims))(*dims)
    return int(lib.mlp_param_count(len(dims) - 1, arr))


class MLPTrainer:
    """Device buffers of one dense ReLU MLP and a call of mlp_train_step per step.

    params / velocity are f32 flat buffers [W1, b1, W2, b2, ...]; with FP16
    storage an FP16 working copy of the parameters is kept beside them.
    plan: "auto" (the one-launch persistent step where it applies, else the
    launch chain), "chain" or "persistent".
    """

    PLANS = {"auto": 0, "chain": 1, "persistent": 2}

    def __init__(self, dims, batch: int, storage=torch.float32, device="cuda", params=None, plan: str = "auto"):
        self.dims = list(dims)
        self.batch = batch
        self.storage = storage
        self._dims_c = (C.c_int64 * len(dims))(*dims)
        self.desc = MlpDesc(len(dims) - 1, self._dims_c, dtype_code(storage), self.PLANS[plan])
        P = mlp_param_count(dims)
        self.P = P
        self.params = torch.zeros(P, dtype=torch.float32, device=device)
        if params is not None:
            self.params.copy_(params)
        self.grads = torch.zeros(P, dtype=torch.float32, device=device)
        self.velocity = torch.zeros(P, dtype=torch.float32, device=device)
        self.params_lowp = None
        if storage == torch.float16:
            self.params_lowp = torch.empty(P, dtype=torch.float16, device=device)
            params_to_lowp(self.params, self.params_lowp)
        nbytes = int(lib.mlp_workspace_bytes(C.byref(self.desc), batch))
        check(0 if nbytes >= 0 else -1, "mlp_workspace_bytes")
        self.workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
        self.loss = torch.zeros(1, dtype=torch.float32, device=device)
        self.bufs = MlpBuffers(self.params.data_ptr(), self.grads.data_ptr(),
                               self.velocity.data_ptr(),
                               None if self.params_lowp is None else self.params_lowp.data_ptr(),
                               self.workspace.data_ptr(), self.workspace.numel())

    def sync_lowp(self):
        if self.params_lowp is not None:
            params_to_lowp(self.params, self.params_lowp)

    def step(self, X, labels, lr: float, momentum: float, batch=None):
        B = X.shape[0] if batch is None else batch
        if B > self.batch:
            raise ValueError("batch larger than the workspace was sized for")
        check(lib.mlp_train_step(C.byref(self.desc), C.byref(self.bufs), _ptr(X), _ptr(labels), B,
                                 lr, momentum, _ptr(self.loss), _stream()), "mlp_train_step")
        return self.loss

    def workspace_views(self, B=None):
        """Views of the stored activations H_1..H_{L-1}, logits Z, dZ, row losses
        and the masked hidden gradients dH_l still held after the step (the
        two gradient buffers alternate, so with more than three layers only
        the last two written survive; the others are None)."""
        B = self.batch if B is None else B
        L = len(self.dims) - 1
        offs = (C.c_int64 * (L + 4))()
        check(lib.mlp_workspace_offsets(C.byref(self.desc), B, offs, L + 4), "mlp_workspace_offsets")
        ws = self.workspace
        es = 2 if self.storage == torch.float16 else 4

        def view(off, rows, cols, dt, size):
            return ws[off:off + rows * cols * size].view(dt).view(rows, cols)

        out = {"H": [view(offs[l - 1], B, self.dims[l], self.storage, es) for l in range(1, L)]}
        Cn = self.dims[-1]
        out["Z"] = view(offs[L - 1], B, Cn, torch.float32, 4)
        out["G"] = view(offs[L], B, Cn, self.storage, es)
        out["row_loss"] = ws[offs[L + 1]:offs[L + 1] + B * 4].view(torch.float32)
        # dH_{L-1} went to buffer 0, dH_{L-2} to buffer 1, dH_{L-3} to buffer 0, ...
        dH = [None] * (L - 1)
        for l in range(L - 1, 0, -1):
            k = (L - 1 - l) % 2
            if L - 1 - l >= (L - 1) - 2:       # among the last two written
                dH[l - 1] = view(offs[L + 2 + k], B, self.dims[l], self.storage, es)
        out["dH"] = dH
        return out


# ------------------------------------------------------------ MLP block ------

def block_workspace_bytes(rows: int, D: int, F: int, dtype=torch.bfloat16) -> int:
    return int(lib.mlp_block_workspace_bytes(rows, D, F, dtype_code(dtype)))


def mlp_block_fwd_bwd(x, w_up, w_down, dy, *, eps: float = 1e-6, slope: float = 0.5, out=None,
                      workspace=None):
    """Transformer MLP block forward + backward (see mlp_block_fwd_bwd in the header).

    Returns a dict of device tensors y, r, n, u, a, du, dn, dx, dW_up, dW_down.
    """
    from ._lib import BlockArgs
    R, D = x.shape
    F = w_up.shape[1]
    dev, t = x.device, x.dtype
    o = out or {}

    def buf(name, shape, dt):
        if name not in o:
            o[name] = torch.empty(shape, dtype=dt, device=dev)
        return o[name]

    for name in ("y", "n", "dx"):
        buf(name, (R, D), t)
    for name in ("u", "a", "du"):
        buf(name, (R, F), t)
    buf("r", (R,), torch.float32)
    buf("dn", (R, D), torch.float32)
    buf("dW_up", (D, F), torch.float32)
    buf("dW_down", (F, D), torch.float32)
    ws = _workspace(block_workspace_bytes(R, D, F, t), dev, workspace)
    a = BlockArgs(R, D, F, eps, slope, dtype_code(t), x.data_ptr(), w_up.data_ptr(),
                  w_down.data_ptr(), dy.data_ptr(), o["y"].data_ptr(), o["r"].data_ptr(),
                  o["n"].data_ptr(), o["u"].data_ptr(), o["a"].data_ptr(), o["du"].data_ptr(),
                  o["dn"].data_ptr(), o["dx"].data_ptr(), o["dW_up"].data_ptr(),
                  o["dW_down"].data_ptr(), None if ws is None else ws.data_ptr(),
                  0 if ws is None else ws.numel())
    for tsr in (x, w_up, w_down, dy):
        if not tsr.is_contiguous():
            raise ValueError("mlp_block_fwd_bwd expects contiguous tensors")
    check(lib.mlp_block_fwd_bwd(C.byref(a), _stream()), "mlp_block_fwd_bwd")
    o["workspace"] = ws
    return o


def mlp_block_fwd_fused(x, w_up, w_down, *, eps: float = 1e-6, slope: float = 0.5, y=None, r=None,
                        n=None, u=None, a=None, workspace=None):
    """The block's forward pass as one kernel (see mlp_block_fwd_fused in the
    header); r, n, u and a are written only when given.  Returns y."""
    from ._lib import BlockFusedArgs
    R, D = x.shape
    F = w_up.shape[1]
    for tsr in (x, w_up, w_down):
        if not tsr.is_contiguous():
            raise ValueError("mlp_block_fwd_fused expects contiguous tensors")
    y = torch.empty((R, D), dtype=x.dtype, device=x.device) if y is None else y
    ws = _workspace(int(lib.mlp_block_fused_workspace_bytes(D, F)), x.device, workspace)
    a = BlockFusedArgs(R, D, F, eps, slope, dtype_code(x.dtype), x.data_ptr(), w_up.data_ptr(), w_down.data_ptr(),
                       y.data_ptr(), _ptr(r), _ptr(n), _ptr(u), _ptr(a), _ptr(ws),
                       0 if ws is None else ws.numel() * ws.element_size())
    check(lib.mlp_block_fwd_fused(C.byref(a), _stream()), "mlp_block_fwd_fused")
    return y


# ------------------------------------------------------- GRU language model ------

def embedding_gather(table, idx, *, out=None, out_dtype=None):
    V, H = table.shape
    n = idx.numel()
    out = torch.empty((n, H), dtype=out_dtype or table.dtype, device=table.device) if out is None else out
    check(lib.embedding_gather(_ptr(table), V, H, _ld(table), dtype_code(table.dtype), _ptr(idx), n,
                               _ptr(out), _ld(out), dtype_code(out.dtype), _stream()), "embedding_gather")
    return out


def embedding_grad(dX, idx, V: int, alpha: float = 1.0, *, out=None, workspace=None):
    n, H = dX.shape
    out = torch.empty((V, H), dtype=torch.float32, device=dX.device) if out is None else out
    ws = _workspace(int(lib.embedding_grad_workspace_bytes(n, V)), dX.device, workspace)
    check(lib.embedding_grad(_ptr(dX), _ld(dX), dtype_code(dX.dtype), _ptr(idx), n, V, H, alpha,
                             _ptr(out), _ld(out), _ptr(ws), 0 if ws is None else ws.numel(), _stream()),
          "embedding_grad")
    return out


def params_to_lowp(w, w_lowp):
    """w_lowp = convert(w), round to nearest even (the GEMMs' working copy)."""
    if w.dtype != torch.float32 or w_lowp.numel() != w.numel():
        raise ValueError("params_to_lowp: f32 source and a working copy of the same size")
    check(lib.params_to_lowp(_ptr(w), _ptr(w_lowp), w.numel(), dtype_code(w_lowp.dtype), _stream()),
          "params_to_lowp")
    return w_lowp


def gru_gates_fwd(GI, GH, h_prev, *, r=None, z=None, n=None, h=None, h_f16=None):
    """One GRU timestep's gates (see gru_gates_fwd in the header); h_prev None = h_0 = 0.
    Returns (r, z, n, h, h_f16)."""
    B, H3 = GI.shape
    H = H3 // 3
    dev = GI.device

    def mk(t, dt=torch.float32):
        return torch.empty((B, H), dtype=dt, device=dev) if t is None else t

    r, z, n, h = mk(r), mk(z), mk(n), mk(h)
    check(lib.gru_gates_fwd(_ptr(GI), _ptr(GH), _ptr(h_prev), B, H, _ptr(r), _ptr(z), _ptr(n), _ptr(h),
                            _ptr(h_f16), _stream()), "gru_gates_fwd")
    return r, z, n, h, h_f16


def gru_gates_bwd(dh_out, carry, r, z, n, GH, h_prev, *, dGH=None, dGI=None, dh_dir=None):
    """One GRU timestep's gate backward (see gru_gates_bwd in the header); carry or
    h_prev None = 0.  Returns (dGH f16, dGI f16, dh_dir f32)."""
    B, H = dh_out.shape
    dev = dh_out.device
    dGH = torch.empty((B, 3 * H), dtype=torch.float16, device=dev) if dGH is None else dGH
    dGI = torch.empty((B, 3 * H), dtype=torch.float16, device=dev) if dGI is None else dGI
    dh_dir = torch.empty((B, H), dtype=torch.float32, device=dev) if dh_dir is None else dh_dir
    check(lib.gru_gates_bwd(_ptr(dh_out), _ptr(carry), _ptr(r), _ptr(z), _ptr(n), _ptr(GH), _ptr(h_prev), B, H,
                            _ptr(dGH), _ptr(dGI), _ptr(dh_dir), _stream()), "gru_gates_bwd")
    return dGH, dGI, dh_dir


def gru_param_count(V: int, H: int) -> int:
    return int(lib.gru_param_count(V, H))


class GRUTrainer:
    """Device buffers of the byte-level GRU LM and one gru_lm_train_step per call.

    Flat f32 parameters [E, W_i, b_i, W_h, b_h, W_c, b_c] with an FP16
    working copy that the update keeps in step.
    """

    def __init__(self, V: int, H: int, B: int, T: int, eps: float = 1e-6, device="cuda", params=None,
                 recurrence: str = "auto"):
        from ._lib import GRU_WS, GruBuffers, GruDesc
        self.V, self.H, self.B, self.T = V, H, B, T
        self.desc = GruDesc(V, H, B, T, eps, {"auto": 0, "stepwise": 1, "persistent": 2}[recurrence])
        P = gru_param_count(V, H)
        self.P = P
        self.params = torch.zeros(P, dtype=torch.float32, device=device)
        if params is not None:
            self.params.copy_(params)
        self.grads = torch.zeros(P, dtype=torch.float32, device=device)
        self.velocity = torch.zeros(P, dtype=torch.float32, device=device)
        self.params_lowp = torch.empty(P, dtype=torch.float16, device=device)
        params_to_lowp(self.params, self.params_lowp)
        nbytes = int(lib.gru_workspace_bytes(C.byref(self.desc)))
        if nbytes < 0:
            raise ValueError("bad GRU sizes (V <= 4096, 4 <= H <= 4096, H % 4 == 0)")
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.loss = torch.zeros(1, dtype=torch.float32, device=device)
        self.bufs = GruBuffers(self.params.data_ptr(), self.grads.data_ptr(), self.velocity.data_ptr(),
                               self.params_lowp.data_ptr(), self.workspace.data_ptr(), nbytes)
        offs = (C.c_int64 * len(GRU_WS))()
        check(lib.gru_workspace_offsets(C.byref(self.desc), offs, len(GRU_WS)), "gru_workspace_offsets")
        self._offs = dict(zip(GRU_WS, list(offs)))

    def step(self, tokens, lr: float, momentum: float):
        if tokens.dtype != torch.int32 or tuple(tokens.shape) != (self.B, self.T + 1):
            raise ValueError("tokens must be int32 [B x (T+1)]")
        check(lib.gru_lm_train_step(C.byref(self.desc), C.byref(self.bufs), _ptr(tokens), lr, momentum,
                                    _ptr(self.loss), _stream()), "gru_lm_train_step")
        return self.loss

    def view(self, name: str):
        """A stored tensor of the last step (rows time-major, t*B + b)."""
        NT, H, V, B = self.B * self.T, self.H, self.V, self.B
        shapes = {"INP": ((NT,), torch.int32), "TGT": ((NT,), torch.int32),
                  "X16": ((NT, H), torch.float16), "GI": ((NT, 3 * H), torch.float32),
                  "GH": ((NT, 3 * H), torch.float32), "H16": ((NT + B, H), torch.float16),
                  "HS": ((NT, H), torch.float32), "R": ((NT, H), torch.float32),
                  "Z": ((NT, H), torch.float32), "N": ((NT, H), torch.float32),
                  "HN": ((NT, H), torch.float16), "RSTD": ((NT,), torch.float32),
                  "LOGITS": ((NT, V), torch.float32), "G": ((NT, V), torch.float16),
                  "ROW_LOSS": ((NT,), torch.float32), "DHN": ((NT, H), torch.float32),
                  "DH_OUT": ((NT, H), torch.float32), "DGH": ((NT, 3 * H), torch.float16),
                  "DGI": ((NT, 3 * H), torch.float16), "DX": ((NT, H), torch.float32)}
        shape, dt = shapes[name]
        n = 1
        for s in shape:
            n *= s
        es = torch.tensor([], dtype=dt).element_size()
        o = self._offs[name]
        return self.workspace[o:o + n * es].view(dt).view(shape)
