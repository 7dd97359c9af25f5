"""Byte-level GRU language-model training step (oracle side; test infrastructure only).

The recurrent trainer of "The Work Moved Down a Layer" (sections "The Work
Moved Down a Layer" and "From Benchmark to Training Stages": GRU gates, the
full cell and recurrent timesteps, RMSNorm, classifier, softmax cross-entropy,
gradient flow, optimizer), with the recurrent state and gate math kept in FP32
and FP16 only for GEMM inputs ("The Debugging Lesson Was Numerical").  The
pages print no GRU equations; the cell is the standard single-layer GRU with
gate blocks (r, z, n) along the 3H columns and the hidden bias inside the
reset product:

    GI = x_t W_i + b_i                 GH = h_{t-1} W_h + b_h
    r  = sigmoid(GI_r + GH_r)          z  = sigmoid(GI_z + GH_z)
    n  = tanh(GI_n + r * GH_n)         h_t = (1 - z) * n + z * h_{t-1},  h_0 = 0

then RMSNorm (eps, no gain) of every h_t, the classifier Z = hn W_c + b_c,
softmax cross-entropy against the next byte (mean over all B*T positions), full
backpropagation through time and one momentum update over the flat buffer
[E, W_i, b_i, W_h, b_h, W_c, b_c].

Storage plan ``"f16"``: GEMM inputs (embedded x_t, the FP16 copy of h_{t-1},
hn, dZ, the gate gradients, FP16 working copies of E and the weights) are FP16;
GI, GH, r, z, n, h, logits, all backward carries and all gradients FP32.  The
loss gradient dZ is stored unscaled (p - onehot), and the whole backward chain
carries that scale; alpha = 1/(B*T) is applied where the weight, bias and
embedding gradients are formed.  ``"f64"`` rounds nothing.  Rows of every
[B*T x .] matrix are time-major (row = t*B + b).
"""
from __future__ import annotations

import numpy as np

from .numerics import round_fmt
from .ops import gemm_epilogue, colsum, softmax_xent, rmsnorm_fwd, rmsnorm_bwd, sgd_momentum

ORDER = ("E", "W_i", "b_i", "W_h", "b_h", "W_c", "b_c")


def _shapes(H: int, V: int):
    return {"E": (V, H), "W_i": (H, 3 * H), "b_i": (3 * H,), "W_h": (H, 3 * H),
            "b_h": (3 * H,), "W_c": (H, V), "b_c": (V,)}


def gru_param_count(H: int = 1024, V: int = 256) -> int:
    return int(sum(int(np.prod(s)) for s in _shapes(H, V).values()))


def gru_flatten(params: dict) -> np.ndarray:
    return np.concatenate([np.asarray(params[k], dtype=np.float64).ravel() for k in ORDER])


def gru_unflatten(flat, H: int = 1024, V: int = 256) -> dict:
    out, off = {}, 0
    for k in ORDER:
        s = _shapes(H, V)[k]
        n = int(np.prod(s))
        out[k] = np.asarray(flat[off:off + n]).reshape(s)
        off += n
    if off != len(flat):
        raise ValueError("flat buffer size does not match H, V")
    return out


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def gru_gates_fwd(GI, GH, h_prev):
    """Gate arithmetic of one forward timestep (the GRU gate stage of the
    recurrent trainer in "The Work Moved Down a Layer"; standard cell):

        r = sigmoid(GI_r + GH_r);  z = sigmoid(GI_z + GH_z)
        n = tanh(GI_n + r * GH_n); h = (1 - z) * n + z * h_prev

    GI, GH: [B x 3H] with column blocks (r | z | n); returns (r, z, n, h),
    float64, unrounded.
    """
    GI = np.asarray(GI, dtype=np.float64)
    GH = np.asarray(GH, dtype=np.float64)
    h_prev = np.asarray(h_prev, dtype=np.float64)
    H = h_prev.shape[1]
    r = _sigmoid(GI[:, :H] + GH[:, :H])
    z = _sigmoid(GI[:, H:2 * H] + GH[:, H:2 * H])
    n = np.tanh(GI[:, 2 * H:] + r * GH[:, 2 * H:])
    return r, z, n, (1.0 - z) * n + z * h_prev


def gru_gates_bwd(dh, r, z, n, GH_n, h_prev):
    """Gate arithmetic of one backward timestep, by the chain rule through
    gru_gates_fwd, given dh = dL/dh_t (the classifier's part plus the carry
    from t+1):

        dn = dh (1 - z);  dz = dh (h_prev - n);  dh_dir = dh z
        dnh = dn (1 - n^2);  dr = dnh GH_n
        dG_r = dr r (1 - r);  dG_z = dz z (1 - z)
        dGH = [dG_r | dG_z | dnh r];  dGI = [dG_r | dG_z | dnh]

    Returns (dGH, dGI, dh_dir), float64, unrounded.
    """
    dh = np.asarray(dh, dtype=np.float64)
    dn = dh * (1.0 - z)
    dz = dh * (h_prev - n)
    dnh = dn * (1.0 - n * n)
    dgr = dnh * GH_n * r * (1.0 - r)
    dgz = dz * z * (1.0 - z)
    return (np.concatenate([dgr, dgz, dnh * r], axis=1), np.concatenate([dgr, dgz, dnh], axis=1), dh * z)


def gru_step(flat, vel, tokens, H: int, V: int, lr: float, momentum: float,
             eps: float = 1e-6, plan: str = "f16", given=None, update: bool = True):
    """One training step; returns a dict of the stored tensors, loss and update.

    ``given``: optional GPU-stored tensors by name, each replacing the
    oracle's own value wherever later stages consume it: "hs" (the recurrence
    at step t then starts from the given h_{t-1}), "R", "Z", "N", "GH",
    "rstd", "hn", "logits", "G", "dhn", "dh_out", "dGH" (also feeds the carry
    into step t-1), "dGI", "dX".  Every stage is then checked on the inputs
    it actually consumed, without inheriting differences from earlier stages.
    """
    given = given or {}
    lo = "f16" if plan == "f16" else "f64"
    hi = "f32" if plan == "f16" else "f64"
    P = gru_unflatten(flat, H, V)
    Pw = {k: round_fmt(P[k], lo) for k in ("E", "W_i", "W_h", "W_c")}
    tokens = np.asarray(tokens)
    Bn, T1 = tokens.shape
    T = T1 - 1
    inp = tokens[:, :T].T.reshape(-1)            # time-major
    tgt = tokens[:, 1:].T.reshape(-1)
    X = Pw["E"][inp]                             # [T*B x H], FP16 values
    GI, _ = gemm_epilogue(X, Pw["W_i"], "NN", bias=P["b_i"], out_fmt=hi)
    hs = np.zeros((T * Bn, H))
    hprev16 = np.zeros((T * Bn, H))
    R = np.zeros((T * Bn, H)); Zg = np.zeros((T * Bn, H))
    Nn = np.zeros((T * Bn, H)); GHn = np.zeros((T * Bn, H))
    h = np.zeros((Bn, H))
    given_hs = given.get("hs")
    for t in range(T):
        rows = slice(t * Bn, (t + 1) * Bn)
        if given_hs is not None and t > 0:
            h = np.asarray(given_hs[(t - 1) * Bn:t * Bn], dtype=np.float64)
        h16 = round_fmt(h, lo)
        GH, _ = gemm_epilogue(h16, Pw["W_h"], "NN", bias=P["b_h"], out_fmt=hi)
        r, z, n, hn_ = gru_gates_fwd(GI[rows], GH, h)
        R[rows] = round_fmt(r, hi); Zg[rows] = round_fmt(z, hi); Nn[rows] = round_fmt(n, hi)
        GHn[rows] = GH[:, 2 * H:]
        hprev16[rows] = h16
        h = round_fmt(hn_, hi)
        hs[rows] = h
    def use(name, own):
        return np.asarray(given[name], dtype=np.float64) if name in given else own

    hs_u = use("hs", hs)
    hprev16 = np.concatenate([np.zeros((Bn, H)), round_fmt(hs_u[:(T - 1) * Bn], lo)])
    R_u, Z_u, N_u = use("R", R), use("Z", Zg), use("N", Nn)
    GHn_u = use("GH", None)[:, 2 * H:] if "GH" in given else GHn
    hn, rr = rmsnorm_fwd(hs_u, eps, y_fmt=lo, r_fmt=hi)
    hn_u, rr_u = use("hn", hn), use("rstd", rr)
    Zl, _ = gemm_epilogue(hn_u, Pw["W_c"], "NN", bias=P["b_c"], out_fmt=hi)
    loss, row_loss, G, argmax = softmax_xent(use("logits", Zl), tgt, 1.0, lo)
    G_u = use("G", G)
    alpha = 1.0 / (T * Bn)
    dW_c, _ = gemm_epilogue(hn_u, G_u, "TN", alpha, out_fmt=hi)
    db_c = colsum(G_u, alpha, hi)
    dhn, _ = gemm_epilogue(G_u, Pw["W_c"], "NT", out_fmt=hi)
    dh_out, _ = rmsnorm_bwd(hs_u, rr_u, use("dhn", dhn), dx_fmt=hi)
    dh_out_u = use("dh_out", dh_out)
    dGH = np.zeros((T * Bn, 3 * H)); dGI = np.zeros((T * Bn, 3 * H))
    gdGH = given.get("dGH")
    carry = np.zeros((Bn, H))
    for t in range(T - 1, -1, -1):
        rows = slice(t * Bn, (t + 1) * Bn)
        r, z, n, ghn = R_u[rows], Z_u[rows], N_u[rows], GHn_u[rows]
        hp = hs_u[(t - 1) * Bn:t * Bn] if t > 0 else np.zeros((Bn, H))
        dgh, dgi, dh_dir = gru_gates_bwd(dh_out_u[rows] + carry, r, z, n, ghn, hp)
        dh_dir = round_fmt(dh_dir, hi)
        dGH[rows] = round_fmt(dgh, lo)
        dGI[rows] = round_fmt(dgi, lo)
        src = dGH[rows] if gdGH is None else np.asarray(gdGH[rows], dtype=np.float64)
        carry, _ = gemm_epilogue(src, Pw["W_h"], "NT", residual=dh_dir, out_fmt=hi)
    dGH_u, dGI_u = use("dGH", dGH), use("dGI", dGI)
    dW_h, _ = gemm_epilogue(hprev16, dGH_u, "TN", alpha, out_fmt=hi)
    dW_i, _ = gemm_epilogue(X, dGI_u, "TN", alpha, out_fmt=hi)
    db_h = colsum(dGH_u, alpha, hi)
    db_i = colsum(dGI_u, alpha, hi)
    dX, _ = gemm_epilogue(dGI_u, Pw["W_i"], "NT", out_fmt=hi)
    dE = np.zeros((V, H))
    np.add.at(dE, inp, use("dX", dX))
    dE = round_fmt(alpha * dE, hi)
    grads = {"E": dE, "W_i": dW_i, "b_i": db_i, "W_h": dW_h, "b_h": db_h,
             "W_c": dW_c, "b_c": db_c}
    gflat = gru_flatten(grads)
    out = dict(loss=loss, row_loss=row_loss, GI=GI, hs=hs, R=R, Zg=Zg, N=Nn, GHn=GHn,
               hn=hn, rstd=rr, logits=Zl, G=G, argmax=argmax, dhn=dhn, dh_out=dh_out,
               dGH=dGH, dGI=dGI, dX=dX, grads=gflat)
    if update:
        if plan == "f64":
            v2 = momentum * np.asarray(vel, dtype=np.float64) - lr * gflat
            out.update(params=np.asarray(flat, dtype=np.float64) + v2, vel=v2, params_lowp=None)
        else:
            w2, v2, wl = sgd_momentum(flat, gflat, vel, lr, momentum, "f16")
            out.update(params=w2, vel=v2, params_lowp=wl)
    return out


def gru_loss_only(flat, tokens, H: int, V: int, eps: float = 1e-6) -> float:
    """Mean next-byte cross-entropy of the f64 plan (for finite differences)."""
    return gru_step(flat, np.zeros(len(flat)), tokens, H, V, 0.0, 0.0, eps,
                    plan="f64", update=False)["loss"]
