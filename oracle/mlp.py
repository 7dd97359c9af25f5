"""Dense ReLU MLP training step, float64 (oracle side; test infrastructure only).

Model, equations and update follow "Capstone 5: train a network with your CUDA
kernels": H = ReLU(X W1 + b1), Z = H W2 + b2, stable softmax cross-entropy
("The minimum model"); dW2 = H^T dZ, db2 = sum_rows(dZ), dH = (dZ W2^T)*(H>0),
dW1 = X^T dH, db1 = sum_rows(dH) ("Work through the backward pass"); one flat
buffer holding all parameter tensors and one momentum update over it ("Read
the worked reference").  Deeper nets repeat the hidden layer.

Storage plans (where each tensor is rounded, mirroring the GPU path):

* ``"f32"`` -- everything FP32; dZ carries the 1/B of the mean loss.
* ``"f16"`` -- X, the GEMM working copies of the weights, hidden activations,
  dZ and dH are FP16; logits, weight/bias gradients, master weights and
  velocity FP32.  dZ is stored *unscaled* (p - onehot) and 1/B is applied in
  the weight- and bias-gradient epilogues instead (a static loss scale of B,
  which keeps FP16 gradients out of the subnormal range).
* ``"f64"`` -- no rounding at all (for finite-difference checks).

Flat layout: [W1, b1, W2, b2, ...], W_l row-major [d_{l-1} x d_l].
"""
from __future__ import annotations

import numpy as np

from .numerics import round_fmt
from .ops import gemm_epilogue, colsum, softmax_xent, sgd_momentum


def mlp_param_count(dims) -> int:
    """Number of parameters of the dense net with layer widths ``dims``."""
    return int(sum(a * b + b for a, b in zip(dims[:-1], dims[1:])))


def mlp_unflatten(flat, dims):
    """Views [(W1, b1), (W2, b2), ...] into a flat parameter vector."""
    flat = np.asarray(flat)
    out, off = [], 0
    for a, b in zip(dims[:-1], dims[1:]):
        W = flat[off:off + a * b].reshape(a, b)
        off += a * b
        bias = flat[off:off + b]
        off += b
        out.append((W, bias))
    if off != flat.size:
        raise ValueError("flat buffer size does not match dims")
    return out


def _plan(plan: str):
    if plan == "f32":
        return dict(act="f32", gemm_w=None, logits="f32", dz="f32", unscaled=False)
    if plan == "f16":
        return dict(act="f16", gemm_w="f16", logits="f32", dz="f16", unscaled=True)
    if plan == "f64":
        return dict(act="f64", gemm_w=None, logits="f64", dz="f64", unscaled=False)
    raise ValueError(plan)


def mlp_forward(params, dims, X, plan: str = "f32", given_H=None):
    """Forward pass; returns (list of stored activations [X, H1, ...], pre-activations, Z).

    ``given_H`` (optional list [H1, ...]) makes layer l read the given stored
    H_{l-1} instead of the oracle's own, so each layer is checked on the
    inputs it actually consumed.
    """
    P = _plan(plan)
    layers = mlp_unflatten(params, dims)
    Hs, pres = [np.asarray(X, dtype=np.float64)], []
    L = len(layers)
    for li, (W, b) in enumerate(layers):
        Wg = round_fmt(W, P["gemm_w"]) if P["gemm_w"] else W
        last = li == L - 1
        inp = Hs[-1] if (given_H is None or li == 0) else np.asarray(given_H[li - 1], np.float64)
        out, pre = gemm_epilogue(inp, Wg, "NN", 1.0, b, "none" if last else "relu",
                                 out_fmt=P["logits"] if last else P["act"], pre_fmt="f64")
        pres.append(pre)
        if last:
            return Hs, pres, out
        Hs.append(out)


def mlp_step(params, vel, dims, X, labels, lr: float, momentum: float,
             plan: str = "f32", mask_hint=None, tie_abs: float = 0.0, given=None):
    """One training step; returns a dict of every stored tensor and the update.

    ``mask_hint``: optional list of the GPU's stored hidden activations
    [H1, H2, ...].  Where the oracle's pre-activation is within ``tie_abs`` of
    zero, the ReLU-mask bit of the backward pass is taken from the hint (both
    bits are correct within the forward rounding error); the number of such
    adopted bits that differ is reported as ``mask_ties``.

    ``given``: optional dict of stored tensors -- "H" [H1, ...], "Z", "G",
    "dH" [dH_1, ...] (dH_l is the masked gradient at H_l) -- each stage then
    starts from the stored inputs it consumed (stage-wise check).  The given
    tensors are inputs only: every returned tensor is the oracle's own value,
    computed from the inputs of its stage.  So "H"[l] is layer l+1's output
    computed from given H_l (X for the first layer), "Z" is computed from the
    given last hidden layer, "argmax" from that own "Z", while "loss",
    "row_loss" and "G" are the loss stage applied to the given "Z" and the
    weight gradients use the given H and G / dH as their operands.
    """
    P = _plan(plan)
    given = given or {}
    X = np.asarray(X, dtype=np.float64)
    B = X.shape[0]
    layers = mlp_unflatten(params, dims)
    L = len(layers)
    gH = given.get("H")
    Hs, pres, Z = mlp_forward(params, dims, X, plan, given_H=gH)
    H_own = Hs[1:]
    if gH is not None:
        # the backward stages consume the stored activations
        Hs = [Hs[0]] + [np.asarray(h, np.float64) for h in gH]
    grad_scale = 1.0 if P["unscaled"] else 1.0 / B
    alpha = 1.0 / B if P["unscaled"] else 1.0
    Zin = np.asarray(given["Z"], np.float64) if "Z" in given else Z
    loss, row_loss, G, _ = softmax_xent(Zin, labels, grad_scale, P["dz"])
    argmax = np.asarray(Z).argmax(axis=1).astype(np.int32)
    grads = [None] * L
    dHs = [None] * L
    ties = 0
    Gl = np.asarray(given["G"], np.float64) if "G" in given else G
    for li in range(L - 1, -1, -1):
        W, _ = layers[li]
        Wg = round_fmt(W, P["gemm_w"]) if P["gemm_w"] else W
        dW, _ = gemm_epilogue(Hs[li], Gl, "TN", alpha, out_fmt="f32" if plan != "f64" else "f64")
        db = colsum(Gl, alpha, out_fmt="f32" if plan != "f64" else "f64")
        grads[li] = (dW, db)
        if li > 0:
            Hprev = Hs[li]
            mask_src = Hprev
            if mask_hint is not None and tie_abs > 0:
                hint = np.asarray(mask_hint[li - 1], dtype=np.float64)
                tie = np.abs(pres[li - 1]) <= tie_abs
                ties += int(np.count_nonzero(tie & ((hint > 0) != (Hprev > 0))))
                mask_src = np.where(tie, hint, Hprev)
            Gl, _ = gemm_epilogue(Gl, Wg, "NT", 1.0, act="relu_mask_bwd", aux=mask_src,
                                  out_fmt=P["act"])
            dHs[li - 1] = Gl
            if "dH" in given:
                Gl = np.asarray(given["dH"][li - 1], np.float64)
    gflat = np.concatenate([np.concatenate([dW.ravel(), db]) for dW, db in grads])
    if plan == "f64":
        vnew = momentum * np.asarray(vel, dtype=np.float64) - lr * gflat
        wnew = np.asarray(params, dtype=np.float64) + vnew
        wlow = None
    else:
        wnew, vnew, wlow = sgd_momentum(params, gflat, vel, lr, momentum,
                                        "f16" if plan == "f16" else None)
    return dict(loss=loss, row_loss=row_loss, Z=Z, G=G, argmax=argmax, H=H_own,
                pre=pres, dH=dHs[:-1] if L > 1 else [], grads=gflat,
                params=wnew, vel=vnew, params_lowp=wlow, mask_ties=ties)


def mlp_loss_only(params, dims, X, labels) -> float:
    """Mean cross-entropy loss of the f64 plan (for finite differences)."""
    _, _, Z = mlp_forward(params, dims, X, "f64")
    return softmax_xent(Z, labels, 1.0, "f64")[0]
