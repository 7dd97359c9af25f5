"""Single operations of the path, float64 (oracle side; test infrastructure only).

Each function follows one passage of the pages; the docstring names it.
"""
from __future__ import annotations

import numpy as np

from .numerics import round_fmt

ACTS = ("none", "relu", "lrelu_sq", "relu_mask_bwd", "lrelu_sq_bwd")


def act_forward(v, act: str, slope: float = 0.5):
    """Forward activations applied in the GEMM epilogue.

    relu: max(v, 0), with NaN mapped to 0 like ``fmaxf(acc, 0)`` in the
    capstone's epilogue ("Capstone 5", section "Read the worked reference").
    lrelu_sq: (v if v > 0 else slope*v)**2, the LeakyReLU-squared activation of
    the MLP block ("Full-Depth MLP Megakernel ...", section "What Worked").
    """
    v = np.asarray(v, dtype=np.float64)
    if act == "none":
        return v.copy()
    if act == "relu":
        return np.where(v > 0, v, 0.0)
    if act == "lrelu_sq":
        t = np.where(v > 0, v, slope * v)
        return t * t
    raise ValueError(act)


def act_backward_factor(aux, act: str, slope: float = 0.5):
    """Derivative factor multiplied into a dgrad GEMM's accumulator.

    relu_mask_bwd: [aux > 0] -- a hidden value at or below zero passed no
    output, so its gradient is zero ("Capstone 5", sections "Work through the
    backward pass" and "Check your mapping").
    lrelu_sq_bwd: d/du (leaky(u))^2 = 2u for u > 0 and 2*slope^2*u otherwise
    (the block's "backward epilogue", "Full-Depth MLP Megakernel ...",
    section "Credits"; the derivative is elementary calculus).
    """
    aux = np.asarray(aux, dtype=np.float64)
    if act == "relu_mask_bwd":
        return (aux > 0).astype(np.float64)
    if act == "lrelu_sq_bwd":
        return np.where(aux > 0, 2.0 * aux, 2.0 * slope * slope * aux)
    raise ValueError(act)


def gemm_epilogue(A, B, layout: str = "NN", alpha: float = 1.0, bias=None,
                  act: str = "none", slope: float = 0.5, aux=None, residual=None,
                  out_fmt: str = "f32", pre_fmt: str | None = None):
    """C = round(act(alpha * op(A) op(B) + bias) [+ residual]).

    Layouts (all row-major storage): NN  C = A B      with A [M x K], B [K x N];
                                     NT  C = A B^T    with B stored [N x K];
                                     TN  C = A^T B    with A stored [K x M].
    The forward GEMM keeps bias and ReLU in its epilogue and writes no
    separate bias or ReLU array ("Capstone 5", "Read the worked reference");
    the accumulator stays in high precision, bias and activation are applied
    there and the conversion happens once at the store ("The Work Moved Down
    a Layer", "The Debugging Lesson Was Numerical").  The weight gradients
    X^T dH and the input gradient dH W^T are the same product with one
    transposed operand ("Capstone 5", "Retrieve what you need", "Work through
    the backward pass").

    For the backward activations the epilogue multiplies by the derivative
    factor of ``aux`` (the stored forward value) instead of applying an
    activation.  Returns (C, pre) where ``pre`` = round(alpha*acc + bias,
    pre_fmt) when ``pre_fmt`` is given, else None.
    """
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    opA = A if layout in ("NN", "NT") else A.T
    opB = B if layout in ("NN", "TN") else B.T
    if opA.shape[1] != opB.shape[0]:
        raise ValueError("inner dimensions differ")
    v = alpha * (opA @ opB)
    if bias is not None:
        v = v + np.asarray(bias, dtype=np.float64)[None, :]
    pre = round_fmt(v, pre_fmt) if pre_fmt is not None else None
    if act in ("none", "relu", "lrelu_sq"):
        v = act_forward(v, act, slope)
    elif act in ("relu_mask_bwd", "lrelu_sq_bwd"):
        if aux is None:
            raise ValueError("backward activation needs aux")
        v = v * act_backward_factor(aux, act, slope)
    else:
        raise ValueError(act)
    if residual is not None:
        v = v + np.asarray(residual, dtype=np.float64)
    return round_fmt(v, out_fmt), pre


def colsum(X, alpha: float = 1.0, out_fmt: str = "f32"):
    """s_j = alpha * sum over rows m of X[m, j].

    Each bias gradient is a column reduction over the batch ("Capstone 5",
    "Work through the backward pass": db = sum_rows(dZ); "Check your
    mapping": one gradient per image for each unit, one bias per unit).
    """
    X = np.asarray(X, dtype=np.float64)
    return round_fmt(alpha * X.sum(axis=0), out_fmt)


def softmax_xent(Z, labels, grad_scale: float, d_fmt: str = "f32"):
    """Stable softmax cross-entropy, forward and backward, per row.

    m = max_c z_c;  lse = m + ln(sum_c exp(z_c - m));  loss_row = lse - z_y;
    loss = mean over rows;  dZ_c = grad_scale * (exp(z_c - lse) - [c == y]);
    argmax = lowest index of the maximum.  Subtracting each row's maximum
    before exponentiating is what keeps +-60 logits finite ("Capstone 5",
    "Read the worked reference", last paragraph).

    Returns (loss_mean, row_loss, dZ rounded to d_fmt, argmax).
    """
    Z = np.asarray(Z, dtype=np.float64)
    labels = np.asarray(labels, dtype=np.int64)
    rows = np.arange(Z.shape[0])
    m = Z.max(axis=1, keepdims=True)
    lse = m + np.log(np.exp(Z - m).sum(axis=1, keepdims=True))
    row_loss = (lse[:, 0] - Z[rows, labels])
    p = np.exp(Z - lse)
    onehot = np.zeros_like(Z)
    onehot[rows, labels] = 1.0
    dZ = round_fmt(grad_scale * (p - onehot), d_fmt)
    argmax = Z.argmax(axis=1).astype(np.int32)
    loss_mean = row_loss.mean() if Z.shape[0] else 0.0
    return loss_mean, row_loss, dZ, argmax


def rmsnorm_fwd(x, eps: float, gamma=None, y_fmt: str = "f32", r_fmt: str = "f32"):
    """RMSNorm forward with float statistics.

    ms = mean_j x_j^2;  r = 1/sqrt(ms + eps);  y = x * r (* gamma).
    Statistics stay in high precision ("The Work Moved Down a Layer", "The
    Debugging Lesson Was Numerical"); the step itself is the first operation
    of the MLP block ("Full-Depth MLP Megakernel ...", "What Worked").
    Returns (y rounded to y_fmt, r rounded to r_fmt).
    """
    x = np.asarray(x, dtype=np.float64)
    ms = (x * x).mean(axis=1)
    r = 1.0 / np.sqrt(ms + eps)
    y = x * r[:, None]
    if gamma is not None:
        y = y * np.asarray(gamma, dtype=np.float64)[None, :]
    return round_fmt(y, y_fmt), round_fmt(r, r_fmt)


def rmsnorm_bwd(x, r, dy, dres=None, gamma=None, dx_fmt: str = "f32", dg_fmt: str = "f32"):
    """RMSNorm backward from the stored row statistic r.

    xh = x * r;  g = dy * gamma;  c = mean_j g_j xh_j;
    dx = r * (g - xh * c) + dres;  dgamma = sum_rows dy * xh.
    (Chain rule through y = x * (mean x^2 + eps)^(-1/2) * gamma.)
    Returns (dx rounded to dx_fmt, dgamma rounded to f32 or None).
    """
    x = np.asarray(x, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)[:, None]
    dy = np.asarray(dy, dtype=np.float64)
    xh = x * r
    g = dy if gamma is None else dy * np.asarray(gamma, dtype=np.float64)[None, :]
    c = (g * xh).mean(axis=1, keepdims=True)
    dx = r * (g - xh * c)
    if dres is not None:
        dx = dx + np.asarray(dres, dtype=np.float64)
    dgamma = None if gamma is None else round_fmt((dy * xh).sum(axis=0), dg_fmt)
    return round_fmt(dx, dx_fmt), dgamma


def sgd_momentum(w, g, v, lr: float, momentum: float, lowp_fmt: str | None = None):
    """One momentum update over a flat buffer.

    vel = momentum * v - lr * g;  v <- vel;  w <- w + vel, for every element
    of the one flat parameter buffer ("Capstone 5", "Read the worked
    reference").  Computed in float64 from the stored values, then stored as
    float32; optionally also a low-precision working copy of the new w.
    Returns (w_new, v_new, w_lowp or None).
    """
    w = np.asarray(w, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    vel = momentum * v - lr * g
    w_new = round_fmt(w + vel, "f32")
    v_new = round_fmt(vel, "f32")
    w_lowp = round_fmt(w_new, lowp_fmt) if lowp_fmt else None
    return w_new, v_new, w_lowp
