"""Bit-exact FP32 definitions of the path's primitives (oracle side; test
infrastructure only).

The library's bit-exact mode computes each primitive as the fixed sequence of
IEEE binary32 operations written out here, each operation rounded to nearest
even, with no fused multiply-add, every sum taken in linear order (first term
first), and divide and square root correctly rounded.  The mode follows the
precision recipe of "HIP + Vulkan backends -- Phase 3" (sections "Phase-3 bug
hunt" and the bit-accuracy summary): a linear left-to-right sum in place of
the hardware reduction tree, a correctly rounded divide in place of a * (1/b),
and a refined reciprocal square root.  The pages' refined rsqrt is within one
ulp but depends on the hardware estimate it starts from, so this definition
takes the reading that a CPU reproduces bit for bit: a correctly rounded
square root followed by a correctly rounded reciprocal.

numpy float32 arithmetic is IEEE binary32 with round-to-nearest-even per
operation, and each expression below is one numpy operation per rounding, so
the functions are the definitions themselves; the loops run over the summed
dimension only, vectorised over the independent outputs.

Inputs are float arrays whose values are exact in their storage format
(binary32, binary16 or bfloat16 values convert to binary32 exactly).  The
softmax cross-entropy is not part of the mode: exp and log keep their library
rounding, as in the pages' own precision work.
"""
from __future__ import annotations

import numpy as np

from .numerics import round_fmt

F = np.float32


def _f(x):
    return np.asarray(x, dtype=np.float64).astype(F)


def linear_sum(X, axis: int = 0):
    """s = (((x_0 + x_1) + x_2) + ...) in binary32 along ``axis``, starting
    from +0.  An empty sum is +0."""
    X = np.moveaxis(_f(X), axis, 0)
    s = np.zeros(X.shape[1:], dtype=F)
    for i in range(X.shape[0]):
        s = s + X[i]
    return s


def gemm(A, B, layout: str = "NN", alpha: float = 1.0, bias=None, act: str = "none",
         slope: float = 0.5, aux=None, residual=None, out_fmt: str = "f32", pre_fmt: str | None = None):
    """C = convert(act(alpha * op(A) op(B) + bias) [+ residual]), bit-exact.

    acc = +0;  for k = 0 .. K-1:  acc = acc + a_k * b_k   (two roundings; the
    product of two binary16 or bfloat16 values is exact in binary32);
    v = alpha * acc;  v = v + bias[n];  pre = convert(v);
    relu: v = v if v > 0 else +0;  lrelu_sq: t = v if v > 0 else slope * v, v = t * t;
    relu_mask_bwd: v = v * f with f = 1 if aux > 0 else 0;
    lrelu_sq_bwd: v = v * f with f = 2 * aux if aux > 0 else c * aux, c = (2 * slope) * slope;
    v = v + residual;  C = convert(v).
    The operations are the epilogue of "Capstone 5" ("Read the worked
    reference") and of the MLP block ("Full-Depth MLP Megakernel ...",
    "What Worked", "Credits"), in the order the library documents.
    Returns (C, pre) as float64 arrays of exactly representable values.
    """
    A = _f(A)
    B = _f(B)
    opA = A if layout in ("NN", "NT") else A.T
    opB = B if layout in ("NN", "TN") else B.T
    M, K = opA.shape
    N = opB.shape[1]
    acc = np.zeros((M, N), dtype=F)
    for k in range(K):
        acc = acc + opA[:, k:k + 1] * opB[k:k + 1, :]
    v = F(alpha) * acc
    if bias is not None:
        v = v + _f(bias)[None, :]
    pre = round_fmt(v.astype(np.float64), pre_fmt) if pre_fmt is not None else None
    if act == "relu":
        v = np.where(v > 0, v, F(0))
    elif act == "lrelu_sq":
        t = np.where(v > 0, v, F(slope) * v)
        v = t * t
    elif act == "relu_mask_bwd":
        v = v * np.where(_f(aux) > 0, F(1), F(0))
    elif act == "lrelu_sq_bwd":
        a = _f(aux)
        c = (F(2) * F(slope)) * F(slope)
        v = v * np.where(a > 0, F(2) * a, c * a)
    elif act != "none":
        raise ValueError(act)
    if residual is not None:
        v = v + _f(residual)
    return round_fmt(v.astype(np.float64), out_fmt), pre


def colsum(X, alpha: float = 1.0, out=None):
    """out[n] = alpha * s_n, or out[n] + alpha * s_n with ``out`` given,
    where s_n is the linear sum of column n over the rows in row order
    (the bias gradient of "Capstone 5", "Work through the backward pass")."""
    t = F(alpha) * linear_sum(X, axis=0)
    if out is not None:
        t = _f(out) + t
    return t.astype(np.float64)


def sgd_momentum(w, g, v, lr: float, momentum: float, lowp_fmt: str | None = None):
    """vel = momentum * v - lr * g;  v <- vel;  w <- w + vel, each product
    and sum rounded on its own ("Capstone 5", "Read the worked reference").
    Returns (w_new, v_new, w_lowp or None)."""
    vel = F(momentum) * _f(v) - F(lr) * _f(g)
    w_new = _f(w) + vel
    w64 = w_new.astype(np.float64)
    return w64, vel.astype(np.float64), round_fmt(w64, lowp_fmt) if lowp_fmt else None


def rmsnorm_fwd(x, eps: float, gamma=None, y_fmt: str = "f32"):
    """ss = linear sum of x_j * x_j;  ms = ss / D;  r = 1 / sqrt(ms + eps)
    (divides and square root correctly rounded);  y = x * r, then * gamma.
    RMSNorm with FP32 statistics ("The Work Moved Down a Layer", "The
    Debugging Lesson Was Numerical"; "Full-Depth MLP Megakernel ...", "What
    Worked").  Returns (y converted to y_fmt, r) as float64."""
    x = _f(x)
    D = x.shape[1]
    ss = linear_sum(x * x, axis=1)
    ms = ss / F(D)
    r = F(1) / np.sqrt(ms + F(eps))
    y = x * r[:, None]
    if gamma is not None:
        y = y * _f(gamma)[None, :]
    return round_fmt(y.astype(np.float64), y_fmt), r.astype(np.float64)


def rmsnorm_bwd(x, r, dy, dres=None, gamma=None, dx_fmt: str = "f32"):
    """xh = x * r;  g = dy * gamma (or dy);  c = (linear sum of g_j * xh_j) / D;
    dx = r * (g - xh * c), then + dres;  dgamma[j] = linear sum over the rows
    (in row order) of dy * xh.  The chain rule through y = x r gamma.
    Returns (dx converted to dx_fmt, dgamma or None) as float64."""
    x = _f(x)
    r = _f(r)[:, None]
    dy = _f(dy)
    D = x.shape[1]
    xh = x * r
    g = dy if gamma is None else dy * _f(gamma)[None, :]
    c = linear_sum(g * xh, axis=1)[:, None] / F(D)
    dx = r * (g - xh * c)
    if dres is not None:
        dx = dx + _f(dres)
    dgamma = None if gamma is None else linear_sum(dy * xh, axis=0).astype(np.float64)
    return round_fmt(dx.astype(np.float64), dx_fmt), dgamma
