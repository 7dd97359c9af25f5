"""Pins for the oracle's single operations (CPU only).

Each check is independent of the oracle's own formula: brute-force loops on
tiny inputs, closed forms, invariants, finite differences, and torch-CPU
float64 library routines.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import datagen
from oracle import (act_backward_factor, act_forward, colsum, gemm_epilogue,
                    rmsnorm_bwd, rmsnorm_fwd, round_fmt, sgd_momentum, softmax_xent)

ACTS_FWD = ["none", "relu", "lrelu_sq"]


def _brute_gemm(A, B, layout, alpha, bias, act, slope, aux, res):
    """Triple loop written independently of the oracle (Python scalars)."""
    if layout == "NN":
        M, K = A.shape; N = B.shape[1]
        a = lambda i, k: A[i][k]; b = lambda k, j: B[k][j]
    elif layout == "NT":
        M, K = A.shape; N = B.shape[0]
        a = lambda i, k: A[i][k]; b = lambda k, j: B[j][k]
    else:
        K, M = A.shape; N = B.shape[1]
        a = lambda i, k: A[k][i]; b = lambda k, j: B[k][j]
    C = [[0.0] * N for _ in range(M)]
    for i in range(M):
        for j in range(N):
            s = 0.0
            for k in range(K):
                s += float(a(i, k)) * float(b(k, j))
            v = alpha * s + (float(bias[j]) if bias is not None else 0.0)
            if act == "relu":
                v = v if v > 0 else 0.0
            elif act == "lrelu_sq":
                v = (v if v > 0 else slope * v) ** 2
            elif act == "relu_mask_bwd":
                v = v if aux[i][j] > 0 else 0.0
            elif act == "lrelu_sq_bwd":
                u = float(aux[i][j])
                v = v * (2 * u if u > 0 else 2 * slope * slope * u)
            if res is not None:
                v += float(res[i][j])
            C[i][j] = v
    return np.array(C)


@pytest.mark.parametrize("layout", ["NN", "NT", "TN"])
@pytest.mark.parametrize("act", ["none", "relu", "lrelu_sq", "relu_mask_bwd", "lrelu_sq_bwd"])
def test_gemm_matches_brute_force(layout, act):
    g = np.random.default_rng(3)
    M, N, K = 3, 4, 5
    A = g.normal(size=(M, K) if layout != "TN" else (K, M))
    B = g.normal(size=(K, N) if layout != "NT" else (N, K))
    bias = g.normal(size=N) if act in ACTS_FWD else None
    aux = g.normal(size=(M, N))
    res = g.normal(size=(M, N))
    got, pre = gemm_epilogue(A, B, layout, 0.75, bias, act, 0.5, aux, res, out_fmt="f64",
                             pre_fmt="f64")
    ref = _brute_gemm(A, B, layout, 0.75, bias, act, 0.5, aux, res)
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-13)
    ref_pre = _brute_gemm(A, B, layout, 0.75, bias, "none", 0.5, None, None)
    np.testing.assert_allclose(pre, ref_pre, rtol=1e-13, atol=1e-13)


def test_gemm_layouts_agree_and_integer_exact():
    A = datagen.integer_matrix((37, 29), 1)
    B = datagen.integer_matrix((29, 41), 2)
    c_nn, _ = gemm_epilogue(A, B, "NN", out_fmt="f16")
    c_nt, _ = gemm_epilogue(A, B.T.copy(), "NT", out_fmt="f16")
    c_tn, _ = gemm_epilogue(A.T.copy(), B, "TN", out_fmt="f16")
    np.testing.assert_array_equal(c_nn, c_nt)
    np.testing.assert_array_equal(c_nn, c_tn)
    assert np.all(c_nn == np.round(c_nn))          # integer-valued, exact in f16
    assert np.abs(c_nn).max() <= 29 * 4


def test_gemm_identity_zero_outer():
    g = np.random.default_rng(4)
    B = g.normal(size=(6, 7)); bias = g.normal(size=7)
    c, _ = gemm_epilogue(np.eye(6), B, "NN", bias=bias, act="relu", out_fmt="f64")
    np.testing.assert_allclose(c, np.maximum(B + bias, 0.0), rtol=0, atol=1e-15)
    c0, _ = gemm_epilogue(g.normal(size=(5, 6)), np.zeros((6, 7)), "NN", bias=bias,
                          act="lrelu_sq", out_fmt="f64")
    np.testing.assert_allclose(c0, np.tile(np.where(bias > 0, bias, 0.5 * bias) ** 2, (5, 1)))
    u = g.normal(size=(5, 1)); v = g.normal(size=(1, 7))
    c1, _ = gemm_epilogue(u, v, "NN", out_fmt="f64")
    np.testing.assert_allclose(c1, np.outer(u[:, 0], v[0]), rtol=1e-15)


def test_activation_values_and_derivatives():
    assert act_forward(np.array([np.nan]), "relu")[0] == 0.0       # fmaxf(NaN, 0) = 0
    np.testing.assert_array_equal(act_forward(np.array([-2.0, 0.0, 3.0]), "lrelu_sq", 0.5),
                                  [1.0, 0.0, 9.0])
    np.testing.assert_array_equal(act_backward_factor(np.array([-1.0, 0.0, 2.0]), "relu_mask_bwd"),
                                  [0.0, 0.0, 1.0])
    u = np.random.default_rng(5).normal(size=1000)
    u = u[np.abs(u) > 1e-3]
    h = 1e-6
    fd = (act_forward(u + h, "lrelu_sq") - act_forward(u - h, "lrelu_sq")) / (2 * h)
    np.testing.assert_allclose(act_backward_factor(u, "lrelu_sq_bwd"), fd, rtol=1e-7, atol=1e-9)
    fd = (act_forward(u + h, "relu") - act_forward(u - h, "relu")) / (2 * h)
    np.testing.assert_allclose(act_backward_factor(u, "relu_mask_bwd"), fd, atol=1e-9)


def test_gemm_rounds_once_at_store():
    # the post-activation value comes from the unrounded accumulator
    A = np.array([[1.0 + 2.0 ** -12]]); B = np.array([[1.0]])
    c, pre = gemm_epilogue(A, B, "NN", act="lrelu_sq", out_fmt="f16", pre_fmt="f16")
    assert pre[0, 0] == 1.0                            # rounded pre-activation
    assert c[0, 0] == round_fmt(np.array([(1.0 + 2.0 ** -12) ** 2]), "f16")[0]


def test_colsum():
    X = np.ones((300, 7))
    np.testing.assert_array_equal(colsum(X), np.full(7, 300.0))
    Xi = datagen.integer_matrix((129, 11), 3)
    ref = [sum(Xi[m][j] for m in range(129)) for j in range(11)]
    np.testing.assert_array_equal(colsum(Xi, 0.5), 0.5 * np.array(ref))


def test_softmax_xent_zero_logits_is_ln_c(pins):
    for C in (10, 256):
        Z = np.zeros((5, C)); y = np.arange(5) % C
        loss, rl, dZ, am = softmax_xent(Z, y, 1 / 5, "f64")
        assert loss == pytest.approx(math.log(C), rel=1e-15)
        onehot = np.eye(C)[y]
        np.testing.assert_allclose(dZ, (1.0 / C - onehot) / 5, rtol=1e-14, atol=1e-17)
        assert np.all(am == 0)                       # ties -> lowest index


def test_softmax_xent_extreme_logits(pins):
    E = pins["extreme_logit"]
    for k in (1, 2, 5):
        Z = np.full((2, 10), -E); Z[:, :k] = E
        y = np.array([0, 9])                         # label on a +E entry / on a -E entry
        loss, rl, dZ, am = softmax_xent(Z, y, 1.0, "f32")
        assert np.all(np.isfinite(rl)) and np.all(np.isfinite(dZ))
        assert rl[0] == pytest.approx(math.log(k), abs=1e-12)
        assert rl[1] == pytest.approx(2 * E + math.log(k), rel=1e-12)


def test_softmax_xent_gradient_and_library():
    g = np.random.default_rng(6)
    Z = g.normal(scale=3.0, size=(7, 10)); y = g.integers(0, 10, size=7)
    loss, rl, dZ, am = softmax_xent(Z, y, 1 / 7, "f64")
    np.testing.assert_allclose(dZ.sum(axis=1), 0.0, atol=1e-15)
    tl = F.cross_entropy(torch.from_numpy(Z), torch.from_numpy(y).long())
    assert loss == pytest.approx(tl.item(), rel=1e-14)
    h = 1e-6
    fd = np.zeros_like(Z)
    for i in range(Z.shape[0]):
        for c in range(Z.shape[1]):
            Zp = Z.copy(); Zp[i, c] += h
            Zm = Z.copy(); Zm[i, c] -= h
            fd[i, c] = (softmax_xent(Zp, y, 1, "f64")[0] - softmax_xent(Zm, y, 1, "f64")[0]) / (2 * h)
    np.testing.assert_allclose(dZ, fd, rtol=1e-6, atol=1e-9)
    np.testing.assert_array_equal(am, Z.argmax(axis=1))


def test_rmsnorm_forward():
    c = np.array([[3.0] * 8, [-0.5] * 8])
    y, r = rmsnorm_fwd(c, 1e-6, y_fmt="f64", r_fmt="f64")
    np.testing.assert_allclose(y[:, 0], c[:, 0] / np.sqrt(c[:, 0] ** 2 + 1e-6), rtol=1e-15)
    x = np.random.default_rng(7).normal(size=(9, 16))
    y, r = rmsnorm_fwd(x, 1e-6, y_fmt="f64", r_fmt="f64")
    ty = F.rms_norm(torch.from_numpy(x), (16,), eps=1e-6)
    np.testing.assert_allclose(y, ty.numpy(), rtol=1e-13)
    y2, _ = rmsnorm_fwd(1e3 * x, 0.0, y_fmt="f64", r_fmt="f64")
    np.testing.assert_allclose(y2, rmsnorm_fwd(x, 0.0, y_fmt="f64", r_fmt="f64")[0], rtol=1e-13)


def test_rmsnorm_backward():
    g = np.random.default_rng(8)
    x = g.normal(size=(6, 12)); dy = g.normal(size=(6, 12)); gam = g.normal(size=12)
    eps = 1e-3
    _, r = rmsnorm_fwd(x, eps, y_fmt="f64", r_fmt="f64")
    dx, dg = rmsnorm_bwd(x, r, dy, gamma=gam, dx_fmt="f64", dg_fmt="f64")
    tx = torch.from_numpy(x).requires_grad_(); tg = torch.from_numpy(gam).requires_grad_()
    (F.rms_norm(tx, (12,), weight=tg, eps=eps) * torch.from_numpy(dy)).sum().backward()
    np.testing.assert_allclose(dx, tx.grad.numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dg, tg.grad.numpy(), rtol=1e-12, atol=1e-13)
    # closed-form invariant: x . dx = r (x . g) eps / (ms + eps), row by row
    dx0, _ = rmsnorm_bwd(x, r, dy, dx_fmt="f64")
    ms = (x * x).mean(axis=1)
    np.testing.assert_allclose((x * dx0).sum(axis=1), r * (x * dy).sum(axis=1) * eps / (ms + eps),
                               rtol=1e-9, atol=1e-13)
    dres = g.normal(size=(6, 12))
    dx1, _ = rmsnorm_bwd(x, r, dy, dres=dres, dx_fmt="f64")
    np.testing.assert_allclose(dx1 - dres, dx0, atol=1e-14)


def test_sgd_momentum_closed_form(pins):
    lr, mu = pins["lr"], pins["momentum"]
    w0 = np.array([0.5, -0.25, 1.0]); g = np.array([0.1, -0.2, 0.0])
    w, v = w0.copy(), np.zeros(3)
    for t in range(1, 31):
        w, v, _ = sgd_momentum(w, g, v, lr, mu)
        v_ref = -lr * g * (1 - mu ** t) / (1 - mu)
        w_ref = w0 - lr * g * sum((1 - mu ** s) / (1 - mu) for s in range(1, t + 1))
        tol = pins["step_tol_abs"] + pins["step_tol_rel"] * np.abs(w_ref)
        assert np.all(np.abs(w - w_ref) <= tol)
        np.testing.assert_allclose(v, v_ref, rtol=1e-5, atol=1e-7)
    w2, v2, wl = sgd_momentum(w0, np.zeros(3), np.zeros(3), lr, mu, "f16")
    np.testing.assert_array_equal(w2, w0)
    np.testing.assert_array_equal(v2, 0.0)
    np.testing.assert_array_equal(wl, round_fmt(w0, "f16"))
