"""Pins of the bit-exact FP32 oracle (oracle/exact.py) against what the
arithmetic fixes: sums whose value depends on their order, exactly
representable closed forms, single-rounding cases and the standard error
bound of a recursive sum.  CPU only."""
import math

import numpy as np
import pytest

import datagen
from oracle import exact, gemm_epilogue, round_fmt

E = 2.0 ** -24          # half an ulp of 1.0 in binary32


def f32bits(x):
    return np.asarray(x, dtype=np.float64).astype(np.float32).view(np.uint32)


def test_linear_sum_is_first_term_first():
    # 1 + e rounds back to 1 (a tie, to even), 1000 times over; the reverse
    # order first gathers 1000 e exactly and then adds it to 1
    col = np.array([1.0] + [E] * 1000)[:, None]
    assert exact.linear_sum(col)[0] == np.float32(1.0)
    assert exact.linear_sum(col[::-1])[0] == np.float32(1.0 + 1000 * E)
    # a pairwise or FP64 sum would give the second value for both orders
    assert float(np.sum(col)) != 1.0
    # empty sum
    assert exact.linear_sum(np.zeros((0, 3))).tolist() == [0.0, 0.0, 0.0]


def test_colsum_order_alpha_and_accumulate():
    X = np.array([[1.0, E], [E, 1.0]] + [[E, E]] * 999)
    s = exact.colsum(X, 1.0)
    assert s[0] == 1.0                                # 1 first: every e is lost
    assert s[1] == np.float32(np.float32(E) + np.float32(1.0)) and s[1] == 1.0
    # alpha after the sum, one rounding; accumulate adds to what is there
    X2 = np.array([[3.0], [5.0]])
    assert exact.colsum(X2, 0.5)[0] == 4.0
    assert exact.colsum(X2, 0.5, out=np.array([1.5]))[0] == 5.5


def test_gemm_integer_products_are_exact():
    rng = datagen.rng(7, "misc")
    A = rng.integers(-8, 9, size=(13, 37)).astype(np.float64)
    B = rng.integers(-8, 9, size=(37, 11)).astype(np.float64)
    C, _ = exact.gemm(A, B, "NN")
    np.testing.assert_array_equal(C, A @ B)            # every partial sum is an exact integer
    # the three layouts are the same product of the stored operands
    np.testing.assert_array_equal(exact.gemm(A, B.T.copy(), "NT")[0], A @ B)
    np.testing.assert_array_equal(exact.gemm(A.T.copy(), B, "TN")[0], A @ B)


def test_gemm_sums_k_in_order():
    A = np.array([[1.0] + [E] * 200])
    B = np.ones((201, 1))
    assert exact.gemm(A, B, "NN")[0][0, 0] == 1.0
    assert exact.gemm(A[:, ::-1].copy(), B, "NN")[0][0, 0] == np.float32(1.0 + 200 * E)


def test_gemm_fp32_products_round_before_the_add():
    # a*b is rounded to binary32 and then added: for a = b = 1 + 2^-12 the
    # product's last bit (2^-24) is a tie that rounds to even, so
    # acc = 0 + a*b = 1 + 2^-11 exactly, where a fused multiply-add would keep
    # 1 + 2^-11 + 2^-24 and then round once more with the next term
    a = 1.0 + 2.0 ** -12
    A = np.array([[a, -1.0]])
    B = np.array([[a], [1.0 + 2.0 ** -11]])
    assert exact.gemm(A, B, "NN")[0][0, 0] == 0.0
    # with one fused rounding the result would be 2^-24
    assert a * a - (1.0 + 2.0 ** -11) == 2.0 ** -24


def test_gemm_epilogue_closed_forms():
    A = np.array([[1.0, 2.0], [-3.0, 0.5]])
    B = np.eye(2)
    bias = np.array([0.25, -1.0])
    C, pre = exact.gemm(A, B, "NN", alpha=2.0, bias=bias, act="relu", pre_fmt="f32")
    np.testing.assert_array_equal(pre, [[2.25, 3.0], [-5.75, 0.0]])
    np.testing.assert_array_equal(C, [[2.25, 3.0], [0.0, 0.0]])
    C, _ = exact.gemm(A, B, "NN", act="lrelu_sq", slope=0.5)
    np.testing.assert_array_equal(C, [[1.0, 4.0], [2.25, 0.25]])
    aux = np.array([[1.0, -1.0], [0.0, 2.0]])
    C, _ = exact.gemm(A, B, "NN", act="relu_mask_bwd", aux=aux)
    assert C.tolist() == [[1.0, 0.0], [0.0, 0.5]]
    assert np.signbit(C[1, 0])                           # -3 * 0 = -0: a product, not a select
    C, _ = exact.gemm(A, B, "NN", act="lrelu_sq_bwd", slope=0.5, aux=aux)
    np.testing.assert_array_equal(C, [[2.0, -1.0], [-0.0, 2.0]])   # 2*1, 2*(0.5^2)*(-1)*2 ...
    C, _ = exact.gemm(A, B, "NN", residual=np.array([[1.0, 1.0], [1.0, 1.0]]), out_fmt="f16")
    np.testing.assert_array_equal(C, [[2.0, 3.0], [-2.0, 1.5]])


def test_gemm_within_the_recursive_sum_bound():
    # |C - C_exact| <= gamma_K * sum_k |a_k b_k|, gamma_K = K u / (1 - K u),
    # for a recursive sum of rounded products (u = 2^-24); a dropped term, a
    # wrong index or a transposed operand breaks the bound by many orders
    rng = datagen.rng(3, "misc")
    for layout, fmt in (("NN", "f32"), ("NT", "f16"), ("TN", "bf16")):
        M, N, K = 9, 7, 300
        A = round_fmt(rng.standard_normal((M, K) if layout != "TN" else (K, M)), fmt)
        B = round_fmt(rng.standard_normal((K, N) if layout != "NT" else (N, K)), fmt)
        C, _ = exact.gemm(A, B, layout)
        ref, _ = gemm_epilogue(A, B, layout, out_fmt="f64")
        opA = A if layout != "TN" else A.T
        opB = B if layout != "NT" else B.T
        u = 2.0 ** -24
        g = (K + 1) * u / (1 - (K + 1) * u)
        bound = g * (np.abs(opA) @ np.abs(opB))
        assert np.all(np.abs(C - ref) <= bound), layout
        assert np.any(C != round_fmt(ref, "f32"))          # not simply the rounded exact value


def test_sgd_closed_forms():
    w = np.array([1.0, 2.0, -3.0])
    g = np.array([0.5, -1.0, 2.0])
    v = np.array([0.25, 0.0, -1.0])
    w1, v1, _ = exact.sgd_momentum(w, g, v, lr=0.5, momentum=0.5)
    np.testing.assert_array_equal(v1, [-0.125, 0.5, -1.5])
    np.testing.assert_array_equal(w1, [0.875, 2.5, -4.5])
    # two roundings (mu v, lr g) then the difference: 0.1f * 3 and 0.1f * 0.7f
    # are each rounded before the subtraction
    w2, v2, lp = exact.sgd_momentum([0.0], [0.7], [3.0], lr=0.1, momentum=0.1, lowp_fmt="bf16")
    want = np.float32(np.float32(0.1) * np.float32(3.0)) - np.float32(np.float32(0.1) * np.float32(0.7))
    assert v2[0] == want and w2[0] == want and lp[0] == round_fmt(np.float64(want), "bf16")


def test_rmsnorm_fwd_closed_forms_and_order():
    # x = 2 everywhere: ss = 4 D, ms = 4, sqrt = 2, r = 0.5, y = 1, all exact
    y, r = exact.rmsnorm_fwd(np.full((2, 8), 2.0), 0.0)
    assert r.tolist() == [0.5, 0.5] and np.all(y == 1.0)
    # with eps making ms + eps a square: ms = 9/4, eps = 7/4 -> r = 1/2
    y, r = exact.rmsnorm_fwd(np.array([[1.5, -1.5, 1.5, 1.5]]), 1.75)
    assert r[0] == 0.5 and y.tolist() == [[0.75, -0.75, 0.75, 0.75]]
    # the sum of squares is linear: 1 + 2^-13 squared loses its tail when
    # added after 1, and the reverse order keeps it
    t = 2.0 ** -13
    row = np.array([[1.0] + [t] * 64])
    row_rev = row[:, ::-1].copy()
    _, r1 = exact.rmsnorm_fwd(row, 0.0)
    _, r2 = exact.rmsnorm_fwd(row_rev, 0.0)
    ms1 = np.float32(1.0) / np.float32(65)
    assert r1[0] == np.float32(1) / np.sqrt(ms1) and r1[0] != r2[0]
    # correctly rounded divide, add and square root: each step equals its
    # float64 result rounded once to binary32 (53 >= 2 * 24 + 2 bits, so the
    # float64 step rounds innocuously), an independent route to the same bits
    x = round_fmt(datagen.normal((5, 64), 1.0, seed=5), "f32")
    _, r = exact.rmsnorm_fwd(x, 1e-6)
    ss = exact.linear_sum(x * x, axis=1).astype(np.float64)
    ms = (ss / 64).astype(np.float32).astype(np.float64)
    t = (ms + float(np.float32(1e-6))).astype(np.float32).astype(np.float64)
    s = np.sqrt(t).astype(np.float32).astype(np.float64)
    np.testing.assert_array_equal(f32bits(r), f32bits((1.0 / s).astype(np.float32)))


def test_rmsnorm_bwd_against_the_float64_chain_rule():
    x = round_fmt(datagen.normal((6, 48), 1.0, seed=8), "bf16")
    dy = round_fmt(datagen.normal((6, 48), 1.0, seed=9), "bf16")
    gam = round_fmt(datagen.normal((48,), 1.0, seed=10), "f32")
    dres = round_fmt(datagen.normal((6, 48), 1.0, seed=11), "f32")
    _, r = exact.rmsnorm_fwd(x, 1e-6)
    dx, dg = exact.rmsnorm_bwd(x, r, dy, dres, gam)
    # the float64 oracle's chain rule from the same stored r: within a few
    # ulps of the summed magnitudes
    from oracle import rmsnorm_bwd
    dx64, dg64 = rmsnorm_bwd(x, r, dy, dres, gam, dx_fmt="f64", dg_fmt="f64")
    assert np.all(np.abs(dx - dx64) <= 1e-5 * (1 + np.abs(dx64)))
    assert np.all(np.abs(dg - dg64) <= 1e-5 * (1 + np.abs(dy * x * r[:, None]).sum(axis=0)))
    # D = 1: xh = x r = +-1 (up to rounding), c = g xh, and dx = r (g - xh g xh)
    # vanishes exactly when xh = +-1
    x1 = np.array([[2.0], [-4.0]])
    _, r1 = exact.rmsnorm_fwd(x1, 0.0)
    dx1, _ = exact.rmsnorm_bwd(x1, r1, np.array([[3.0], [5.0]]))
    assert np.all(dx1 == 0.0)
