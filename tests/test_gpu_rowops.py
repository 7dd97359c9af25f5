"""GPU parity of colsum, softmax_xent_fwd_bwd, rmsnorm_fwd_bwd and sgd_momentum."""
import math

import numpy as np
import pytest
import torch

import datagen
import oracle
from parity import TOL_F32, TOL_LOSS, TOL_LOWP, assert_parity

pytestmark = pytest.mark.gpu
TD = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@pytest.fixture(scope="module")
def ge():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import gemm_epilogue_amd
    return gemm_epilogue_amd


def dev(x, fmt):
    return torch.from_numpy(np.ascontiguousarray(x)).to(TD[fmt]).cuda()


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("fmt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("shape", [(1, 1), (128, 10), (128, 256), (4096, 10), (5000, 1003), (4096, 4096),
                                   (8192, 3072), (3000, 4100), (1024, 8200)])
def test_colsum(ge, fmt, shape):
    X = datagen.normal(shape, 1.0, seed=shape[0] + shape[1], fmt=fmt)
    out = ge.colsum(dev(X, fmt), 0.25)
    assert_parity(host(out), oracle.colsum(X, 0.25), TOL_F32 if fmt == "f32" else TOL_LOWP, "f32",
                  f"colsum {shape} {fmt}", cancel=True)


@pytest.mark.parametrize("shape", [(10000, 777), (3000, 8200)])
def test_colsum_deterministic(ge, shape):
    X = dev(datagen.normal(shape, 1.0, seed=5), "f32")
    a, b = ge.colsum(X), ge.colsum(X)
    assert torch.equal(a, b)


@pytest.mark.parametrize("B,C", [(1, 10), (128, 10), (112, 10), (4096, 10), (8192, 256), (33, 1000)])
@pytest.mark.parametrize("dfmt", ["f32", "f16"])
def test_softmax_xent(ge, B, C, dfmt):
    Z = datagen.normal((B, C), 3.0, seed=B + C, fmt="f32")
    y = datagen.rng(B, "labels").integers(0, C, size=B).astype(np.int32)
    scale = 1.0 / B if dfmt == "f32" else 1.0
    loss, rl, dZ, am = ge.softmax_xent_fwd_bwd(dev(Z, "f32"), torch.from_numpy(y).cuda(), scale,
                                               d_dtype=TD[dfmt])
    rl_ref_mean, rl_ref, dZ_ref, am_ref = oracle.softmax_xent(Z, y, scale, dfmt)
    assert abs(host(loss)[0] - rl_ref_mean) <= TOL_LOSS * abs(rl_ref_mean)
    assert_parity(host(rl), rl_ref, TOL_F32, "f32", "row loss")
    assert_parity(host(dZ), dZ_ref, TOL_F32 if dfmt == "f32" else TOL_LOWP, dfmt, "dZ")
    # argmax identical except where the oracle's top-2 gap is below 1e-4
    srt = np.sort(Z, axis=1)
    gap = srt[:, -1] - (srt[:, -2] if C > 1 else -np.inf)
    amg = am.cpu().numpy()
    assert np.all((amg == am_ref) | (gap < 1e-4))


def test_softmax_xent_extreme_and_ties(ge, pins):
    E = pins["extreme_logit"]
    Z = np.full((4, 10), -E)
    Z[0, :1] = E; Z[1, :2] = E; Z[2, :5] = E; Z[3, :] = 0.0
    y = np.array([0, 9, 3, 7], dtype=np.int32)
    loss, rl, dZ, am = ge.softmax_xent_fwd_bwd(dev(Z, "f32"), torch.from_numpy(y).cuda(), 0.25)
    r = host(rl)
    assert np.all(np.isfinite(r)) and torch.isfinite(dZ).all()
    np.testing.assert_allclose(r, [0.0, 2 * E + math.log(2), math.log(5), math.log(10)], rtol=1e-6,
                               atol=1e-6)
    np.testing.assert_array_equal(am.cpu().numpy(), [0, 0, 0, 0])     # lowest index on ties
    ref = oracle.softmax_xent(Z, y, 0.25, "f32")
    assert_parity(host(dZ), ref[2], TOL_F32, "f32", "dZ extreme")


@pytest.mark.parametrize("rows,D,fmt", [(1, 1, "f32"), (37, 100, "f32"), (300, 512, "bf16"),
                                        (98304, 512, "bf16"), (700, 1024, "f32"), (64, 1024, "f16"),
                                        (9, 4096, "f32")])
def test_rmsnorm_fwd_bwd(ge, rows, D, fmt):
    x = datagen.normal((rows, D), 1.0, seed=rows + D, fmt=fmt)
    dy = datagen.normal((rows, D), 1.0, seed=rows + D + 1, fmt=fmt)
    dres = datagen.normal((rows, D), 1.0, seed=rows + D + 2, fmt=fmt)
    tx = dev(x, fmt)
    y, r = ge.rmsnorm_fwd(tx, 1e-6)
    y_ref, r_ref = oracle.rmsnorm_fwd(x, 1e-6, y_fmt=fmt)
    tol = TOL_F32 if fmt == "f32" else TOL_LOWP
    assert_parity(host(r), r_ref, TOL_F32, "f32", "r")
    assert_parity(host(y), y_ref, tol, fmt, "y")
    # backward from the GPU's stored r (lock-step)
    dx, _ = ge.rmsnorm_bwd(tx, r, dev(dy, fmt), dres=dev(dres, fmt))
    dx_ref, _ = oracle.rmsnorm_bwd(x, host(r), dy, dres=dres, dx_fmt=fmt)
    assert_parity(host(dx), dx_ref, tol, fmt, "dx", cancel=True)


def test_rmsnorm_gamma_and_dgamma(ge):
    rows, D = 513, 768
    x = datagen.normal((rows, D), 1.0, seed=81)
    dy = datagen.normal((rows, D), 1.0, seed=82)
    gam = datagen.normal((D,), 1.0, seed=83)
    tg = dev(gam, "f32")
    y, r = ge.rmsnorm_fwd(dev(x, "f32"), 1e-5, gamma=tg)
    y_ref, r_ref = oracle.rmsnorm_fwd(x, 1e-5, gamma=gam)
    assert_parity(host(y), y_ref, TOL_F32, "f32", "y")
    dg = torch.empty(D, dtype=torch.float32, device="cuda")
    dx, dg = ge.rmsnorm_bwd(dev(x, "f32"), r, dev(dy, "f32"), gamma=tg, dgamma=dg)
    dx_ref, dg_ref = oracle.rmsnorm_bwd(x, host(r), dy, gamma=gam)
    assert_parity(host(dx), dx_ref, TOL_F32, "f32", "dx", cancel=True)
    assert_parity(host(dg), dg_ref, TOL_F32, "f32", "dgamma", cancel=True)


@pytest.mark.parametrize("n", [1, 7, 203530, 5824522])
@pytest.mark.parametrize("lowp", [None, "f16", "bf16"])
def test_sgd_momentum(ge, pins, n, lowp):
    w = datagen.normal((n,), 0.05, seed=n)
    g = datagen.normal((n,), 0.01, seed=n + 1)
    v = datagen.normal((n,), 0.001, seed=n + 2)
    tw, tg, tv = dev(w, "f32"), dev(g, "f32"), dev(v, "f32")
    tl = torch.empty(n, dtype=TD[lowp], device="cuda") if lowp else None
    ge.sgd_momentum(tw, tg, tv, pins["lr"], pins["momentum"], tl)
    w_ref, v_ref, wl_ref = oracle.sgd_momentum(w, g, v, pins["lr"], pins["momentum"], lowp)
    tol = pins["step_tol_abs"] + pins["step_tol_rel"] * np.abs(w_ref)
    assert np.all(np.abs(host(tw) - w_ref) <= tol)
    assert np.all(np.abs(host(tv) - v_ref) <= pins["step_tol_abs"] + pins["step_tol_rel"] * np.abs(v_ref))
    if lowp:
        # the working copy is the rounding of the GPU's own new FP32 weights
        np.testing.assert_array_equal(host(tl), oracle.round_fmt(host(tw), lowp))


@pytest.mark.parametrize("fmt", ["f32", "f16"])
@pytest.mark.parametrize("shape", [(100, 37), (5000, 1003), (4096, 4096), (3000, 8200)])
def test_colsum_accumulate(ge, fmt, shape):
    """accumulate adds the column sums to what out holds (both the one-pass
    and the two-pass reduction)."""
    X = datagen.normal(shape, 1.0, seed=shape[0] + 7, fmt=fmt)
    base = datagen.normal((shape[1],), 1.0, seed=shape[1] + 8)
    out = dev(base, "f32")
    ge.colsum(dev(X, fmt), 0.5, out=out, accumulate=True)
    ref = oracle.round_fmt(base + oracle.colsum(X, 0.5, out_fmt="f64"), "f32")
    assert_parity(host(out), ref, TOL_F32 if fmt == "f32" else TOL_LOWP, "f32", f"colsum acc {shape} {fmt}",
                  cancel=True)


def test_softmax_xent_bad_label_count(ge):
    """Labels outside [0, C) are counted (and give NaN row losses); valid
    rows are unaffected."""
    B, C = 300, 10
    Z = datagen.normal((B, C), 2.0, seed=91, fmt="f32")
    y = datagen.rng(92, "labels").integers(0, C, size=B).astype(np.int32)
    y[[3, 77, 150]] = [-1, 10, 1 << 20]
    bad = torch.full((1,), -5, dtype=torch.int32, device="cuda")
    loss, rl, dZ, am = ge.softmax_xent_fwd_bwd(dev(Z, "f32"), torch.from_numpy(y).cuda(), 1.0 / B,
                                               bad_label_count=bad)
    assert int(bad.item()) == 3
    r = host(rl)
    assert np.all(np.isnan(r[[3, 77, 150]]))
    ok = np.ones(B, bool)
    ok[[3, 77, 150]] = False
    ref = oracle.softmax_xent(Z[ok], y[ok], 1.0 / B, "f32")
    assert_parity(r[ok], ref[1], TOL_F32, "f32", "row loss with bad labels present")
    y2 = np.clip(y, 0, C - 1)
    ge.softmax_xent_fwd_bwd(dev(Z, "f32"), torch.from_numpy(y2).cuda(), 1.0 / B, bad_label_count=bad)
    assert int(bad.item()) == 0


@pytest.mark.parametrize("n", [1, 7, 203530, 5824522])
@pytest.mark.parametrize("lowp", ["f16", "bf16"])
def test_params_to_lowp(ge, n, lowp):
    """The working copy is the round-to-nearest-even conversion of each value."""
    w = datagen.normal((n,), 0.05, seed=n + 3)
    w[:min(n, 4)] = [65520.0, -1e-8, 3.0e38, 0.0][:min(n, 4)]     # overflow, subnormal, bf16 range, zero
    w = datagen.representable(w, "f32")
    tl = torch.empty(n, dtype=TD[lowp], device="cuda")
    ge.params_to_lowp(dev(w, "f32"), tl)
    np.testing.assert_array_equal(host(tl), oracle.round_fmt(w, lowp))
