"""Pins for the oracle's composite steps: MLP, transformer MLP block, GRU LM (CPU only)."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import datagen
from oracle import (block_fwd_bwd, gru_flatten, gru_loss_only, gru_param_count,
                    gru_step, gru_unflatten, mlp_loss_only, mlp_param_count, mlp_step,
                    mlp_unflatten)


# ---------------------------------------------------------------- MLP ------

def test_param_counts(pins):
    assert mlp_param_count([784, 256, 10]) == pins["param_count_784_256_10"]
    assert mlp_param_count([784, 2048, 2048, 10]) == 5_824_522
    assert gru_param_count(1024, 256) == 6_822_144


def test_zero_weights_loss_ln10():
    dims = [784, 256, 10]
    x, y = datagen.template_images(16, 11)
    out = mlp_step(np.zeros(mlp_param_count(dims)), np.zeros(mlp_param_count(dims)),
                   dims, x, y, 0.1, 0.9, plan="f64")
    assert out["loss"] == pytest.approx(math.log(10), rel=1e-15)
    (W1, b1), (W2, b2) = mlp_unflatten(out["grads"], dims)
    assert np.all(W1 == 0) and np.all(W2 == 0) and np.all(b1 == 0)
    onehot = np.eye(10)[y]
    np.testing.assert_allclose(b2, (0.1 - onehot).mean(axis=0), atol=1e-16)


def _relu_safe_fd(params, dims, X, y, idx, h=1e-6):
    gp = params.copy(); gp[idx] += h
    gm = params.copy(); gm[idx] -= h
    return (mlp_loss_only(gp, dims, X, y) - mlp_loss_only(gm, dims, X, y)) / (2 * h)


def test_mlp_gradient_finite_differences_tiny():
    dims = [6, 5, 3]
    g = np.random.default_rng(12)
    p = g.normal(scale=0.7, size=mlp_param_count(dims))
    X = g.normal(size=(4, 6)); y = np.array([0, 2, 1, 2])
    out = mlp_step(p, np.zeros_like(p), dims, X, y, 0.0, 0.0, plan="f64")
    pre = out["pre"][0]
    assert np.abs(pre).min() > 1e-3            # no kink within the FD step
    fd = np.array([_relu_safe_fd(p, dims, X, y, i) for i in range(p.size)])
    np.testing.assert_allclose(out["grads"], fd, rtol=1e-6, atol=1e-9)


def test_mlp_gradient_200_coordinates(pins):
    dims = [784, 256, 10]
    p = datagen.he_uniform_flat(dims)
    X, y = datagen.template_images(32, 13)
    out = mlp_step(p, np.zeros_like(p), dims, X, y, 0.0, 0.0, plan="f64")
    g = np.random.default_rng(pins["weight_seed"])
    idx = g.choice(p.size, size=pins["grad_check_coords"], replace=False)
    fd = np.array([_relu_safe_fd(p, dims, X, y, i, h=1e-5) for i in idx])
    an = out["grads"][idx]
    np.testing.assert_allclose(an, fd, rtol=1e-4, atol=1e-8)


def test_mlp_overfit_32(pins):
    dims = [784, 256, 10]
    p = datagen.he_uniform_flat(dims)
    v = np.zeros_like(p)
    X, y = datagen.template_images(pins["overfit_images"], 14)
    for _ in range(pins["overfit_steps"]):
        out = mlp_step(p, v, dims, X, y, pins["lr"], pins["momentum"], plan="f32")
        p, v = out["params"], out["vel"]
    final = mlp_step(p, v, dims, X, y, 0.0, 0.0, plan="f32")["loss"]
    assert final < pins["overfit_loss_below"]


def test_mlp_f16_plan_close_to_f64():
    dims = [784, 64, 64, 10]
    p = datagen.he_uniform_flat(dims)
    X, y = datagen.template_images(64, 15, fmt="f16")
    a = mlp_step(p, np.zeros_like(p), dims, X, y, 0.05, 0.9, plan="f16")
    b = mlp_step(p, np.zeros_like(p), dims, X, y, 0.05, 0.9, plan="f64")
    assert a["loss"] == pytest.approx(b["loss"], rel=2e-3)
    cos = a["grads"] @ b["grads"] / np.linalg.norm(a["grads"]) / np.linalg.norm(b["grads"])
    assert cos > 0.9999
    assert np.all(a["params_lowp"] == np.asarray(a["params_lowp"], np.float16).astype(np.float64))


def test_mlp_mask_hint_adopts_tie_bits():
    dims = [5, 4, 3]
    g = np.random.default_rng(16)
    p = g.normal(size=mlp_param_count(dims)); X = g.normal(size=(3, 5)); y = np.array([0, 1, 2])
    base = mlp_step(p, np.zeros_like(p), dims, X, y, 0.0, 0.0, plan="f64")
    pre = base["pre"][0]
    flip = np.zeros_like(pre); flip.flat[np.argmin(np.abs(pre))] = 1
    hint = np.where(flip > 0, np.where(pre > 0, 0.0, 1e-9), base["H"][0])
    tied = mlp_step(p, np.zeros_like(p), dims, X, y, 0.0, 0.0, plan="f64",
                    mask_hint=[hint], tie_abs=np.abs(pre).min() * 1.0001)
    assert tied["mask_ties"] == 1
    assert not np.allclose(tied["grads"], base["grads"])


# -------------------------------------------------------------- block ------

def _torch_block(x, wu, wd, dy, eps, slope):
    tx = torch.from_numpy(x).requires_grad_()
    tu = torch.from_numpy(wu).requires_grad_()
    td = torch.from_numpy(wd).requires_grad_()
    n = F.rms_norm(tx, (x.shape[1],), eps=eps)
    u = n @ tu
    a = F.leaky_relu(u, slope) ** 2
    y = tx + a @ td
    (y * torch.from_numpy(dy)).sum().backward()
    return y.detach().numpy(), tx.grad.numpy(), tu.grad.numpy(), td.grad.numpy()


def test_block_matches_torch_autograd_f64():
    g = np.random.default_rng(17)
    R, D, Fh = 5, 8, 12
    x = g.normal(size=(R, D)); wu = g.normal(scale=0.3, size=(D, Fh))
    wd = g.normal(scale=0.3, size=(Fh, D)); dy = g.normal(size=(R, D))
    o = block_fwd_bwd(x, wu, wd, dy, eps=1e-6, slope=0.5, fmt="f64")
    y, dx, dwu, dwd = _torch_block(x, wu, wd, dy, 1e-6, 0.5)
    np.testing.assert_allclose(o["y"], y, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(o["dx"], dx, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(o["dW_up"], dwu, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(o["dW_down"], dwd, rtol=1e-10, atol=1e-12)


def test_block_finite_differences():
    g = np.random.default_rng(18)
    R, D, Fh = 3, 4, 6
    x = g.normal(size=(R, D)); wu = g.normal(scale=0.5, size=(D, Fh))
    wd = g.normal(scale=0.5, size=(Fh, D)); dy = g.normal(size=(R, D))
    o = block_fwd_bwd(x, wu, wd, dy, eps=1e-6, fmt="f64")
    L = lambda xx, a, b: (block_fwd_bwd(xx, a, b, dy, eps=1e-6, fmt="f64")["y"] * dy).sum()
    h = 1e-6
    for name, arr, grad in (("x", x, o["dx"]), ("wu", wu, o["dW_up"]), ("wd", wd, o["dW_down"])):
        fd = np.zeros_like(arr)
        for i in np.ndindex(arr.shape):
            ap = arr.copy(); ap[i] += h
            am = arr.copy(); am[i] -= h
            args_p = {"x": (ap, wu, wd), "wu": (x, ap, wd), "wd": (x, wu, ap)}[name]
            args_m = {"x": (am, wu, wd), "wu": (x, am, wd), "wd": (x, wu, am)}[name]
            fd[i] = (L(*args_p) - L(*args_m)) / (2 * h)
        np.testing.assert_allclose(grad, fd, rtol=1e-6, atol=1e-8)


def test_block_zero_down_projection():
    x, wu, wd, dy = datagen.block_inputs(16, D=32, F=48)
    o = block_fwd_bwd(x, wu, np.zeros_like(wd), dy, fmt="bf16")
    np.testing.assert_array_equal(o["y"], x)
    np.testing.assert_array_equal(o["du"], 0.0)
    np.testing.assert_array_equal(o["dW_up"], 0.0)
    np.testing.assert_array_equal(o["dx"], dy)


# ---------------------------------------------------------------- GRU ------

def _small_gru(H=8, V=16, seed=19, scale=1.0):
    g = np.random.default_rng(seed)
    P = {"E": g.normal(size=(V, H)), "W_i": g.normal(scale=0.4 * scale, size=(H, 3 * H)),
         "b_i": g.normal(scale=0.1, size=3 * H), "W_h": g.normal(scale=0.4 * scale, size=(H, 3 * H)),
         "b_h": g.normal(scale=0.1, size=3 * H), "W_c": g.normal(scale=0.4, size=(H, V)),
         "b_c": g.normal(scale=0.1, size=V)}
    return P


def test_gru_zero_weights_loss_ln256():
    H, V = 32, 256
    tok = datagen.zipf_tokens(3, 6)
    flat = np.zeros(gru_param_count(H, V))
    o = gru_step(flat, np.zeros_like(flat), tok, H, V, 0.0, 0.0, plan="f64", update=False)
    assert o["loss"] == pytest.approx(math.log(256), rel=1e-15)
    assert np.all(o["hs"] == 0)


def test_gru_matches_torch_f64():
    H, V, Bn, T = 8, 16, 3, 5
    P = _small_gru(H, V)
    tok = np.random.default_rng(20).integers(0, V, size=(Bn, T + 1))
    flat = gru_flatten(P)
    o = gru_step(flat, np.zeros_like(flat), tok, H, V, 0.0, 0.0, eps=1e-6, plan="f64",
                 update=False)
    tp = {k: torch.from_numpy(v.copy()).requires_grad_() for k, v in P.items()}
    xin = tp["E"][torch.from_numpy(tok[:, :T].T.copy()).long()]           # [T, B, H]
    out, _ = torch._VF.gru(xin, torch.zeros(1, Bn, H, dtype=torch.float64),
                           [tp["W_i"].t(), tp["W_h"].t(), tp["b_i"], tp["b_h"]],
                           True, 1, 0.0, False, False, False)
    hs = out.reshape(T * Bn, H)
    np.testing.assert_allclose(o["hs"], hs.detach().numpy(), rtol=1e-12, atol=1e-13)
    hn = F.rms_norm(hs, (H,), eps=1e-6)
    Z = hn @ tp["W_c"] + tp["b_c"]
    loss = F.cross_entropy(Z, torch.from_numpy(tok[:, 1:].T.reshape(-1).copy()).long())
    loss.backward()
    assert o["loss"] == pytest.approx(loss.item(), rel=1e-13)
    mine = gru_unflatten(o["grads"], H, V)
    for k in P:
        np.testing.assert_allclose(mine[k], tp[k].grad.numpy(), rtol=1e-9, atol=1e-12,
                                   err_msg=k)


def test_gru_finite_differences_sample():
    H, V, Bn, T = 6, 10, 2, 4
    P = _small_gru(H, V, seed=21)
    tok = np.random.default_rng(22).integers(0, V, size=(Bn, T + 1))
    flat = gru_flatten(P)
    o = gru_step(flat, np.zeros_like(flat), tok, H, V, 0.0, 0.0, plan="f64", update=False)
    idx = np.random.default_rng(23).choice(flat.size, size=60, replace=False)
    h = 1e-6
    for i in idx:
        fp = flat.copy(); fp[i] += h
        fm = flat.copy(); fm[i] -= h
        fd = (gru_loss_only(fp, tok, H, V) - gru_loss_only(fm, tok, H, V)) / (2 * h)
        assert o["grads"][i] == pytest.approx(fd, rel=1e-5, abs=1e-9)


def test_gru_f16_plan_close_to_f64():
    H, V, Bn, T = 64, 256, 4, 12
    P = datagen.gru_params(H, V)
    tok = datagen.zipf_tokens(Bn, T + 1)
    flat = gru_flatten(P)
    a = gru_step(flat, np.zeros_like(flat), tok, H, V, 0.01, 0.9, plan="f16")
    b = gru_step(flat, np.zeros_like(flat), tok, H, V, 0.01, 0.9, plan="f64")
    assert a["loss"] == pytest.approx(b["loss"], rel=1e-3)
    cos = a["grads"] @ b["grads"] / np.linalg.norm(a["grads"]) / np.linalg.norm(b["grads"])
    assert cos > 0.999


# ------------------------------------------- stage-wise (given=) mode ------
# The stage-wise mode feeds each stage the stored inputs it consumed.  Pins:
# fed the oracle's own intermediates it reproduces the plain step exactly, and
# a given tensor is only ever an input -- never handed back as an output.

def _same(a, b, what):
    if isinstance(a, (list, tuple)):
        assert len(a) == len(b), what
        for i, (x, y) in enumerate(zip(a, b)):
            _same(x, y, f"{what}[{i}]")
    elif a is None or isinstance(a, (int, float, np.integer, np.floating)):
        assert a == b, what
    else:
        np.testing.assert_array_equal(np.asarray(a), np.asarray(b), err_msg=what)


@pytest.mark.parametrize("plan,dims", [("f32", [30, 12, 9, 5]), ("f16", [24, 16, 8, 10])])
def test_mlp_given_own_intermediates_reproduces_plain(plan, dims):
    p = datagen.he_uniform_flat(dims)
    g = np.random.default_rng(31)
    X = datagen.representable(g.normal(size=(7, dims[0])), plan)
    y = g.integers(0, dims[-1], size=7)
    v = datagen.representable(g.normal(scale=1e-3, size=p.size), "f32")
    plain = mlp_step(p, v, dims, X, y, 0.05, 0.9, plan=plan)
    given = {"H": plain["H"], "Z": plain["Z"], "G": plain["G"], "dH": plain["dH"]}
    staged = mlp_step(p, v, dims, X, y, 0.05, 0.9, plan=plan, given=given)
    for k in ("loss", "row_loss", "Z", "G", "argmax", "H", "pre", "dH", "grads", "params", "vel",
              "params_lowp"):
        _same(staged[k], plain[k], k)


def test_mlp_given_is_never_returned():
    dims = [20, 9, 7, 6]
    p = datagen.he_uniform_flat(dims)
    g = np.random.default_rng(32)
    X = g.normal(size=(5, 20))
    y = g.integers(0, 6, size=5)
    plain = mlp_step(p, np.zeros_like(p), dims, X, y, 0.0, 0.0, plan="f32")
    # all 7s: layer 2's input and the loss stage's input are perturbed; the
    # given Z's dominant column is one the oracle's own Z never picks
    H = [plain["H"][0], np.full_like(plain["H"][1], 7.0)]
    W3, b3 = mlp_unflatten(p, dims)[2]
    col = int(np.argmin(np.full(7, 7.0) @ W3 + b3))
    Zg = np.zeros_like(plain["Z"])
    Zg[:, col] = 50.0
    staged = mlp_step(p, np.zeros_like(p), dims, X, y, 0.0, 0.0, plan="f32",
                      given={"H": H, "Z": Zg})
    # returned H are the oracle's own layer outputs from the given inputs of
    # each layer: H1 from X and H2 from the given H1 are unchanged
    _same(staged["H"], plain["H"], "H")
    assert not np.any(staged["H"][1] == 7.0)
    # Z is the output layer applied to the given (perturbed) H2
    assert not np.allclose(staged["Z"], plain["Z"])
    ref_Z = np.asarray(np.float32(np.full((5, 7), 7.0) @ W3 + b3), np.float64)
    np.testing.assert_allclose(staged["Z"], ref_Z, rtol=1e-6)
    # argmax comes from the oracle's own Z, never from the given one
    np.testing.assert_array_equal(staged["argmax"], staged["Z"].argmax(axis=1))
    assert not np.any(staged["argmax"] == col)
    # the loss stage is applied to the given Z: that column dominates every row
    np.testing.assert_allclose(staged["row_loss"], np.where(y == col, 0.0, 50.0), atol=1e-12)


def test_block_given_own_intermediates_reproduces_plain():
    x, wu, wd, dy = datagen.block_inputs(24, D=16, F=40, seed=33)
    plain = block_fwd_bwd(x, wu, wd, dy, fmt="bf16")
    staged = block_fwd_bwd(x, wu, wd, dy, fmt="bf16",
                           given={k: plain[k] for k in ("r", "n", "u", "a", "du", "dn")})
    for k in plain:
        _same(staged[k], plain[k], k)


def test_block_given_is_never_returned():
    x, wu, wd, dy = datagen.block_inputs(24, D=16, F=40, seed=34)
    plain = block_fwd_bwd(x, wu, wd, dy, fmt="bf16")
    staged = block_fwd_bwd(x, wu, wd, dy, fmt="bf16", given={"u": plain["u"] + 1.0})
    _same(staged["u"], plain["u"], "u")
    assert not np.array_equal(staged["du"], plain["du"])     # du consumes the given u


def test_gru_given_own_intermediates_reproduces_plain():
    H, V, Bn, T = 12, 20, 3, 5
    P = datagen.gru_params(H, V)
    tok = datagen.zipf_tokens(Bn, T + 1, seed=35, vocab=V)
    flat = datagen.representable(gru_flatten(P), "f32")
    v = np.zeros_like(flat)
    plain = gru_step(flat, v, tok, H, V, 0.01, 0.9, plan="f16")
    GH = np.concatenate([np.zeros((T * Bn, 2 * H)), plain["GHn"]], axis=1)
    given = {"hs": plain["hs"], "R": plain["R"], "Z": plain["Zg"], "N": plain["N"], "GH": GH,
             "rstd": plain["rstd"], "hn": plain["hn"], "logits": plain["logits"], "G": plain["G"],
             "dhn": plain["dhn"], "dh_out": plain["dh_out"], "dGH": plain["dGH"],
             "dGI": plain["dGI"], "dX": plain["dX"]}
    staged = gru_step(flat, v, tok, H, V, 0.01, 0.9, plan="f16", given=given)
    for k in plain:
        _same(staged[k], plain[k], k)


def test_gru_given_is_never_returned():
    H, V, Bn, T = 12, 20, 3, 5
    P = datagen.gru_params(H, V)
    tok = datagen.zipf_tokens(Bn, T + 1, seed=36, vocab=V)
    flat = datagen.representable(gru_flatten(P), "f32")
    plain = gru_step(flat, np.zeros_like(flat), tok, H, V, 0.0, 0.0, plan="f16", update=False)
    staged = gru_step(flat, np.zeros_like(flat), tok, H, V, 0.0, 0.0, plan="f16", update=False,
                      given={"hs": plain["hs"] * 0.5, "logits": plain["logits"] + 3.0})
    # the recurrence output at t=0 does not depend on a given h; later steps
    # start from the given (halved) h_{t-1}, so they differ, but none equals it
    _same(staged["hs"][:Bn], plain["hs"][:Bn], "hs t=0")
    assert not np.allclose(staged["hs"][Bn:], plain["hs"][Bn:] * 0.5)
    # logits are the classifier of the oracle's own hn of the given hs
    assert not np.allclose(staged["logits"], plain["logits"] + 3.0)


def test_gru_gates_bwd_is_the_gradient_of_gates_fwd():
    """gru_gates_bwd against torch float64 autograd of gru_gates_fwd: with GI,
    GH and h_prev independent inputs, dGI = dL/dGI, dGH = dL/dGH and
    dh_dir = dL/dh_prev for L = sum(dh * h)."""
    from oracle import gru_gates_bwd, gru_gates_fwd
    g = np.random.default_rng(37)
    B, H = 5, 7
    GI, GH = g.normal(size=(B, 3 * H)), g.normal(size=(B, 3 * H))
    hp, dh = g.normal(size=(B, H)), g.normal(size=(B, H))
    tGI, tGH, thp = (torch.from_numpy(a.copy()).requires_grad_() for a in (GI, GH, hp))
    r = torch.sigmoid(tGI[:, :H] + tGH[:, :H])
    z = torch.sigmoid(tGI[:, H:2 * H] + tGH[:, H:2 * H])
    n = torch.tanh(tGI[:, 2 * H:] + r * tGH[:, 2 * H:])
    h = (1 - z) * n + z * thp
    (h * torch.from_numpy(dh)).sum().backward()
    rr, zz, nn, hh = gru_gates_fwd(GI, GH, hp)
    np.testing.assert_allclose(hh, h.detach().numpy(), rtol=1e-14, atol=1e-15)
    dGH, dGI, dd = gru_gates_bwd(dh, rr, zz, nn, GH[:, 2 * H:], hp)
    np.testing.assert_allclose(dGI, tGI.grad.numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dGH, tGH.grad.numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dd, thp.grad.numpy(), rtol=1e-12, atol=1e-14)
