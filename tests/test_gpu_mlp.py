"""GPU parity of mlp_train_step: the 784-256-10 FP32 epoch and the
784-2048-2048-10 FP16 step, lock-step against the oracle (each step starts
from the GPU's own pre-step parameters and velocity)."""
import numpy as np
import pytest
import torch

import datagen
import oracle
from parity import TOL_F32, TOL_LOSS, TOL_LOWP, assert_parity, compare

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ge():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import gemm_epilogue_amd
    return gemm_epilogue_amd


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _check_step(tr, dims, X, y, lr, mu, plan, w0, v0, tie_abs, what):
    """Stage-wise check: every stored tensor against the oracle applied to the
    stored inputs that stage consumed (strict rule); then the oracle's own
    end-to-end step, where one-ulp storage differences propagate (reported,
    loosely bounded)."""
    B = X.shape[0]
    ws = tr.workspace_views(B)
    torch.cuda.synchronize()
    fmt = "f32" if plan == "f32" else "f16"
    tol = TOL_F32 if plan == "f32" else TOL_LOWP
    H_gpu = [host(h) for h in ws["H"]]
    Z = host(ws["Z"])
    given = {"H": H_gpu, "Z": Z, "G": host(ws["G"]), "dH": [host(h) for h in ws["dH"]]}
    ref = oracle.mlp_step(w0, v0, dims, X, y, lr, mu, plan=plan, given=given)
    loss = host(tr.loss)[0]
    assert abs(loss - ref["loss"]) <= TOL_LOSS * abs(ref["loss"]), (what, loss, ref["loss"])
    for i, (hg, hr) in enumerate(zip(H_gpu, ref["H"])):
        assert_parity(hg, hr, tol, fmt, f"{what} H{i + 1}")
    assert_parity(Z, ref["Z"], tol, "f32", f"{what} Z")
    assert_parity(given["G"], ref["G"], tol, fmt, f"{what} G")
    for i, (dg, dr) in enumerate(zip(given["dH"], ref["dH"])):
        assert_parity(dg, dr, tol, fmt, f"{what} dH{i + 1}")
    assert_parity(host(tr.grads), ref["grads"], tol, "f32", f"{what} grads")
    assert_parity(host(tr.velocity), ref["vel"], tol, "f32", f"{what} velocity")
    assert_parity(host(tr.params), ref["params"], tol, "f32", f"{what} params")
    if plan == "f16":
        np.testing.assert_array_equal(host(tr.params_lowp), oracle.round_fmt(host(tr.params), "f16"))
    srt = np.sort(ref["Z"], axis=1)
    gap = srt[:, -1] - srt[:, -2]
    pred = Z.argmax(axis=1)
    assert np.all((pred == ref["argmax"]) | (gap < 1e-4)), what
    # end to end from the pre-step state, the oracle's own intermediates
    e2e = oracle.mlp_step(w0, v0, dims, X, y, lr, mu, plan=plan, mask_hint=H_gpu, tie_abs=tie_abs)
    rl = abs(loss - e2e["loss"]) / abs(e2e["loss"])
    gc = compare(host(tr.grads), e2e["grads"], tol, "f32")
    print(f"{what}: end-to-end loss rel diff {rl:.2e}, grads cos {gc['cos']:.9f}, "
          f"mask ties adopted {e2e['mask_ties']}")
    assert rl < 1e-3 and gc["cos"] > 0.99999, what
    assert_parity(host(tr.params), e2e["params"], tol, "f32", f"{what} params end-to-end")
    return ref


def test_cfg0_epoch_lockstep(ge, pins):
    """One epoch of the 784-256-10 FP32 net: 46 batches of 128 and one of 112."""
    dims = datagen.mlp_dims_cfg0()
    lr, mu, bs = pins["lr"], pins["momentum"], pins["batch"]
    Xall, yall = datagen.template_images(6000, 100, fmt="f32")
    p0 = datagen.he_uniform_flat(dims)
    tr = ge.MLPTrainer(dims, bs, torch.float32, params=torch.from_numpy(p0).float().cuda())
    tX = torch.from_numpy(Xall).float().cuda()
    ty = torch.from_numpy(yall).cuda()
    n_steps = 0
    for s in range(0, 6000, bs):
        e = min(6000, s + bs)
        w0, v0 = host(tr.params), host(tr.velocity)
        tr.step(tX[s:e], ty[s:e], lr, mu)
        _check_step(tr, dims, Xall[s:e], yall[s:e], lr, mu, "f32", w0, v0, 1e-6, f"step {n_steps}")
        n_steps += 1
    assert n_steps == 47


def test_cfg0_free_running_loss(ge, pins):
    """Independent trajectories (GPU vs oracle, both from the initial weights):
    the loss curve is reported; errors compound, so only drift is bounded."""
    dims = datagen.mlp_dims_cfg0()
    lr, mu, bs = pins["lr"], pins["momentum"], pins["batch"]
    Xall, yall = datagen.template_images(6000, 100, fmt="f32")
    p0 = datagen.he_uniform_flat(dims)
    tr = ge.MLPTrainer(dims, bs, torch.float32, params=torch.from_numpy(p0).float().cuda())
    tX = torch.from_numpy(Xall).float().cuda()
    ty = torch.from_numpy(yall).cuda()
    w, v = p0.copy(), np.zeros_like(p0)
    worst = 0.0
    for s in range(0, 6000, bs):
        e = min(6000, s + bs)
        tr.step(tX[s:e], ty[s:e], lr, mu)
        ref = oracle.mlp_step(w, v, dims, Xall[s:e], yall[s:e], lr, mu, plan="f32")
        w, v = ref["params"], ref["vel"]
        worst = max(worst, abs(host(tr.loss)[0] - ref["loss"]) / ref["loss"])
    print(f"free-running worst relative loss drift over the epoch: {worst:.3e}")
    assert worst < 1e-2


def test_overfit_32(ge, pins):
    dims = datagen.mlp_dims_cfg0()
    X, y = datagen.template_images(pins["overfit_images"], 14)
    p0 = datagen.he_uniform_flat(dims)
    tr = ge.MLPTrainer(dims, 32, torch.float32, params=torch.from_numpy(p0).float().cuda())
    tX, ty = torch.from_numpy(X).float().cuda(), torch.from_numpy(y).cuda()
    for _ in range(pins["overfit_steps"]):
        tr.step(tX, ty, pins["lr"], pins["momentum"])
    tr.step(tX, ty, 0.0, 0.0)
    assert host(tr.loss)[0] < pins["overfit_loss_below"]


def test_cfg2_step_lockstep(ge):
    """784-2048-2048-10, FP16 storage, batch 4096, lr 0.05, momentum 0.9: two steps."""
    dims = datagen.mlp_dims_cfg2()
    B, lr, mu = 4096, 0.05, 0.9
    p0 = datagen.he_uniform_flat(dims)
    tr = ge.MLPTrainer(dims, B, torch.float16, params=torch.from_numpy(p0).float().cuda())
    for step in range(2):
        X, y = datagen.template_images(B, 200, fmt="f16", batch=step)
        w0, v0 = host(tr.params), host(tr.velocity)
        print(f"cfg2 step {step}", flush=True)
        tr.step(torch.from_numpy(X).half().cuda(), torch.from_numpy(y).cuda(), lr, mu)
        _check_step(tr, dims, X, y, lr, mu, "f16", w0, v0, 1e-5, f"cfg2 step {step}")


def test_mlp_step_deterministic(ge):
    dims = [784, 512, 512, 10]
    X, y = datagen.template_images(1000, 9, fmt="f16")
    p0 = torch.from_numpy(datagen.he_uniform_flat(dims)).float().cuda()
    outs = []
    for _ in range(2):
        tr = ge.MLPTrainer(dims, 1000, torch.float16, params=p0)
        for _ in range(3):
            tr.step(torch.from_numpy(X).half().cuda(), torch.from_numpy(y).cuda(), 0.05, 0.9)
        outs.append(tr.params.clone())
    assert torch.equal(outs[0], outs[1])
