"""GPU parity of the byte-level GRU LM step (gru_lm_train_step) and the
embedding entry points, against the oracle."""
import math

import numpy as np
import pytest
import torch

import datagen
import oracle
from parity import TOL_LOSS, TOL_LOWP, assert_parity, compare

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ge():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import gemm_epilogue_amd
    return gemm_epilogue_amd


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


# GPU workspace name -> (oracle name, storage format)
STAGES = {"GI": ("GI", "f32"), "HS": ("hs", "f32"), "R": ("R", "f32"), "Z": ("Zg", "f32"),
          "N": ("N", "f32"), "HN": ("hn", "f16"), "RSTD": ("rstd", "f32"), "LOGITS": ("logits", "f32"),
          "G": ("G", "f16"), "DHN": ("dhn", "f32"), "DH_OUT": ("dh_out", "f32"), "DGH": ("dGH", "f16"),
          "DGI": ("dGI", "f16"), "DX": ("dX", "f32")}
# stages whose values are formed from cancelling sums (GEMM outputs, the
# recurrence mix (1-z) n + z h, tanh of GI_n + r GH_n, the RMSNorm input
# gradient, the carried gate gradients); r, z (sigmoids), hn, rstd and the
# softmax gradient are held to the plain rule
NO_CANCEL = ("R", "Z", "HN", "RSTD", "G")
GIVEN = {"HS": "hs", "R": "R", "Z": "Z", "N": "N", "GH": "GH", "RSTD": "rstd", "HN": "hn",
         "LOGITS": "logits", "G": "G", "DHN": "dhn", "DH_OUT": "dh_out", "DGH": "dGH", "DGI": "dGI",
         "DX": "dX"}


def _run_and_check(ge, V, H, B, T, lr, mu, params, what, steps=1, recurrence="auto"):
    tok = datagen.zipf_tokens(B, T + 1, seed=B + T, vocab=V)
    flat = datagen.representable(params, "f32")
    tr = ge.GRUTrainer(V, H, B, T, eps=1e-6, params=torch.from_numpy(flat).float().cuda(), recurrence=recurrence)
    vel = np.zeros_like(flat)
    for s in range(steps):
        w0, v0 = host(tr.params), host(tr.velocity)
        tr.step(torch.from_numpy(tok).cuda(), lr, mu)
        torch.cuda.synchronize()
        got = {k: host(tr.view(k)) for k in list(STAGES) + ["GH"]}
        given = {GIVEN[k]: got[k] for k in GIVEN}
        print(f"{what} step {s}: oracle", flush=True)
        ref = oracle.gru_step(w0, v0, tok, H, V, lr, mu, eps=1e-6, plan="f16", given=given)
        loss = host(tr.loss)[0]
        assert abs(loss - ref["loss"]) <= TOL_LOSS * abs(ref["loss"]), (what, loss, ref["loss"])
        for k, (rk, fmt) in STAGES.items():
            assert_parity(got[k], ref[rk], TOL_LOWP, fmt, f"{what} {k}", cancel=k not in NO_CANCEL)
        assert_parity(host(tr.grads), ref["grads"], TOL_LOWP, "f32", f"{what} grads", cancel=True)
        assert_parity(host(tr.params), ref["params"], TOL_LOWP, "f32", f"{what} params", cancel=True)
        np.testing.assert_array_equal(host(tr.params_lowp), oracle.round_fmt(host(tr.params), "f16"))
        # end to end from the pre-step state (oracle's own intermediates): reported
        e2e = oracle.gru_step(w0, v0, tok, H, V, lr, mu, eps=1e-6, plan="f16")
        rl = abs(loss - e2e["loss"]) / e2e["loss"]
        c = compare(host(tr.grads), e2e["grads"], TOL_LOWP, "f32", cancel=True)
        print(f"{what} step {s}: end-to-end loss rel diff {rl:.2e}, grads cos {c['cos']:.8f}")
        assert rl < 1e-3 and c["cos"] > 0.9999
    return tr


def test_gru_small_ragged(ge):
    V, H, B, T = 100, 68, 3, 7
    p = oracle.gru_flatten(datagen.gru_params(H, V))
    _run_and_check(ge, V, H, B, T, 0.01, 0.9, p, "small", steps=2)


@pytest.mark.parametrize("recurrence", ["persistent", "stepwise"])
def test_gru_full_size(ge, recurrence):
    """Byte vocabulary 256, hidden 1024, batch 64, sequence 128, lr 0.01,
    momentum 0.9, with the persistent recurrence (W_h resident in LDS, one
    launch per direction) and with one GEMM and one gate launch per timestep."""
    V, H, B, T = 256, 1024, 64, 128
    p = oracle.gru_flatten(datagen.gru_params(H, V))
    _run_and_check(ge, V, H, B, T, 0.01, 0.9, p, f"cfg4 {recurrence}", recurrence=recurrence)


@pytest.mark.parametrize("H,B,T", [(256, 16, 9), (768, 48, 5)])
def test_gru_persistent_small(ge, H, B, T):
    """The persistent recurrence at the smallest size it takes (B 16, H 256:
    one row group of 16 blocks) and at H 768, B 48 (three row groups, each
    with a barrier of its own), two steps, lock-step against the oracle."""
    V = 97
    p = oracle.gru_flatten(datagen.gru_params(H, V))
    _run_and_check(ge, V, H, B, T, 0.01, 0.9, p, f"persistent H{H} B{B}", steps=2, recurrence="persistent")


def test_gru_persistent_refuses_unsupported_sizes(ge):
    from gemm_epilogue_amd._lib import GEError
    tr = ge.GRUTrainer(100, 68, 3, 7, recurrence="persistent")
    tok = torch.from_numpy(datagen.zipf_tokens(3, 8, seed=1, vocab=100)).cuda()
    with pytest.raises(GEError, match="persistent"):
        tr.step(tok, 0.01, 0.9)


def test_gru_zero_weights_ln256(ge):
    V, H, B, T = 256, 64, 4, 9
    tr = ge.GRUTrainer(V, H, B, T)
    tok = datagen.zipf_tokens(B, T + 1, seed=5)
    tr.step(torch.from_numpy(tok).cuda(), 0.0, 0.0)
    assert abs(host(tr.loss)[0] - math.log(256)) <= 1e-6 * math.log(256)
    assert torch.all(tr.view("HS") == 0)


def test_embedding_gather_and_grad(ge):
    V, H, n = 37, 130, 1000
    E = datagen.normal((V, H), 1.0, seed=1, fmt="f16")
    idx = datagen.rng(2, "tokens").integers(-2, V + 2, size=n).astype(np.int32)   # some out of range
    tE = torch.from_numpy(E).half().cuda()
    ti = torch.from_numpy(idx).cuda()
    out = ge.embedding_gather(tE, ti)
    ok = (idx >= 0) & (idx < V)
    ref = np.where(ok[:, None], E[np.clip(idx, 0, V - 1)], 0.0)
    np.testing.assert_array_equal(host(out), ref)
    dX = datagen.normal((n, H), 1.0, seed=3)
    vi = np.clip(idx, 0, V - 1).astype(np.int32)
    g = ge.embedding_grad(torch.from_numpy(dX).float().cuda(), torch.from_numpy(vi).cuda(), V, 0.5)
    dE = np.zeros((V, H))
    np.add.at(dE, vi, dX)
    assert_parity(host(g), oracle.round_fmt(0.5 * dE, "f32"), 1e-4, "f32", "dE", cancel=True)
    g2 = ge.embedding_grad(torch.from_numpy(dX).float().cuda(), torch.from_numpy(vi).cuda(), V, 0.5)
    assert torch.equal(g, g2)


@pytest.mark.parametrize("B,H", [(3, 68), (64, 1024)])
def test_gru_gates_entry_points(ge, B, H):
    """gru_gates_fwd / gru_gates_bwd through the C ABI against the oracle's
    gate arithmetic, from the same stored inputs (with and without h_prev and
    carry)."""
    g = np.random.default_rng(B + H)
    f32 = lambda a: datagen.representable(a, "f32")
    GI, GH = f32(g.normal(size=(B, 3 * H))), f32(g.normal(size=(B, 3 * H)))
    hp, dho, carry = f32(g.normal(size=(B, H))), f32(g.normal(size=(B, H))), f32(g.normal(size=(B, H)))
    t = lambda a: torch.from_numpy(a).float().cuda()
    for with_state in (True, False):
        h16 = torch.empty((B, H), dtype=torch.float16, device="cuda")
        r, z, n, h, _ = ge.gru_gates_fwd(t(GI), t(GH), t(hp) if with_state else None, h_f16=h16)
        hp_ref = hp if with_state else np.zeros_like(hp)
        rr, zr, nr, hr = oracle.gru_gates_fwd(GI, GH, hp_ref)
        for name, got, ref, cancel in (("r", r, rr, False), ("z", z, zr, False), ("n", n, nr, True),
                                       ("h", h, hr, True)):
            assert_parity(host(got), oracle.round_fmt(ref, "f32"), 1e-4, "f32", f"gates fwd {name} B={B}",
                          cancel=cancel)
        np.testing.assert_array_equal(host(h16), oracle.round_fmt(host(h), "f16"))
        # backward from the GPU's stored r, z, n
        dGH, dGI, dd = ge.gru_gates_bwd(t(dho), t(carry) if with_state else None, r, z, n, t(GH),
                                        t(hp) if with_state else None)
        dh = dho + (carry if with_state else 0.0)
        gH, gI, gd = oracle.gru_gates_bwd(dh, host(r), host(z), host(n), GH[:, 2 * H:], hp_ref)
        assert_parity(host(dGH), oracle.round_fmt(gH, "f16"), 5e-3, "f16", f"gates dGH B={B}", cancel=True)
        assert_parity(host(dGI), oracle.round_fmt(gI, "f16"), 5e-3, "f16", f"gates dGI B={B}", cancel=True)
        assert_parity(host(dd), oracle.round_fmt(gd, "f32"), 1e-4, "f32", f"gates dh_dir B={B}")


def test_embedding_grad_zipf_full_size(ge):
    """8,192 positions (64 x 128) of Zipf(1.1) byte tokens, H = 1024: the most
    frequent byte holds ~20% of the rows, so its run spans every wave of its
    block; deterministic and against the oracle's scatter-add."""
    V, H = 256, 1024
    tok = datagen.zipf_tokens(64, 128, seed=41)
    idx = tok.T.reshape(-1).astype(np.int32)
    dX = datagen.normal((idx.size, H), 1.0, seed=42)
    tX, ti = torch.from_numpy(dX).float().cuda(), torch.from_numpy(idx).cuda()
    alpha = 1.0 / idx.size
    g1 = ge.embedding_grad(tX, ti, V, alpha)
    g2 = ge.embedding_grad(tX, ti, V, alpha)
    assert torch.equal(g1, g2)
    dE = np.zeros((V, H))
    np.add.at(dE, idx, dX)
    assert_parity(host(g1), oracle.round_fmt(alpha * dE, "f32"), 1e-4, "f32", "dE zipf", cancel=True)
    counts = np.bincount(idx, minlength=V)
    assert counts.max() > 0.15 * idx.size and np.all(host(g1)[counts == 0] == 0.0)
