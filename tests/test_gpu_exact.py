"""Bit-exact mode on the GPU: every output bit of gemm_bias_act, colsum, the
RMSNorm passes and sgd_momentum equals the binary32 operation sequence of
oracle/exact.py on the same inputs (bitwise, signed zeros included)."""
import numpy as np
import pytest
import torch

import datagen
from oracle import exact, round_fmt

pytestmark = pytest.mark.gpu

TD = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
INT = {torch.float32: torch.int32, torch.float16: torch.int16, torch.bfloat16: torch.int16}


@pytest.fixture(scope="module")
def ge():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import gemm_epilogue_amd
    return gemm_epilogue_amd


def bits(t):
    return t.detach().contiguous().view(INT[t.dtype]).cpu().numpy()


def want_bits(x64, dtype):
    return bits(torch.from_numpy(np.ascontiguousarray(x64)).to(dtype))


def dev(x64, fmt):
    # a fresh tensor, so empty dimensions get row-major strides too
    t = torch.empty(np.shape(x64), dtype=TD[fmt], device="cuda")
    return t.copy_(torch.from_numpy(np.ascontiguousarray(x64)))


def assert_bitwise(got, ref64, what):
    gb, wb = bits(got), want_bits(ref64, got.dtype)
    bad = np.count_nonzero(gb != wb)
    assert bad == 0, f"{what}: {bad} of {gb.size} outputs differ in their bits"


def inputs(shape, fmt, seed, std=1.0):
    return round_fmt(datagen.normal(shape, std, seed=seed), fmt)


EPILOGUES = [
    dict(act="relu", alpha=0.5, bias=True, out="f16", pre="f32"),
    dict(act="lrelu_sq", alpha=1.0, bias=True, out="bf16", pre=None),
    dict(act="relu_mask_bwd", alpha=0.125, bias=False, out="f32", pre=None, aux="f16"),
    dict(act="lrelu_sq_bwd", alpha=1.0, bias=True, out="f32", pre="bf16", aux="f32", res="bf16"),
]


@pytest.mark.parametrize("layout", ["NN", "NT", "TN"])
@pytest.mark.parametrize("fmt", ["f32", "f16", "bf16"])
def test_exact_gemm_every_layout_type_and_epilogue(ge, layout, fmt):
    for (M, N, K) in ((77, 45, 131), (64, 128, 64), (1, 3, 1), (130, 70, 0), (200, 65, 1000)):
        for i, ep in enumerate(EPILOGUES):
            seed = M * 7 + N * 3 + K + i
            sa = (M, K) if layout != "TN" else (K, M)
            sb = (K, N) if layout != "NT" else (N, K)
            A = inputs(sa, fmt, seed, 1.0 / max(1, K) ** 0.5)
            B = inputs(sb, fmt, seed + 1)
            bias = inputs((N,), "f32", seed + 2, 0.1) if ep["bias"] else None
            aux = inputs((M, N), ep["aux"], seed + 3) if "aux" in ep else None
            res = inputs((M, N), ep["res"], seed + 4) if "res" in ep else None
            ref, pre_ref = exact.gemm(A, B, layout, alpha=ep["alpha"], bias=bias, act=ep["act"], slope=0.5,
                                      aux=aux, residual=res, out_fmt=ep["out"], pre_fmt=ep["pre"])
            pre = torch.empty((M, N), dtype=TD[ep["pre"]], device="cuda") if ep["pre"] else None
            with ge.bit_exact():
                C = ge.gemm_bias_act(dev(A, fmt), dev(B, fmt), layout, out_dtype=TD[ep["out"]], alpha=ep["alpha"],
                                     bias=None if bias is None else dev(bias, "f32"), act=ep["act"], slope=0.5,
                                     aux=None if aux is None else dev(aux, ep["aux"]),
                                     residual=None if res is None else dev(res, ep["res"]), pre=pre)
            torch.cuda.synchronize()
            what = f"{layout} {fmt} {M}x{N}x{K} {ep['act']}"
            assert_bitwise(C, ref, what)
            if pre is not None:
                assert_bitwise(pre, pre_ref, what + " pre")


def test_exact_gemm_4096_sampled_and_independent_of_the_split(ge):
    """The 4096^3 FP16 NN GEMM with bias and ReLU: a 48x48 sample of the
    outputs against the oracle (each output depends only on its row and
    column), and every output bit the same for any split_k request."""
    M = N = K = 4096
    A = inputs((M, K), "f16", 11, 1.0 / 64)
    B = inputs((K, N), "f16", 12)
    bias = inputs((N,), "f32", 13, 0.1)
    tA, tB, tb = dev(A, "f16"), dev(B, "f16"), dev(bias, "f32")
    with ge.bit_exact():
        C = ge.gemm_bias_act(tA, tB, "NN", out_dtype=torch.float32, bias=tb, act="relu")
        C4 = ge.gemm_bias_act(tA, tB, "NN", out_dtype=torch.float32, bias=tb, act="relu", split_k=4)
    torch.cuda.synchronize()
    assert np.array_equal(bits(C), bits(C4))
    rng = datagen.rng(14, "misc")
    rows = np.sort(rng.choice(M, 48, replace=False))
    cols = np.sort(rng.choice(N, 48, replace=False))
    ref, _ = exact.gemm(A[rows], B[:, cols], "NN", bias=bias[cols], act="relu")
    assert_bitwise(C[torch.from_numpy(rows).cuda()][:, torch.from_numpy(cols).cuda()], ref, "4096^3 sample")
    # the default mode is back after the block, and within the FP16-input tolerance of it
    assert ge.lib.ge_bit_exact() == 0
    Cn = ge.gemm_bias_act(tA, tB, "NN", out_dtype=torch.float32, bias=tb, act="relu")
    assert float((Cn - C).abs().max()) <= 1e-3 * float(C.abs().max())


@pytest.mark.parametrize("fmt", ["f32", "f16", "bf16"])
def test_exact_colsum(ge, fmt):
    for (M, N) in ((3000, 77), (1, 5), (4096, 300)):
        X = inputs((M, N), fmt, M + N)
        out0 = inputs((N,), "f32", M + N + 1)
        with ge.bit_exact():
            s = ge.colsum(dev(X, fmt), 0.25)
            acc = dev(out0, "f32")
            ge.colsum(dev(X, fmt), 0.25, out=acc, accumulate=True)
        torch.cuda.synchronize()
        assert_bitwise(s, exact.colsum(X, 0.25), f"colsum {fmt} {M}x{N}")
        assert_bitwise(acc, exact.colsum(X, 0.25, out=out0), f"colsum accumulate {fmt} {M}x{N}")


@pytest.mark.parametrize("lowp", [None, "f16", "bf16"])
def test_exact_sgd(ge, lowp):
    n = 100_003
    w = inputs((n,), "f32", 1)
    g = inputs((n,), "f32", 2, 0.01)
    v = inputs((n,), "f32", 3, 0.1)
    tw, tg, tv = dev(w, "f32"), dev(g, "f32"), dev(v, "f32")
    tl = torch.empty(n, dtype=TD[lowp], device="cuda") if lowp else None
    with ge.bit_exact():
        ge.sgd_momentum(tw, tg, tv, 0.05, 0.9, tl)
    torch.cuda.synchronize()
    w1, v1, wl = exact.sgd_momentum(w, g, v, 0.05, 0.9, lowp)
    assert_bitwise(tw, w1, "sgd w")
    assert_bitwise(tv, v1, "sgd v")
    if lowp:
        assert_bitwise(tl, wl, "sgd lowp copy")


@pytest.mark.parametrize("rows,D,xf,yf", [(513, 384, "bf16", "bf16"), (300, 512, "f32", "f32"),
                                          (98304, 512, "bf16", "bf16"), (7, 1, "f16", "f32")])
def test_exact_rmsnorm(ge, rows, D, xf, yf):
    x = inputs((rows, D), xf, rows + D)
    gam = inputs((D,), "f32", rows + D + 1)
    dy = inputs((rows, D), xf, rows + D + 2)
    dres = inputs((rows, D), "f32", rows + D + 3)
    tx = dev(x, xf)
    with ge.bit_exact():
        y, r = ge.rmsnorm_fwd(tx, 1e-6, y_dtype=TD[yf], gamma=dev(gam, "f32"))
        y0, r0 = ge.rmsnorm_fwd(tx, 1e-6, y_dtype=TD[yf])
        dgam = torch.empty(D, dtype=torch.float32, device="cuda")
        dx, _ = ge.rmsnorm_bwd(tx, r, dev(dy, xf), dres=dev(dres, "f32"), gamma=dev(gam, "f32"), dx_dtype=TD[yf],
                               dgamma=dgam)
    torch.cuda.synchronize()
    y_ref, r_ref = exact.rmsnorm_fwd(x, 1e-6, gam, y_fmt=yf)
    y0_ref, _ = exact.rmsnorm_fwd(x, 1e-6, None, y_fmt=yf)
    assert_bitwise(r, r_ref, "rmsnorm r")
    assert_bitwise(y, y_ref, "rmsnorm y")
    assert_bitwise(y0, y0_ref, "rmsnorm y without gamma")
    dx_ref, dg_ref = exact.rmsnorm_bwd(x, r_ref, dy, dres, gam, dx_fmt=yf)
    assert_bitwise(dx, dx_ref, "rmsnorm dx")
    assert_bitwise(dgam, dg_ref, "rmsnorm dgamma")
