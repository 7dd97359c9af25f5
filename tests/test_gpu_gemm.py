"""GPU parity of gemm_bias_act (all layouts, input types, epilogues) and colsum
against the oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import datagen
import oracle
from parity import TOL_F32, TOL_LOWP, assert_parity, compare

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


def shapes_of(M, N, K, layout):
    sa = (M, K) if layout in ("NN", "NT") else (K, M)
    sb = (K, N) if layout in ("NN", "TN") else (N, K)
    return sa, sb


def _tol(fmt):
    return TOL_F32 if fmt == "f32" else TOL_LOWP


# includes narrow outputs (N <= 16: 128x16 tiles with short K splits), a
# long-K shape that takes 256x256 tiles with split-K, aligned ragged shapes
# whose edge tiles take clamped vector loads, and one that takes 256x128 tiles
RAGGED = [(1, 1, 1), (15, 17, 63), (65, 130, 100), (200, 72, 784), (130, 257, 129),
          (1800, 1800, 130), (96, 80, 3000), (300, 10, 1000), (33, 1, 70), (4096, 16, 2048),
          (1000, 700, 8200), (776, 264, 1000), (3000, 2000, 1600)]


@pytest.mark.parametrize("fmt", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("layout", ["NN", "NT", "TN"])
@pytest.mark.parametrize("shape", RAGGED, ids=lambda s: "x".join(map(str, s)))
def test_gemm_bias_relu_ragged(ge, fmt, layout, shape):
    M, N, K = shape
    print(f"gemm {layout} {fmt} {M}x{N}x{K}", flush=True)
    sa, sb = shapes_of(M, N, K, layout)
    A = datagen.normal(sa, 1 / np.sqrt(K), seed=M + 3 * N + 7 * K, stream="gemm_a", fmt=fmt)
    B = datagen.normal(sb, 1 / np.sqrt(K), seed=M + 3 * N + 7 * K, stream="gemm_b", fmt=fmt)
    bias = datagen.normal((N,), 0.1, seed=K, stream="gemm_bias")
    ref, pre_ref = oracle.gemm_epilogue(A, B, layout, 1.0, bias, "relu", out_fmt="f32", pre_fmt="f32")
    tA, tB, tb = dev(A, fmt), dev(B, fmt), dev(bias, "f32")
    pre = torch.empty((M, N), dtype=torch.float32, device="cuda")
    out = ge.gemm_bias_act(tA, tB, layout, bias=tb, act="relu", out_dtype=torch.float32, pre=pre)
    assert_parity(host(out), ref, _tol(fmt), "f32", f"C {layout} {fmt} {shape}", cancel=True)
    assert_parity(host(pre), pre_ref, _tol(fmt), "f32", f"pre {layout} {fmt} {shape}", cancel=True)
    if fmt != "f32":
        ref16, _ = oracle.gemm_epilogue(A, B, layout, 1.0, bias, "relu", out_fmt=fmt)
        out16 = ge.gemm_bias_act(tA, tB, layout, bias=tb, act="relu", out_dtype=TD[fmt])
        assert_parity(host(out16), ref16, TOL_LOWP, fmt, f"C16 {layout} {fmt} {shape}", cancel=True)


@pytest.mark.parametrize("fmt", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("layout", ["NN", "NT", "TN"])
def test_gemm_integer_inputs_bitwise(ge, fmt, layout):
    M, N, K = 257, 190, 784
    sa, sb = shapes_of(M, N, K, layout)
    A = datagen.integer_matrix(sa, 31)
    B = datagen.integer_matrix(sb, 32)
    bias = datagen.integer_matrix((N,), 33)
    for ofmt in ({"f32", fmt}):
        ref, _ = oracle.gemm_epilogue(A, B, layout, 1.0, bias, "none", out_fmt=ofmt)
        out = ge.gemm_bias_act(dev(A, fmt), dev(B, fmt), layout, bias=dev(bias, "f32"),
                               out_dtype=TD[ofmt])
        np.testing.assert_array_equal(host(out), ref)


@pytest.mark.parametrize("act", ["lrelu_sq", "relu_mask_bwd", "lrelu_sq_bwd", "none"])
@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_gemm_epilogue_variants(ge, act, fmt):
    M, N, K = 300, 200, 256
    layout = "NT" if act.endswith("bwd") else "NN"
    sa, sb = shapes_of(M, N, K, layout)
    A = datagen.normal(sa, 1.0, seed=41, fmt=fmt)
    B = datagen.normal(sb, 0.05, seed=42, fmt=fmt)
    aux = datagen.normal((M, N), 1.0, seed=43, fmt=fmt)
    res = datagen.normal((M, N), 1.0, seed=44, fmt=fmt)
    bias = None if act.endswith("bwd") else datagen.normal((N,), 0.1, seed=45)
    alpha = 0.75
    ref, pre_ref = oracle.gemm_epilogue(A, B, layout, alpha, bias, act, 0.5, aux, res, out_fmt=fmt,
                                        pre_fmt=fmt)
    pre = torch.empty((M, N), dtype=TD[fmt], device="cuda")
    out = ge.gemm_bias_act(dev(A, fmt), dev(B, fmt), layout, alpha=alpha,
                           bias=None if bias is None else dev(bias, "f32"), act=act, slope=0.5,
                           aux=dev(aux, fmt), residual=dev(res, fmt), pre=pre, out_dtype=TD[fmt])
    assert_parity(host(out), ref, TOL_LOWP, fmt, f"{act} C", cancel=True)
    assert_parity(host(pre), pre_ref, TOL_LOWP, fmt, f"{act} pre", cancel=True)


@pytest.mark.parametrize("act", ["relu_mask_bwd", "lrelu_sq_bwd"])
@pytest.mark.parametrize("fmt,aux_fmt,out_fmt", [("f32", "f32", "f32"), ("f16", "f16", "f16"),
                                                 ("f16", "f32", "f32"), ("bf16", "bf16", "f32"),
                                                 ("f16", "f16", "f32")])
@pytest.mark.parametrize("shape", [(128, 256, 10), (512, 384, 200), (300, 200, 64)],
                         ids=lambda s: "x".join(map(str, s)))
def test_gemm_derivative_epilogue_aux_only(ge, act, fmt, aux_fmt, out_fmt, shape):
    """Backward epilogues with aux and no residual, on interior (aligned) and edge tiles."""
    M, N, K = shape
    sa, sb = shapes_of(M, N, K, "NT")
    A = datagen.normal(sa, 1.0, seed=M + K, fmt=fmt)
    B = datagen.normal(sb, 0.05, seed=N + K, fmt=fmt)
    aux = datagen.normal((M, N), 1.0, seed=M + N, fmt=aux_fmt)
    ref, _ = oracle.gemm_epilogue(A, B, "NT", 1.0, None, act, 0.5, aux, None, out_fmt=out_fmt)
    out = ge.gemm_bias_act(dev(A, fmt), dev(B, fmt), "NT", act=act, slope=0.5, aux=dev(aux, aux_fmt),
                           out_dtype=TD[out_fmt])
    assert_parity(host(out), ref, _tol(fmt), out_fmt, f"{act} {fmt}/{aux_fmt}/{out_fmt} {shape}", cancel=True)


def test_gemm_strided_and_unaligned_operands(ge):
    # leading dimensions larger than the rows, and odd ones that rule out vector loads
    M, N, K = 70, 90, 110
    for lda, ldb, ldc in ((128, 96, 96), (111, 91, 93)):
        A = datagen.normal((M, lda), 0.1, seed=51, fmt="f16")
        B = datagen.normal((K, ldb), 0.1, seed=52, fmt="f16")
        tA = dev(A, "f16")[:, :K]
        tB = dev(B, "f16")[:, :N]
        Cbuf = torch.full((M, ldc), -7.0, dtype=torch.float32, device="cuda")
        out = ge.gemm_bias_act(tA, tB, "NN", out=Cbuf[:, :N])
        ref, _ = oracle.gemm_epilogue(A[:, :K], B[:, :N], "NN", out_fmt="f32")
        assert_parity(host(out), ref, TOL_LOWP, "f32", f"ld {lda},{ldb},{ldc}", cancel=True)
        assert torch.all(Cbuf[:, N:] == -7.0), "wrote outside the output columns"


def test_gemm_k_zero_and_empty(ge):
    bias = datagen.normal((33,), 0.5, seed=61)
    A = torch.empty((20, 0), dtype=torch.float16, device="cuda")
    B = torch.empty((0, 33), dtype=torch.float16, device="cuda")
    out = ge.gemm_bias_act(A, B, "NN", bias=dev(bias, "f32"), act="relu")
    np.testing.assert_array_equal(host(out), np.tile(np.maximum(bias, 0), (20, 1)))
    e = ge.gemm_bias_act(torch.empty((0, 8), dtype=torch.float16, device="cuda"),
                         torch.empty((8, 5), dtype=torch.float16, device="cuda"), "NN")
    assert e.shape == (0, 5)


def test_gemm_split_k_deterministic(ge):
    M, N, K = 160, 96, 8192
    A = datagen.normal((K, M), 0.02, seed=71, fmt="bf16")
    B = datagen.normal((K, N), 1.0, seed=72, fmt="bf16")
    tA, tB = dev(A, "bf16"), dev(B, "bf16")
    ref, _ = oracle.gemm_epilogue(A, B, "TN", out_fmt="f32")
    outs = []
    for s in (0, 1, 3, 16):
        out = ge.gemm_bias_act(tA, tB, "TN", split_k=s)
        assert_parity(host(out), ref, TOL_LOWP, "f32", f"split {s}", cancel=True)
        outs.append(out)
    again = ge.gemm_bias_act(tA, tB, "TN", split_k=16)
    assert torch.equal(again, outs[3])


# ------------------------- the standalone GEMM workload: 128x256x784, 4096^3 --

@pytest.mark.parametrize("layout", ["NN", "NT", "TN"])
def test_cfg1_small_shape_full(ge, layout):
    M, N, K = 128, 256, 784
    A, B, bias = datagen.gemm_operands(M, N, K, layout, seed=1)
    tA, tB, tb = dev(A, "f16"), dev(B, "f16"), dev(bias, "f32")
    for ofmt in ("f16", "f32"):
        ref, _ = oracle.gemm_epilogue(A, B, layout, 1.0, bias, "relu", out_fmt=ofmt)
        out = ge.gemm_bias_act(tA, tB, layout, bias=tb, act="relu", out_dtype=TD[ofmt])
        assert_parity(host(out), ref, TOL_LOWP, ofmt, f"{layout} {ofmt}", cancel=True)
        cs = ge.colsum(out)
        assert_parity(host(cs), oracle.colsum(host(out)), TOL_F32, "f32", "colsum", cancel=True)


@pytest.mark.parametrize("layout", ["NN", "NT", "TN"])
def test_cfg1_4096_sampled(ge, layout):
    M = N = K = 4096
    A, B, bias = datagen.gemm_operands(M, N, K, layout, seed=2)
    tA, tB, tb = dev(A, "f16"), dev(B, "f16"), dev(bias, "f32")
    g = np.random.default_rng(3)
    rows = np.sort(g.choice(M, 96, replace=False))
    cols = np.sort(g.choice(N, 96, replace=False))
    rows[-1], cols[-1] = M - 1, N - 1
    opA = A if layout != "TN" else A.T
    opB = B if layout != "NT" else B.T
    for ofmt in ("f16", "f32"):
        out = ge.gemm_bias_act(tA, tB, layout, bias=tb, act="relu", out_dtype=TD[ofmt])
        ref, _ = oracle.gemm_epilogue(opA[rows], opB[:, cols], "NN", 1.0, bias[cols], "relu", out_fmt=ofmt)
        got = host(out)[np.ix_(rows, cols)]
        assert_parity(got, ref, TOL_LOWP, ofmt, f"4096 {layout} {ofmt}", cancel=True)
        # colsum over M of the full output: check sampled columns against the
        # oracle's sum of the GPU's stored column
        cs = host(ge.colsum(out))
        full = host(out)
        assert_parity(cs[cols], oracle.colsum(full[:, cols]), TOL_F32, "f32", "colsum 4096", cancel=True)


# ----------- shapes that take the eight-wave 256x256 kernel (32x32x16 MFMA) --
# whole 256x256 tiles and K a multiple of 64: unsplit when the tiles fill the
# GPU, split-K (then the finishing pass applies the epilogue) when they do not
# 256x256 tiles for the first three; 256x128 tiles (eight waves, 64x64 each)
# for the last two, the shapes of the 784-2048-2048-10 step's middle layer
# whole tiles; then the step's K = 784 and M = 784 shapes (a partial last
# k-tile, an edge row of tiles) and edge tiles along both M and N with a
# k-tail of 8 (4120 x 3000 x 200) or of 8 in a single k-tile (1032 x 12296 x 72)
X8 = [(4096, 3072, 256), (3072, 4096, 512), (512, 512, 16384), (4096, 2048, 2048), (4096, 1536, 1536),
      (4096, 2048, 784), (784, 2048, 4096), (4120, 3000, 200), (1032, 12296, 72)]


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("layout", ["NN", "NT", "TN"])
@pytest.mark.parametrize("shape", X8, ids=lambda s: "x".join(map(str, s)))
def test_gemm_x8_tiles_full(ge, fmt, layout, shape):
    M, N, K = shape
    print(f"gemm x8 {layout} {fmt} {M}x{N}x{K}", flush=True)
    sa, sb = shapes_of(M, N, K, layout)
    A = datagen.normal(sa, 1 / np.sqrt(K), seed=M + N + K, stream="gemm_a", fmt=fmt)
    B = datagen.normal(sb, 1 / np.sqrt(K), seed=M + N + K, stream="gemm_b", fmt=fmt)
    bias = datagen.normal((N,), 0.1, seed=K + 1, stream="gemm_bias")
    tA, tB, tb = dev(A, fmt), dev(B, fmt), dev(bias, "f32")
    ref, pre_ref = oracle.gemm_epilogue(A, B, layout, 1.0, bias, "relu", out_fmt=fmt, pre_fmt="f32")
    pre = torch.empty((M, N), dtype=torch.float32, device="cuda")
    out = ge.gemm_bias_act(tA, tB, layout, bias=tb, act="relu", out_dtype=TD[fmt], pre=pre)
    assert_parity(host(out), ref, TOL_LOWP, fmt, f"x8 C {layout} {fmt} {shape}", cancel=True)
    assert_parity(host(pre), pre_ref, TOL_LOWP, "f32", f"x8 pre {layout} {fmt} {shape}", cancel=True)


@pytest.mark.parametrize("act", ["lrelu_sq", "relu_mask_bwd", "lrelu_sq_bwd"])
def test_gemm_x8_epilogue_variants(ge, act):
    """The fused epilogues on the eight-wave kernel: LeakyReLU^2 with the
    pre-activation store and a residual, the derivative epilogues on aux."""
    M, N, K, fmt = 2048, 6144, 512, "bf16"
    layout = "NT" if act.endswith("bwd") else "NN"
    sa, sb = shapes_of(M, N, K, layout)
    A = datagen.normal(sa, 1.0, seed=81, fmt=fmt)
    B = datagen.normal(sb, 0.05, seed=82, fmt=fmt)
    aux = datagen.normal((M, N), 1.0, seed=83, fmt=fmt) if act.endswith("bwd") else None
    res = None if act.endswith("bwd") else datagen.normal((M, N), 1.0, seed=84, fmt=fmt)
    ref, pre_ref = oracle.gemm_epilogue(A, B, layout, 0.5, None, act, 0.5, aux, res, out_fmt=fmt, pre_fmt=fmt)
    pre = torch.empty((M, N), dtype=TD[fmt], device="cuda")
    out = ge.gemm_bias_act(dev(A, fmt), dev(B, fmt), layout, alpha=0.5, act=act, slope=0.5,
                           aux=None if aux is None else dev(aux, fmt),
                           residual=None if res is None else dev(res, fmt), pre=pre, out_dtype=TD[fmt])
    assert_parity(host(out), ref, TOL_LOWP, fmt, f"x8 {act} C", cancel=True)
    assert_parity(host(pre), pre_ref, TOL_LOWP, fmt, f"x8 {act} pre", cancel=True)


# ------------------------------------------- launches captured in a graph --

@pytest.mark.parametrize("shape,layout", [((128, 256, 784), "NN"), ((128, 256, 784), "TN"),
                                          ((4096, 16, 2048), "NN"), ((512, 512, 512), "NT")],
                         ids=lambda v: "x".join(map(str, v)) if isinstance(v, tuple) else v)
def test_gemm_graph_replays_match_eager(ge, shape, layout):
    """gemm_bias_act captured in a graph (split-K with its finishing pass for
    the short-k and narrow shapes, one launch for the last): every replay,
    with eager work between them, gives the eager result bit for bit."""
    M, N, K = shape
    print(f"graph gemm {layout} {M}x{N}x{K}", flush=True)
    A, B, bias = datagen.gemm_operands(M, N, K, layout, seed=9)
    tA, tB, tb = dev(A, "f16"), dev(B, "f16"), dev(bias, "f32")
    ws = torch.empty(max(1, ge.gemm_workspace_bytes(layout, torch.float16, M, N, K)), dtype=torch.uint8,
                     device="cuda")
    C = torch.empty(M, N, dtype=torch.float16, device="cuda")
    ge.gemm_bias_act(tA, tB, layout, bias=tb, act="relu", out=C, workspace=ws)
    torch.cuda.synchronize()
    ref = C.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        ge.gemm_bias_act(tA, tB, layout, bias=tb, act="relu", out=C, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ge.gemm_bias_act(tA, tB, layout, bias=tb, act="relu", out=C, workspace=ws)
    for i in range(3):
        C.zero_()
        ws.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(C, ref), f"replay {i}"
        # eager work between the replays, on the same buffers
        ge.gemm_bias_act(tA, tB, layout, bias=tb, act="none", out=C, workspace=ws)
        torch.cuda.synchronize()
    assert_parity(host(ref), oracle.gemm_epilogue(A, B, layout, 1.0, bias, "relu", out_fmt="f16")[0], TOL_LOWP,
                  "f16", f"graph {layout} {M}x{N}x{K}", cancel=True)
