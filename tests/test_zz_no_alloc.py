"""gemm_bias_act_noalloc through the C ABI: the same results as gemm_bias_act
with a caller workspace, on two calls in a row (the second smaller), with
split-K partials in the library's fixed scratch; an oversized problem is
refused before anything is enqueued."""
import ctypes as C

import numpy as np
import pytest
import torch

import datagen

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ge():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import gemm_epilogue_amd
    return gemm_epilogue_amd


def _args(ge, A, B, layout, M, N, K, bias, out, ws=None):
    from gemm_epilogue_amd._lib import GemmArgs, LAYOUT
    from gemm_epilogue_amd.ops import dtype_code
    a = GemmArgs()
    a.layout, a.ab_type, a.M, a.N, a.K = LAYOUT[layout], dtype_code(A.dtype), M, N, K
    a.A, a.lda = A.data_ptr(), A.stride(0)
    a.B, a.ldb = B.data_ptr(), B.stride(0)
    a.alpha = 1.0
    a.bias = bias.data_ptr()
    a.act = 1  # ReLU
    a.C, a.ldc, a.c_type = out.data_ptr(), out.stride(0), dtype_code(out.dtype)
    a.aux_type = a.res_type = a.pre_type = 0
    if ws is not None:
        a.workspace, a.workspace_bytes = ws.data_ptr(), ws.numel()
    return a


@pytest.mark.parametrize("cases", [[(2048, 2048, 4096, "TN"), (512, 256, 8192, "TN")],
                                   [(784, 2048, 4096, "TN"), (300, 200, 3000, "NN")]])
def test_noalloc_matches_workspace_entry(ge, cases):
    from gemm_epilogue_amd._lib import check, lib
    stream = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    for M, N, K, layout in cases:
        print(f"noalloc {layout} {M}x{N}x{K}", flush=True)
        need = ge.gemm_workspace_bytes(layout, torch.float16, M, N, K)
        assert 0 < need <= 64 << 20
        sa = (M, K) if layout != "TN" else (K, M)
        sb = (K, N) if layout != "NT" else (N, K)
        A = torch.from_numpy(datagen.normal(sa, 1 / np.sqrt(K), seed=M + K, fmt="f16")).half().cuda()
        B = torch.from_numpy(datagen.normal(sb, 1 / np.sqrt(K), seed=N + K, fmt="f16")).half().cuda()
        bias = torch.from_numpy(datagen.normal((N,), 0.1, seed=N)).float().cuda()
        ref = torch.empty(M, N, dtype=torch.float32, device="cuda")
        got = torch.full((M, N), -1.0, dtype=torch.float32, device="cuda")
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        check(lib.gemm_bias_act(C.byref(_args(ge, A, B, layout, M, N, K, bias, ref, ws)), stream), "ref")
        check(lib.gemm_bias_act_noalloc(C.byref(_args(ge, A, B, layout, M, N, K, bias, got)), stream), "noalloc")
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"{layout} {M}x{N}x{K}"


def test_noalloc_refuses_oversized_partials(ge):
    from gemm_epilogue_amd._lib import GE_E_WORKSPACE, lib
    M, N, K = 4096, 4096, 1 << 20       # split-K partials far beyond the 64 MiB scratch
    assert ge.gemm_workspace_bytes("TN", torch.float16, 2048, 2048, 1 << 18, split_k=8) > 64 << 20
    A = torch.empty(1, dtype=torch.float16, device="cuda")
    out = torch.empty(1, dtype=torch.float32, device="cuda")
    bias = torch.empty(1, dtype=torch.float32, device="cuda")
    a = _args(ge, A.view(1, 1), A.view(1, 1), "TN", 2048, 2048, 1 << 18, bias, out.view(1, 1))
    a.split_k = 8
    assert lib.gemm_bias_act_noalloc(C.byref(a), None) == GE_E_WORKSPACE
    assert b"scratch" in lib.ge_last_error()
