"""C-ABI contract tests that need no GPU: the library loads, exports every
declared symbol, and rejects bad arguments on the host before enqueuing."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if not fn.endswith(".h"):
            continue
        text = open(os.path.join(ROOT, "include", fn)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, re.M):
            if m.group(1) not in ("defined", "if"):
                names.add(m.group(1))
    return names


@pytest.fixture(scope="module")
def ge():
    import gemm_epilogue_amd as g
    return g


def test_library_exports_every_declared_symbol(ge):
    names = _declared_functions()
    assert {"gemm_bias_act", "colsum", "softmax_xent_fwd_bwd", "rmsnorm_fwd_bwd", "sgd_momentum",
            "mlp_train_step"} <= names
    missing = [n for n in sorted(names) if not hasattr(ge.lib, n)]
    assert not missing, f"not exported: {missing}"


def test_binding_declares_every_symbol(ge):
    from gemm_epilogue_amd._lib import SIGNATURES
    assert _declared_functions() <= set(SIGNATURES)


def test_version_and_param_count(ge, pins):
    assert ge.lib.ge_abi_version() == 1
    assert ge.mlp_param_count([784, 256, 10]) == pins["param_count_784_256_10"]
    assert ge.mlp_param_count([784, 2048, 2048, 10]) == 5_824_522


def test_gemm_rejects_bad_arguments_without_launch(ge):
    from gemm_epilogue_amd._lib import GE_E_INVALID, GemmArgs
    a = GemmArgs()
    a.layout, a.ab_type, a.M, a.N, a.K = 7, 1, 4, 4, 4
    assert ge.lib.gemm_bias_act(C.byref(a), None) == GE_E_INVALID
    assert b"layout" in ge.lib.ge_last_error()
    a.layout = 0
    a.A = a.B = a.C = 16
    a.lda, a.ldb, a.ldc = 3, 4, 4            # lda < K
    assert ge.lib.gemm_bias_act(C.byref(a), None) == GE_E_INVALID
    a.lda = 4
    a.act = 3                                 # mask backward without aux
    assert ge.lib.gemm_bias_act(C.byref(a), None) == GE_E_INVALID
    assert ge.lib.gemm_bias_act(None, None) == GE_E_INVALID
    a.act, a.M = 0, -1
    assert ge.lib.gemm_bias_act(C.byref(a), None) == GE_E_INVALID


def test_other_entry_points_reject_bad_arguments(ge):
    from gemm_epilogue_amd._lib import GE_E_INVALID, RmsnormArgs
    lib = ge.lib
    assert lib.colsum(None, 4, 4, 4, 9, 1.0, 8, 0, None, 0, None) == GE_E_INVALID
    assert lib.colsum(None, 4, 4, 4, 0, 1.0, 8, 1, None, 0, None) == GE_E_INVALID   # X NULL
    assert lib.softmax_xent_fwd_bwd(8, 4, 0, 4, 8, 1.0, 8, 8, None, 0, 0, None, None, None) == GE_E_INVALID
    assert lib.softmax_xent_fwd_bwd(8, 4, 10, 9, 8, 1.0, 8, 8, None, 0, 0, None, 8, None) == GE_E_INVALID
    assert lib.params_to_lowp(16, 16, 10, 0, None) == GE_E_INVALID         # FP32 is not a low-precision copy
    assert lib.params_to_lowp(None, 16, 10, 1, None) == GE_E_INVALID
    assert lib.gru_gates_fwd(16, 16, None, 4, 6, 16, 16, 16, 16, None, None) == GE_E_INVALID   # H % 4
    assert lib.gru_gates_fwd(16, 16, None, 4, 8, 16, 16, 16, 20, None, None) == GE_E_INVALID   # misaligned h
    assert lib.gru_gates_bwd(16, None, 16, 16, 16, 16, None, 4, 8, 16, 16, None, None) == GE_E_INVALID
    assert lib.embedding_grad(16, 8, 0, 16, 10, 20000, 8, 1.0, 16, 8, 16, 1 << 20, None) == GE_E_INVALID
    assert ge.lib.embedding_grad_workspace_bytes(8192, 256) == (8192 + 257) * 4
    r = RmsnormArgs()
    r.pass_, r.rows, r.D = 5, 4, 8
    assert lib.rmsnorm_fwd_bwd(C.byref(r), None) == GE_E_INVALID
    r.pass_, r.D = 0, 5000
    assert lib.rmsnorm_fwd_bwd(C.byref(r), None) == GE_E_INVALID
    assert lib.sgd_momentum(None, None, None, 0.1, 0.9, 10, None, 0, None) == GE_E_INVALID
    assert lib.sgd_momentum(8, 8, 8, 0.1, 0.9, 10, 8, 0, None) == GE_E_INVALID   # lowp must be 16-bit


def test_mlp_workspace_layout(ge):
    from gemm_epilogue_amd._lib import MlpDesc
    dims = (C.c_int64 * 3)(784, 256, 10)
    d = MlpDesc(2, dims, 0)
    n = ge.lib.mlp_workspace_bytes(C.byref(d), 128)
    assert n >= 128 * 256 * 4 + 2 * 128 * 10 * 4 + 128 * 4
    offs = (C.c_int64 * 6)()
    assert ge.lib.mlp_workspace_offsets(C.byref(d), 128, offs, 6) == 0
    assert len(set(offs)) == 6 and all(o % 256 == 0 for o in offs)
    bad = MlpDesc(2, dims, 2)                 # BF16 storage is not a plan of the MLP step
    assert ge.lib.mlp_workspace_bytes(C.byref(bad), 128) == -1
    assert ge.lib.mlp_workspace_bytes(C.byref(MlpDesc(2, dims, 0, 3)), 128) == -1   # no such step plan
    assert ge.lib.mlp_workspace_bytes(C.byref(MlpDesc(2, dims, 0, 2)), 128) == n


def test_workspace_queries(ge):
    from gemm_epilogue_amd.ops import gemm_workspace_bytes
    import torch
    assert gemm_workspace_bytes("NN", torch.float16, 4096, 4096, 4096) == 0
    ws = gemm_workspace_bytes("TN", torch.bfloat16, 1536, 512, 98304)
    assert ws > 0 and ws % (1536 * 512 * 4) == 0
    assert gemm_workspace_bytes("TN", torch.bfloat16, 1536, 512, 98304, split_k=4) == 4 * 1536 * 512 * 4
    assert ge.lib.colsum_workspace_bytes(128, 10) == 0
    assert ge.lib.colsum_workspace_bytes(4096, 4096) > 0


def test_bit_exact_switch(ge):
    assert ge.lib.ge_bit_exact() == 0
    assert ge.lib.ge_set_bit_exact(1) == 0 and ge.lib.ge_bit_exact() == 1
    assert ge.lib.ge_set_bit_exact(7) == 1 and ge.lib.ge_bit_exact() == 1   # any nonzero is on
    assert ge.lib.ge_set_bit_exact(0) == 1 and ge.lib.ge_bit_exact() == 0
    with ge.bit_exact():
        assert ge.lib.ge_bit_exact() == 1
        with ge.bit_exact(False):
            assert ge.lib.ge_bit_exact() == 0
        assert ge.lib.ge_bit_exact() == 1
    assert ge.lib.ge_bit_exact() == 0
