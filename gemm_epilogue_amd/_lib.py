"""ctypes view of libgemm_epilogue.so (declarations mirror include/gemm_epilogue.h).

The library is loaded after torch so that both share the one HIP runtime
already mapped into the process (torch's), which is what makes torch's
device pointers and streams valid inside the library.  Loading fails loudly
when the library has not been built: there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os

import torch  # noqa: F401  (must be loaded first: it maps the HIP runtime)

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libgemm_epilogue.so")

GE_OK, GE_E_INVALID, GE_E_UNSUPPORTED, GE_E_LAUNCH, GE_E_WORKSPACE = 0, -1, -2, -3, -4
GE_F32, GE_F16, GE_BF16 = 0, 1, 2
GE_NN, GE_NT, GE_TN = 0, 1, 2
ACT = {"none": 0, "relu": 1, "lrelu_sq": 2, "relu_mask_bwd": 3, "lrelu_sq_bwd": 4}
LAYOUT = {"NN": GE_NN, "NT": GE_NT, "TN": GE_TN}
GE_FWD, GE_BWD = 0, 1

i32, i64, f32, vp = C.c_int32, C.c_int64, C.c_float, C.c_void_p


class GemmArgs(C.Structure):
    _fields_ = [("layout", i32), ("ab_type", i32), ("M", i64), ("N", i64), ("K", i64),
                ("A", vp), ("lda", i64), ("B", vp), ("ldb", i64), ("alpha", f32),
                ("bias", vp), ("act", i32), ("act_slope", f32),
                ("aux", vp), ("ld_aux", i64), ("aux_type", i32),
                ("residual", vp), ("ld_res", i64), ("res_type", i32),
                ("C", vp), ("ldc", i64), ("c_type", i32),
                ("pre", vp), ("ld_pre", i64), ("pre_type", i32),
                ("workspace", vp), ("workspace_bytes", i64), ("split_k", i32)]


class RmsnormArgs(C.Structure):
    _fields_ = [("pass_", i32), ("rows", i64), ("D", i64), ("eps", f32),
                ("x", vp), ("ld_x", i64), ("x_type", i32), ("gamma", vp),
                ("y", vp), ("ld_y", i64), ("y_type", i32), ("r", vp),
                ("dy", vp), ("ld_dy", i64), ("dy_type", i32),
                ("dres", vp), ("ld_dres", i64), ("dres_type", i32),
                ("dx", vp), ("ld_dx", i64), ("dx_type", i32), ("dgamma", vp),
                ("workspace", vp), ("workspace_bytes", i64)]


class MlpDesc(C.Structure):
    _fields_ = [("n_layers", i32), ("dims", C.POINTER(i64)), ("storage", i32), ("plan", i32)]


class MlpBuffers(C.Structure):
    _fields_ = [("params", vp), ("grads", vp), ("velocity", vp), ("params_lowp", vp),
                ("workspace", vp), ("workspace_bytes", i64)]


class BlockArgs(C.Structure):
    _fields_ = [("rows", i64), ("D", i64), ("F", i64), ("eps", f32), ("slope", f32), ("type", i32),
                ("x", vp), ("w_up", vp), ("w_down", vp), ("dy", vp), ("y", vp), ("r", vp),
                ("n", vp), ("u", vp), ("a", vp), ("du", vp), ("dn", vp), ("dx", vp),
                ("dw_up", vp), ("dw_down", vp), ("workspace", vp), ("workspace_bytes", i64)]


class BlockFusedArgs(C.Structure):
    _fields_ = [("rows", i64), ("D", i64), ("F", i64), ("eps", f32), ("slope", f32), ("type", i32),
                ("x", vp), ("w_up", vp), ("w_down", vp), ("y", vp), ("r", vp), ("n", vp), ("u", vp),
                ("a", vp), ("workspace", vp), ("workspace_bytes", i64)]


class GruDesc(C.Structure):
    _fields_ = [("V", i64), ("H", i64), ("B", i64), ("T", i64), ("eps", f32), ("recurrence", i32)]


class GruBuffers(C.Structure):
    _fields_ = [("params", vp), ("grads", vp), ("velocity", vp), ("params_lowp", vp),
                ("workspace", vp), ("workspace_bytes", i64)]


# name -> (restype, argtypes); every function declared in include/*.h
SIGNATURES = {
    "ge_abi_version": (i32, []),
    "ge_last_error": (C.c_char_p, []),
    "ge_launch_count": (i64, []),
    "ge_set_bit_exact": (i32, [i32]),
    "ge_bit_exact": (i32, []),
    "mlp_block_fused_workspace_bytes": (i64, [i64, i64]),
    "mlp_block_fwd_fused": (i32, [C.POINTER(BlockFusedArgs), vp]),
    "ge_clock_probe": (i32, [vp, i32, i32, vp]),
    "gemm_bias_act": (i32, [C.POINTER(GemmArgs), vp]),
    "gemm_bias_act_noalloc": (i32, [C.POINTER(GemmArgs), vp]),
    "gemm_workspace_bytes": (i64, [i32, i32, i64, i64, i64, i32]),
    "colsum": (i32, [vp, i64, i64, i64, i32, f32, vp, i32, vp, i64, vp]),
    "colsum_workspace_bytes": (i64, [i64, i64]),
    "softmax_xent_fwd_bwd": (i32, [vp, i64, i64, i64, vp, f32, vp, vp, vp, i64, i32, vp, vp, vp]),
    "rmsnorm_fwd_bwd": (i32, [C.POINTER(RmsnormArgs), vp]),
    "rmsnorm_workspace_bytes": (i64, [i64, i64]),
    "sgd_momentum": (i32, [vp, vp, vp, f32, f32, i64, vp, i32, vp]),
    "params_to_lowp": (i32, [vp, vp, i64, i32, vp]),
    "mlp_param_count": (i64, [i32, C.POINTER(i64)]),
    "mlp_workspace_bytes": (i64, [C.POINTER(MlpDesc), i64]),
    "mlp_workspace_offsets": (i32, [C.POINTER(MlpDesc), i64, C.POINTER(i64), i32]),
    "mlp_train_step": (i32, [C.POINTER(MlpDesc), C.POINTER(MlpBuffers), vp, vp, i64, f32, f32, vp, vp]),
    "mlp_block_workspace_bytes": (i64, [i64, i64, i64, i32]),
    "mlp_block_fwd_bwd": (i32, [C.POINTER(BlockArgs), vp]),
    "embedding_gather": (i32, [vp, i64, i64, i64, i32, vp, i64, vp, i64, i32, vp]),
    "embedding_grad": (i32, [vp, i64, i32, vp, i64, i64, i64, f32, vp, i64, vp, i64, vp]),
    "embedding_grad_workspace_bytes": (i64, [i64, i64]),
    "gru_gates_fwd": (i32, [vp, vp, vp, i64, i64, vp, vp, vp, vp, vp, vp]),
    "gru_gates_bwd": (i32, [vp, vp, vp, vp, vp, vp, vp, i64, i64, vp, vp, vp, vp]),
    "gru_param_count": (i64, [i64, i64]),
    "gru_workspace_bytes": (i64, [C.POINTER(GruDesc)]),
    "gru_workspace_offsets": (i32, [C.POINTER(GruDesc), C.POINTER(i64), i32]),
    "gru_lm_train_step": (i32, [C.POINTER(GruDesc), C.POINTER(GruBuffers), vp, f32, f32, vp, vp]),
}

GRU_WS = ("INP", "TGT", "X16", "GI", "GH", "H16", "HS", "R", "Z", "N", "HN", "RSTD", "LOGITS", "G",
          "ROW_LOSS", "DHN", "DH_OUT", "DGH", "DGI", "DX", "ZERO_H", "CARRY", "DH_DIR")


def _mapped_hip_runtimes():
    try:
        with open("/proc/self/maps") as f:
            return sorted({ln.split()[-1] for ln in f if "libamdhip64" in ln and "/" in ln})
    except OSError:
        return []


def _load():
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built: run `python -m gemm_epilogue_amd.build` "
                           "(there is no fallback path)")
    lib = C.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name, None)
        if fn is None:
            continue
        fn.restype = res
        fn.argtypes = args
    runtimes = _mapped_hip_runtimes()
    if len(runtimes) > 1:
        raise RuntimeError(f"two HIP runtimes are mapped ({runtimes}); import torch before "
                           "gemm_epilogue_amd")
    return lib


lib = _load()


class GEError(RuntimeError):
    pass


def check(status: int, what: str = ""):
    if status != GE_OK:
        msg = lib.ge_last_error().decode(errors="replace")
        raise GEError(f"{what or 'call'} failed with status {status}: {msg}")
