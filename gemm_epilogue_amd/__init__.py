"""MI355X (gfx950) GEMM-epilogue training path: Python binding.

The compute lives in ``libgemm_epilogue.so`` (hand-written HIP, built with
``python -m gemm_epilogue_amd.build``); this package only marshals torch
tensors (device memory and the current stream) into its C ABI.
"""
from ._lib import GEError, lib  # noqa: F401  (fails loudly when the library is missing)
from .ops import (MLPTrainer, colsum, dtype_code, gemm_bias_act, gemm_workspace_bytes,  # noqa: F401
                  mlp_block_fwd_bwd, mlp_param_count, rmsnorm_bwd, rmsnorm_fwd, sgd_momentum,
                  softmax_xent_fwd_bwd, GRUTrainer, embedding_gather, embedding_grad, gru_param_count,
                  params_to_lowp, gru_gates_fwd, gru_gates_bwd, bit_exact,
                  mlp_block_fwd_fused)
