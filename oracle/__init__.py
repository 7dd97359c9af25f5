"""CPU oracle for the GEMM-epilogue training path -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the package's ``__graft_entry__.smoke()`` check and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(the HIP library and its Python binding) never imports, calls or links it, and
it never imports the product path.

Everything here is plain, slow, obviously-correct float64 numpy: every sum is
an fp64 matrix product or an fp64 ``np.sum``; wherever the GPU path *stores* a
tensor in FP32/FP16/BF16, the oracle rounds its float64 value to that format
(round-to-nearest-even) at the same point, so both sides see the same storage
precision.  Inputs arrive as float64 arrays whose values are already exactly
representable in their storage format (see ``datagen``).

Sources, cited by page title and section:

* "Capstone 5: train a network with your CUDA kernels" (Day 100) -- the
  784-256-10 model ("The minimum model"), the backward equations ("Work through
  the backward pass", "Check your mapping"), the bias/ReLU epilogue and the
  flat-buffer momentum update ("Read the worked reference"), the stable softmax
  ("Read the worked reference", last paragraph) and the test gates ("Practice
  with less help each time", "The independent submission gate").
* "The Work Moved Down a Layer" (Cat Chat) -- FP32 epilogue then one final
  conversion, FP32 reductions, FP32 RMSNorm statistics and recurrent state
  ("The Debugging Lesson Was Numerical"); GEMM, GRU gates, RMSNorm, softmax
  cross-entropy, gradient reduction, optimizer ("The Work Moved Down a Layer").
* "Full-Depth MLP Megakernel + Fused Attention Preprocessing" -- the MLP block
  RMSNorm -> projection -> LeakyReLU^2 -> down projection -> residual ("What
  Worked") and its backward epilogue ("Credits").

``oracle.exact`` holds the bit-exact FP32 definitions of the primitives
(linear-order sums, one rounding per operation, correctly rounded divide and
square root) that the library's bit-exact mode reproduces bit for bit; it
follows "HIP + Vulkan backends -- Phase 3" ("Phase-3 bug hunt").

Every function here is pinned by ``tests/test_oracle_*.py`` against closed
forms, invariants, brute force on tiny inputs, finite differences or an
independent library routine; none is "parity unpinned".
"""
from .numerics import round_fmt, FORMATS
from .ops import (act_forward, act_backward_factor, gemm_epilogue, colsum,
                  softmax_xent, rmsnorm_fwd, rmsnorm_bwd, sgd_momentum)
from .mlp import (mlp_param_count, mlp_unflatten, mlp_step, mlp_forward,
                  mlp_loss_only)
from .block import block_fwd_bwd
from .gru import (gru_param_count, gru_flatten, gru_unflatten, gru_step, gru_loss_only,
                  gru_gates_fwd, gru_gates_bwd)

__all__ = [
    "round_fmt", "FORMATS", "act_forward", "act_backward_factor",
    "gemm_epilogue", "colsum", "softmax_xent", "rmsnorm_fwd", "rmsnorm_bwd",
    "sgd_momentum", "mlp_param_count", "mlp_unflatten", "mlp_step",
    "mlp_forward", "mlp_loss_only", "block_fwd_bwd", "gru_param_count",
    "gru_flatten", "gru_unflatten", "gru_step", "gru_loss_only", "gru_gates_fwd", "gru_gates_bwd",
]
