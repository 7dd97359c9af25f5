"""Transformer MLP block, forward and backward (oracle side; test infrastructure only).

The block is the five-step chain RMSNorm -> up projection -> LeakyReLU^2 ->
down projection -> residual ("Full-Depth MLP Megakernel + Fused Attention
Preprocessing", section "What Worked"), with the up projection a single
[D x F] matrix without bias and the slope of the leaky part 0.5.  RMSNorm
statistics are FP32 ("The Work Moved Down a Layer", "The Debugging Lesson Was
Numerical").  Backward by the chain rule, with the activation derivative
applied as a dgrad-GEMM epilogue ("... Megakernel ...", "Credits": backward
epilogue).

Storage plan ``fmt`` = "bf16": x, n, u, a, y, du, dx stored BF16; the row
statistic r, dn and both weight gradients FP32; the derivative factor is
evaluated on the *stored* u.  ``fmt`` = "f64" rounds nothing.

    r  = 1/sqrt(mean_j x^2 + eps)           n  = x r
    u  = n W_up                              a  = leaky(u)^2   (from unrounded u)
    y  = x + a W_down
    du = (dy W_down^T) * act'(u)             dW_down = a^T dy
    dn = du W_up^T                           dW_up   = n^T du
    dx = dy + r (dn - xh mean_j(dn xh)),     xh = x r

``given`` may supply the GPU's stored intermediates by name ("r", "n", "u",
"a", "du", "dn"); each stage then starts from those values, which checks every
stage on its own inputs.
"""
from __future__ import annotations

import numpy as np

from .ops import gemm_epilogue, rmsnorm_fwd, rmsnorm_bwd


def block_fwd_bwd(x, w_up, w_down, dy, eps: float = 1e-6, slope: float = 0.5,
                  fmt: str = "bf16", given=None):
    given = given or {}
    lo = fmt
    hi = "f32" if fmt != "f64" else "f64"
    x = np.asarray(x, dtype=np.float64)
    n, r = rmsnorm_fwd(x, eps, y_fmt=lo, r_fmt=hi)
    out = {"r": r, "n": n}
    n_in = given.get("n", n)
    r_in = given.get("r", r)
    a, u = gemm_epilogue(n_in, w_up, "NN", act="lrelu_sq", slope=slope,
                         out_fmt=lo, pre_fmt=lo)
    out.update(u=u, a=a)
    u_in = given.get("u", u)
    a_in = given.get("a", a)
    y, _ = gemm_epilogue(a_in, w_down, "NN", residual=x, out_fmt=lo)
    out["y"] = y
    du, _ = gemm_epilogue(dy, w_down, "NT", act="lrelu_sq_bwd", slope=slope,
                          aux=u_in, out_fmt=lo)
    out["du"] = du
    du_in = given.get("du", du)
    out["dW_down"], _ = gemm_epilogue(a_in, dy, "TN", out_fmt=hi)
    dn, _ = gemm_epilogue(du_in, w_up, "NT", out_fmt=hi)
    out["dn"] = dn
    dn_in = given.get("dn", dn)
    out["dW_up"], _ = gemm_epilogue(n_in, du_in, "TN", out_fmt=hi)
    out["dx"], _ = rmsnorm_bwd(x, r_in, dn_in, dres=dy, dx_fmt=lo)
    return out
