"""Storage rounding (oracle side; test infrastructure only).

The GPU path stores tensors as IEEE binary32, binary16 or bfloat16 and always
converts with round-to-nearest, ties to even.  The pages fix the principle
(accumulate and apply the epilogue in FP32, convert once at the final store:
"The Work Moved Down a Layer", section "The Debugging Lesson Was Numerical");
the formats themselves are the IEEE / bfloat16 definitions.

``round_fmt`` rounds float64 values *directly* to the target format (no
intermediate float32 step), with gradual underflow and overflow to +-inf.
"""
from __future__ import annotations

import numpy as np

# name -> (significand bits incl. the hidden bit, minimum normal exponent,
#          exponent at which the value overflows: |x| >= 2**overflow -> inf)
FORMATS = {
    "f32": (24, -126, 128),
    "f16": (11, -14, 16),
    "bf16": (8, -126, 128),
}


def round_fmt(x, fmt: str) -> np.ndarray:
    """Round float64 ``x`` to the nearest value of ``fmt`` (ties to even).

    ``fmt`` is "f32", "f16", "bf16" or "f64" (identity).  The result is
    float64 holding exactly representable values.

    A finite x = m * 2**e with 0.5 <= |m| < 1 lies in the binade whose
    spacing (quantum) is 2**(e - p); below the smallest normal exponent the
    quantum stays at the subnormal spacing 2**(emin - p + 1).  Rounding is
    rint (ties to even) of x / quantum; results at or beyond 2**overflow
    become infinities of the same sign, as IEEE round-to-nearest requires.
    """
    x = np.asarray(x, dtype=np.float64)
    if fmt == "f64":
        return x.copy()
    p, emin, eover = FORMATS[fmt]
    finite = np.isfinite(x)
    xf = np.where(finite, x, 0.0)
    _, e = np.frexp(xf)
    q = np.maximum(e - p, emin - p + 1)
    r = np.ldexp(np.rint(np.ldexp(xf, -q)), q)
    r = np.where(np.abs(r) >= np.ldexp(1.0, eover), np.copysign(np.inf, xf), r)
    return np.where(finite, r, x)
