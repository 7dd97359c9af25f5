"""Element-wise comparison rule for HIP results against the oracle.

Tolerances follow the path's precision: 1e-4 on the FP32 path, 5e-3 on the
FP16/BF16-input path, loss within 1e-5 relative.  An element passes if any of

  (A) |got - ref| <= tol * (|ref| + 1e-6)                 (the verbatim rule)
  (B) the tensor is stored in FP16/BF16 and got is within one unit in the
      last place of the oracle's value rounded to that format
  (C) |got - ref| <= tol * 1e-2 * max|ref|                (tensor-scale floor)

holds.  (B) exists because one BF16 ulp (2^-8..2^-7 relative) is larger than
5e-3, so an FP32-accumulated result may round to the neighbour of the FP64
result's rounding.  (C) applies only where the caller says the tensor is a
sum whose terms cancel (``cancel=True``): GEMM outputs, column sums, weight
and bias gradients, the momentum update (mu v - lr g, then w + vel), the
RMSNorm input gradient and recurrent quantities formed from such sums.  There
the FP32 accumulation error is an absolute amount (~sqrt(K) 2^-24 times the
partial sums), so elements that cancel to near zero carry a large relative
error that says nothing about correctness.  Elementwise outputs with no
cancelling sum (softmax gradients, row losses, normalised rows and their
statistics, gathered rows) are held to (A) and (B) alone.  A wrong index, a
missing tile or a race produces errors of the tensor's typical magnitude,
which none of the clauses admits.

Every comparison is recorded (verbatim max metric, elements admitted only by
(B) or only by (C), cosine) and the session prints the table at its end.
"""
from __future__ import annotations

import numpy as np

from oracle import round_fmt

TOL_F32 = 1e-4
TOL_LOWP = 5e-3
TOL_LOSS = 1e-5


def _ordered_bits(x: np.ndarray, fmt: str) -> np.ndarray:
    if fmt == "f16":
        b = x.astype(np.float16).view(np.int16).astype(np.int64)
        return np.where(b >= 0, b, -(b & 0x7FFF))
    if fmt == "bf16":
        b = (x.astype(np.float32).view(np.uint32) >> 16).astype(np.int64)
        return np.where(b < 0x8000, b, -(b & 0x7FFF))
    raise ValueError(fmt)


def ulp_distance(a: np.ndarray, b: np.ndarray, fmt: str) -> np.ndarray:
    return np.abs(_ordered_bits(a, fmt) - _ordered_bits(b, fmt))


REPORT: list = []


def compare(got, ref, tol: float, fmt: str | None = None, cancel: bool = False,
            floor_frac: float = 1e-2):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if got.size == 0:
        return dict(n=0, fails=0, verbatim=0.0, via_ulp=0, via_floor=0, cos=1.0, worst=None)
    finite = np.isfinite(got) & np.isfinite(ref)
    same_nonfinite = (~np.isfinite(got)) & (~np.isfinite(ref)) & (np.isnan(got) == np.isnan(ref)) & \
        (np.isnan(got) | (got == ref))
    d = np.abs(got - ref)
    rel = np.where(finite, d / (np.abs(ref) + 1e-6), np.inf)
    ok_a = finite & (d <= tol * (np.abs(ref) + 1e-6))
    ok_b = np.zeros_like(ok_a)
    if fmt in ("f16", "bf16"):
        ok_b = finite & (ulp_distance(got, round_fmt(ref, fmt), fmt) <= 1)
    scale = np.max(np.abs(ref[finite])) if finite.any() else 0.0
    ok_c = finite & (d <= tol * floor_frac * scale) if cancel else np.zeros_like(ok_a)
    ok = ok_a | ok_b | ok_c | same_nonfinite
    g, r = got[finite].ravel(), ref[finite].ravel()
    den = np.linalg.norm(g) * np.linalg.norm(r)
    cos = float(g @ r / den) if den > 0 else (1.0 if np.array_equal(g, r) else 0.0)
    bad = np.flatnonzero(~ok.ravel())
    worst = None
    if bad.size:
        i = bad[np.argmax(rel.ravel()[bad])]
        worst = (np.unravel_index(i, got.shape), got.ravel()[i], ref.ravel()[i])
    return dict(n=got.size, fails=int(bad.size), verbatim=float(np.max(rel[finite])) if finite.any() else 0.0,
                via_ulp=int(np.count_nonzero(ok_b & ~ok_a)),
                via_floor=int(np.count_nonzero(ok_c & ~ok_a & ~ok_b)), cos=cos, worst=worst)


def assert_parity(got, ref, tol: float, fmt: str | None = None, what: str = "",
                  cancel: bool = False):
    r = compare(got, ref, tol, fmt, cancel)
    REPORT.append((what, tol, fmt, cancel, r["n"], r["verbatim"], r["via_ulp"], r["via_floor"],
                   r["cos"], r["fails"]))
    assert r["fails"] == 0, f"{what}: {r['fails']}/{r['n']} elements fail; worst {r['worst']}; {r}"
    return r
