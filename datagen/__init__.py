"""Seeded synthetic inputs shared by the oracle-side tests and the HIP path.

This module only draws random numbers and arranges them in the shapes of the
workloads; it holds none of the method's arithmetic (no GEMM, no loss, no
normalisation, no update rule).  Every array it returns is float64 (or int32
for labels / tokens) and every floating value is *exactly representable* in
the storage format requested, so both sides of a parity test start from the
same bit patterns:

* ``"f32"``  -- values drawn in float64 then cast with numpy's float32 cast;
* ``"f16"``  -- values cast with numpy's float16 cast;
* ``"bf16"`` -- values cast to float32 and the low 16 bits of the float32
  pattern cleared (a truncation, chosen as the generator's distribution, not a
  rounding rule of the method).

Workload recipes (sizes, distributions) follow the configurations named in
the design notes: a 784-256-10 MLP on template-plus-noise 28x28 images
(as in "Capstone 5: train a network with your CUDA kernels", section "The
minimum model", which trains on Fashion-MNIST -- not available here, so the
template-plus-noise images stand in for it), the standalone GEMM shapes, the
784-2048-2048-10 MLP, the transformer MLP block and the byte-level GRU LM.
"""
from __future__ import annotations

import numpy as np

WEIGHT_SEED = 20260829          # seed of the capstone recipe (weights)

# Fixed stream offsets so that every consumer derives the same sub-streams.
_STREAM = {
    "templates": 1, "noise": 2, "labels": 3, "gemm_a": 4, "gemm_b": 5,
    "gemm_bias": 6, "block_x": 7, "block_w": 8, "block_dy": 9, "tokens": 10,
    "gru_w": 11, "misc": 12,
}


def rng(seed: int, stream: str, index: int = 0) -> np.random.Generator:
    """A numpy PCG64 generator for (seed, named stream, index)."""
    return np.random.Generator(np.random.PCG64([int(seed), _STREAM[stream], int(index)]))


def representable(x: np.ndarray, fmt: str) -> np.ndarray:
    """Return float64 values exactly representable in ``fmt`` (see module doc)."""
    x = np.asarray(x, dtype=np.float64)
    if fmt == "f64":
        return x.copy()
    if fmt == "f32":
        return x.astype(np.float32).astype(np.float64)
    if fmt == "f16":
        return x.astype(np.float16).astype(np.float64)
    if fmt == "bf16":
        bits = x.astype(np.float32).view(np.uint32) & np.uint32(0xFFFF0000)
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown storage format {fmt!r}")


# ---------------------------------------------------------------------------
# MLP workloads (784-256-10 FP32 and 784-2048-2048-10 FP16)
# ---------------------------------------------------------------------------

def template_images(n: int, seed: int, fmt: str = "f32", n_classes: int = 10,
                    n_pix: int = 784, batch: int = 0):
    """Template-plus-noise images and uniform labels.

    Each class c owns a template T_c with pixels uniform on {0..191}; an image
    of class c is T_c + U{0..64} (so it stays within one byte, no clipping),
    divided by 255 in float64 and made representable in ``fmt``.  Labels are
    uniform over the classes.  The templates depend on ``seed`` only; labels
    and noise also on ``batch``, so batch i of a long run is drawn on its own.
    """
    t = rng(seed, "templates").integers(0, 192, size=(n_classes, n_pix), dtype=np.int64)
    lab_rng = rng(seed, "labels", batch)
    noi_rng = rng(seed, "noise", batch)
    labels = lab_rng.integers(0, n_classes, size=n).astype(np.int32)
    pix = t[labels] + noi_rng.integers(0, 65, size=(n, n_pix), dtype=np.int64)
    x = representable(pix.astype(np.float64) / 255.0, fmt)
    return x, labels


def mlp_dims_cfg0():
    return [784, 256, 10]


def mlp_dims_cfg2():
    return [784, 2048, 2048, 10]


def he_uniform_flat(dims, seed: int = WEIGHT_SEED) -> np.ndarray:
    """Flat float32-representable parameter vector [W1, b1, W2, b2, ...].

    W_l is row-major [d_{l-1} x d_l] drawn U(-sqrt(6/fan_in), +sqrt(6/fan_in))
    with fan_in = d_{l-1}; biases start at zero.
    """
    g = np.random.Generator(np.random.PCG64([int(seed), 0]))
    parts = []
    for fi, fo in zip(dims[:-1], dims[1:]):
        lim = np.sqrt(6.0 / fi)
        parts.append(g.uniform(-lim, lim, size=fi * fo))
        parts.append(np.zeros(fo))
    return representable(np.concatenate(parts), "f32")


# ---------------------------------------------------------------------------
# Standalone GEMM (+bias+act) workload
# ---------------------------------------------------------------------------

def gemm_operands(M: int, N: int, K: int, layout: str, seed: int = 1, fmt: str = "f16"):
    """A, B ~ N(0, std = 1/sqrt(K)) stored in the layout's shapes; bias ~ N(0, 0.1) f32.

    NN: A [M x K], B [K x N];  NT: A [M x K], B [N x K];  TN: A [K x M], B [K x N].
    """
    std = 1.0 / np.sqrt(K)
    sa = (M, K) if layout in ("NN", "NT") else (K, M)
    sb = (K, N) if layout in ("NN", "TN") else (N, K)
    a = representable(rng(seed, "gemm_a").normal(0.0, std, size=sa), fmt)
    b = representable(rng(seed, "gemm_b").normal(0.0, std, size=sb), fmt)
    bias = representable(rng(seed, "gemm_bias").normal(0.0, 0.1, size=N), "f32")
    return a, b, bias


def integer_matrix(shape, seed: int, lo: int = -2, hi: int = 2) -> np.ndarray:
    """Small integers (exact in every format and in any summation order)."""
    return rng(seed, "misc").integers(lo, hi + 1, size=shape).astype(np.float64)


def normal(shape, std: float, seed: int, stream: str = "misc", fmt: str = "f32") -> np.ndarray:
    return representable(rng(seed, stream).normal(0.0, std, size=shape), fmt)


# ---------------------------------------------------------------------------
# Transformer MLP block (RMSNorm -> up -> LeakyReLU^2 -> down -> residual)
# ---------------------------------------------------------------------------

def block_inputs(R: int, D: int = 512, F: int = 1536, seed: int = 3, fmt: str = "bf16"):
    """x ~ N(0,1) [R x D], W_up ~ N(0,0.02) [D x F], W_down ~ N(0,0.02) [F x D], dy ~ N(0,1)."""
    x = representable(rng(seed, "block_x").normal(0.0, 1.0, size=(R, D)), fmt)
    gw = rng(seed, "block_w")
    w_up = representable(gw.normal(0.0, 0.02, size=(D, F)), fmt)
    w_down = representable(gw.normal(0.0, 0.02, size=(F, D)), fmt)
    dy = representable(rng(seed, "block_dy").normal(0.0, 1.0, size=(R, D)), fmt)
    return x, w_up, w_down, dy


# ---------------------------------------------------------------------------
# GRU byte LM
# ---------------------------------------------------------------------------

def zipf_tokens(n_seq: int, length: int, seed: int = 4, vocab: int = 256, s: float = 1.1):
    """Tokens drawn from P(k) proportional to k^-s, k = 1..vocab, emitted as byte k-1.

    Sampled by inverse CDF: a uniform draw u picks the first k whose
    cumulative probability exceeds u.
    """
    k = np.arange(1, vocab + 1, dtype=np.float64)
    p = k ** (-s)
    cdf = np.cumsum(p / p.sum())
    u = rng(seed, "tokens").random(size=(n_seq, length))
    tok = np.searchsorted(cdf, u, side="right")
    return np.minimum(tok, vocab - 1).astype(np.int32)


def gru_params(H: int = 1024, V: int = 256, seed: int = WEIGHT_SEED):
    """GRU LM parameters as a dict of float32-representable float64 arrays.

    E [V x H] ~ N(0,1); W_i, W_h [H x 3H] and b_i, b_h [3H] ~ U(+-1/sqrt(H));
    W_c [H x V] ~ U(+-1/sqrt(H)); b_c = 0.  Gate blocks along 3H are (r, z, n).
    """
    g = rng(seed, "gru_w")
    lim = 1.0 / np.sqrt(H)
    out = {
        "E": g.normal(0.0, 1.0, size=(V, H)),
        "W_i": g.uniform(-lim, lim, size=(H, 3 * H)),
        "b_i": g.uniform(-lim, lim, size=3 * H),
        "W_h": g.uniform(-lim, lim, size=(H, 3 * H)),
        "b_h": g.uniform(-lim, lim, size=3 * H),
        "W_c": g.uniform(-lim, lim, size=(H, V)),
        "b_c": np.zeros(V),
    }
    return {k: representable(v, "f32") for k, v in out.items()}


GRU_PARAM_ORDER = ("E", "W_i", "b_i", "W_h", "b_h", "W_c", "b_c")
