"""Hadamard rotation of the head dimension (oracle; test infrastructure).

The fused quantizer may first mix the head-dimension channels of Q and K with
an orthogonal Hadamard transform, the QuIP/QuIP#-style incoherence step that
spreads outlier channels; dot products are unchanged ([Reading, 4.4], first
bullet "融合量化").  The pages name neither the matrix nor the order of
operations.  Reading taken here: the Sylvester matrix ``H_d`` (entries +-1,
``H_2n = [[H_n, H_n], [H_n, -H_n]]``) scaled by ``1/sqrt(d)``, no random signs,
applied as an fp32 fast Walsh-Hadamard transform in the fixed order below, so
that a GPU running the same sequence of fp32 additions gets the same bits.
"""

from __future__ import annotations

import numpy as np


def sylvester(d: int) -> np.ndarray:
    """The +-1 Sylvester Hadamard matrix of order ``d`` (a power of two)."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    h = np.ones((1, 1), dtype=np.int64)
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def inv_sqrt_fp32(d: int) -> np.float32:
    """fp32 nearest to 1/sqrt(d): exactly 0.125 for d = 64; for d = 128 the
    fp32 rounding of 2**-3.5."""
    return np.float32(1.0 / np.sqrt(np.float64(d)))


def fwht_fp32(x: np.ndarray) -> np.ndarray:
    """Normalised Hadamard transform of the last axis, in fp32.

    For h = 1, 2, 4, ..., d/2: every pair (a, a + h) inside each aligned group
    of 2h channels becomes (x_a + x_{a+h}, x_a - x_{a+h}), each an fp32 sum
    rounded to nearest-even.  Then every element is multiplied once by
    fp32(1/sqrt(d)).  In exact arithmetic the result is ``x @ H_d / sqrt(d)``.
    """
    y = np.array(x, dtype=np.float32, copy=True)
    d = y.shape[-1]
    if d & (d - 1):
        raise ValueError("head dim must be a power of two")
    h = 1
    while h < d:
        g = y.reshape(y.shape[:-1] + (d // (2 * h), 2, h))
        lo = g[..., 0, :].copy()
        hi = g[..., 1, :].copy()
        g[..., 0, :] = lo + hi          # float32 + float32 -> float32 (RNE)
        g[..., 1, :] = lo - hi
        y = g.reshape(y.shape)
        h *= 2
    return (y * inv_sqrt_fp32(d)).astype(np.float32)


def rotate_back_fp64(g: np.ndarray) -> np.ndarray:
    """Gradient w.r.t. the unrotated input: ``g @ H_d / sqrt(d)`` (the
    normalised matrix is symmetric and orthogonal, so it is its own inverse
    transpose).  Exact matrix, fp64."""
    d = g.shape[-1]
    return np.asarray(g, dtype=np.float64) @ (sylvester(d).astype(np.float64) / np.sqrt(d))
