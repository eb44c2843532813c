"""NVFP4 operands of the mixed path (oracle; test infrastructure).

On the mixed path QK^T and its backward recompute use NVFP4 -- E2M1 elements,
one E4M3 scale per 16 head-dimension elements of one token, and one fp32
tensor scale -- while every other product stays E4M3 ([Summary], first
paragraph; [Reading, 4.1] and 4.6; [Reading, part 一] for the NVFP4 format).
Per-token groups keep a query's or key's representation independent of other
tokens ([Summary, §3.2 Causally Safe Scales]).

Readings (the pages print no NVFP4 formula, so parity of this reading is
UNPINNED beyond the E2M1 table and the exactness checks in the tests):

* tensor scale ``t = amax_tensor / 2688`` (one IEEE fp32 division) over the
  whole (rotated) tensor, with 2688 = 6 * 448; ``t = 1`` when the tensor is
  all zero;
* group scale ``s`` = the smallest E4M3 value ``>= amax_g / fp32(6 t)`` (one
  IEEE fp32 division), capped at 448 -- the round-up rule applied to a
  non-power-of-two scale;
* code ``= E2M1_RNE(fp32(x / fp32(s t)))`` saturating at +-6; all codes are
  0 when ``s = 0``;
* ``S_ij = t_Q t_K sum_g s_Q s_K sum_{k in g} q k``, exact in fp64, rounded
  to fp32.
"""

from __future__ import annotations

import numpy as np

from . import formats

GROUP = 16


def e4m3_round_up(x: float) -> float:
    """Smallest E4M3 value >= x (x >= 0), capped at 448."""
    if x <= 0:
        return 0.0
    r = float(formats.e4m3_round(min(x, 448.0)))
    if r < x:
        codes = np.arange(0, 0x7F, dtype=np.uint8)
        vals = formats.e4m3_decode(codes)
        r = float(np.min(vals[vals >= x])) if np.any(vals >= x) else 448.0
    return min(r, 448.0)


def quantize_nvfp4(x, amax=None):
    """x: ``[T, H, d]`` fp32-valued.  Returns (codes u8 [T,H,d] (0..15),
    group scales fp64 [T,H,d/16] (E4M3 values), tensor scale fp32, dequantized
    fp64 [T,H,d]).  ``amax`` is the tensor's max-abs; pass it when x is a
    slice of the tensor (groups are per token, so a slice quantized with the
    whole tensor's amax is the slice of the whole tensor's quantization)."""
    x = np.asarray(x, dtype=np.float32)
    T, H, d = x.shape
    if amax is None:
        amax = np.max(np.abs(x)) if x.size else np.float32(0.0)
    amax = np.float32(amax)
    t = (np.float32(amax) / np.float32(2688.0)).astype(np.float32) if amax > 0 else np.float32(1.0)
    six_t = np.float32(6.0 * np.float64(t))        # exact product, rounded once
    g = x.reshape(T, H, d // GROUP, GROUP)
    gmax = np.max(np.abs(g), axis=-1).astype(np.float32)
    need = (gmax / six_t).astype(np.float32)       # IEEE fp32 division
    scales = np.zeros(gmax.shape)
    for idx in np.ndindex(gmax.shape):
        scales[idx] = e4m3_round_up(float(need[idx]))
    st = (scales.astype(np.float32) * t).astype(np.float32)      # fp32(s * t)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(st[..., None] > 0,
                         (g.astype(np.float32) / st[..., None]).astype(np.float32), 0.0)
    codes = formats.e2m1_encode(ratio.astype(np.float64))
    deq = formats.e2m1_decode(codes) * scales[..., None] * np.float64(t)
    return codes.reshape(T, H, d), scales, t, deq.reshape(T, H, d)
