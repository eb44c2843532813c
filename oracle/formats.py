"""Number formats and the scale-exponent rules (oracle; test infrastructure).

Every rounding here is written out from its definition: the exact fp64 value is
placed on the target grid with round-to-nearest, ties-to-even (``np.rint``),
sign kept, so a negative value that rounds to zero keeps its sign bit.

Formats and where the method uses them:

* E4M3 (OCP "FN" flavour: bias 7, 3 fraction bits, subnormals down to 2^-9,
  largest finite 448, no infinities) -- the 8-bit payload of Q, K, V, dO,
  the probability operand and dS.  [Summary, §3.1 Token-Block Scaling];
  [Reading, 4.1] (codes times a shared power of two) and [Reading, 4.2]
  (448 is the E4M3 ceiling that a scaled maximum must not exceed).
* UE8M0 -- an unsigned biased power-of-two exponent byte, ``e + 127``; the
  shared scale of a token block.  [Reading, part 一, the microscaling
  background paragraph].
* E2M1 -- the 4-bit NVFP4 element (magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6).
  [Reading, part 一] and [Reading, 4.1] (NVFP4 scores).
* bf16 / fp16 -- output and accumulator formats.
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E2M1_MAX = 6.0
E8M0_BIAS = 127
EXP_MIN, EXP_MAX = -127, 127   # the range a UE8M0 byte can hold (255 is NaN)


# ----------------------------------------------------------------------------
# Generic round-to-nearest-even onto a binary floating-point grid
# ----------------------------------------------------------------------------

def round_to_grid(x, frac_bits: int, emin: int, max_finite: float | None = None,
                  saturate: bool = False) -> np.ndarray:
    """Round fp64 ``x`` to the nearest value of a binary format, ties to even.

    The format has ``frac_bits`` stored fraction bits, minimum normal exponent
    ``emin`` (subnormals share that binade's spacing) and largest finite value
    ``max_finite``.  A result above ``max_finite`` raises unless ``saturate``
    is set, in which case it is clamped (the microscaling conversion's clamp).
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    with np.errstate(divide="ignore"):
        _, ex = np.frexp(a)               # a = m * 2**ex, m in [0.5, 1)
    e = np.maximum(ex - 1, emin)          # binade of a (or emin if subnormal)
    q = np.ldexp(a, frac_bits - e)        # exact: scaling by a power of two
    r = np.ldexp(np.rint(q), e - frac_bits)
    if max_finite is not None:
        over = r > max_finite
        if np.any(over):
            if not saturate:
                raise OverflowError("value rounds above the format's largest finite value")
            r = np.where(over, max_finite, r)
    return np.copysign(r, x)


def bf16_round(x) -> np.ndarray:
    """fp64 -> nearest bf16 value (8 significant bits), ties to even."""
    return round_to_grid(x, 7, -126)


def fp16_round(x) -> np.ndarray:
    """fp64 -> nearest IEEE half value, ties to even."""
    return round_to_grid(x, 10, -14, 65504.0)


def fp32_round(x) -> np.ndarray:
    """fp64 -> nearest fp32 (IEEE, ties to even), returned as fp64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------
# E4M3 (OCP FN)
# ----------------------------------------------------------------------------

def e4m3_round(x, saturate: bool = False) -> np.ndarray:
    """Nearest E4M3 value of fp64 ``x`` (RNE; 448 is the largest finite)."""
    return round_to_grid(x, 3, -6, E4M3_MAX, saturate)


def e4m3_bits(v) -> np.ndarray:
    """Bit pattern (uint8) of values that are already exact E4M3 values."""
    v = np.asarray(v, dtype=np.float64)
    sign = np.signbit(v).astype(np.uint8)
    a = np.abs(v)
    sub = a < 2.0 ** -6
    with np.errstate(divide="ignore"):
        _, ex = np.frexp(a)
    e = ex - 1
    mant_norm = np.ldexp(a, 3 - e) - 8.0
    field_e = np.where(sub, 0, e + 7)
    mant = np.where(sub, np.ldexp(a, 9), mant_norm)
    if np.any((mant < 0) | (mant > 7) | (mant != np.floor(mant))):
        raise ValueError("e4m3_bits: input is not an exact E4M3 value")
    return ((sign << 7) | (field_e.astype(np.uint8) << 3) | mant.astype(np.uint8)).astype(np.uint8)


def e4m3_encode(x, saturate: bool = False) -> np.ndarray:
    """fp64 -> E4M3 code bytes (RNE, sign-preserving zero)."""
    return e4m3_bits(e4m3_round(x, saturate))


def e4m3_decode(codes) -> np.ndarray:
    """E4M3 code bytes -> fp64 values (0x7F / 0xFF decode to NaN)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    fe = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(fe == 0, np.ldexp(m.astype(np.float64), -9),
                   np.ldexp(1.0 + m / 8.0, fe - 7))
    val = np.where((c & 0x7F) == 0x7F, np.nan, val)
    return sign * val


# ----------------------------------------------------------------------------
# E2M1 (NVFP4 element)
# ----------------------------------------------------------------------------

E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_round(x) -> np.ndarray:
    """Nearest E2M1 value, ties to even, saturating at +-6 (1 fraction bit,
    minimum normal exponent 0, so the subnormal step is 0.5)."""
    return round_to_grid(x, 1, 0, E2M1_MAX, saturate=True)


def e2m1_encode(x) -> np.ndarray:
    """fp64 -> 4-bit E2M1 codes (uint8 holding 0..15; bit 3 is the sign)."""
    v = e2m1_round(x)
    idx = np.searchsorted(E2M1_MAGNITUDES, np.abs(v))
    if not np.all(E2M1_MAGNITUDES[idx] == np.abs(v)):
        raise AssertionError("e2m1 rounding left the grid")
    return ((np.signbit(v).astype(np.uint8) << 3) | idx.astype(np.uint8)).astype(np.uint8)


def e2m1_decode(codes) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8)
    return np.where(c & 8, -1.0, 1.0) * E2M1_MAGNITUDES[c & 7]


# ----------------------------------------------------------------------------
# Shared power-of-two exponent rules
# ----------------------------------------------------------------------------

def roundup_exponent(amax: float, ceiling: float = E4M3_MAX) -> int:
    """Smallest integer e with ``amax <= ceiling * 2**e``; 0 maps to -127.

    This is the method's scale rule: the exponent is rounded up so the scaled
    block maximum never exceeds the E4M3 ceiling and nothing is clamped
    ([Summary, §3.2 Causally Safe Scales]; [Reading, 4.2]).  Of the exponents
    that never clamp it is the tightest.  The result is clamped to the UE8M0
    range [-127, 127]; the lower clamp keeps ``amax <= ceiling * 2**e``.
    """
    amax = float(amax)
    if not np.isfinite(amax) or amax < 0:
        raise ValueError("amax must be finite and non-negative")
    if amax == 0.0:
        return EXP_MIN
    e = int(np.floor(np.log2(amax / ceiling)))
    while amax > ceiling * 2.0 ** e:          # step up until it fits ...
        e += 1
    while amax <= ceiling * 2.0 ** (e - 1):   # ... and down while it still fits
        e -= 1
    return int(min(max(e, EXP_MIN), EXP_MAX))


def ceil_log2_exponent(amax: float) -> int:
    """Alternative never-clamping rule ``ceil(log2 amax) - 8`` (can waste a
    bit).  Kept as a switch, not the default."""
    amax = float(amax)
    if amax == 0.0:
        return EXP_MIN
    _, ex = np.frexp(amax)
    c = ex - 1 if amax == 2.0 ** (ex - 1) else ex   # ceil(log2(amax))
    return int(min(max(c - 8, EXP_MIN), EXP_MAX))


def floor_exponent(amax: float) -> int:
    """The microscaling reference conversion ``floor(log2 amax) - 8`` (E4M3's
    largest exponent is 8).  The scaled maximum can exceed 448 and is then
    clamped -- the leak mechanism the method removes ([Reading, 4.2]).  Used
    only as a negative control."""
    amax = float(amax)
    if amax == 0.0:
        return EXP_MIN
    _, ex = np.frexp(amax)
    return int(min(max(ex - 1 - 8, EXP_MIN), EXP_MAX))


EXPONENT_RULES = {
    "roundup": roundup_exponent,
    "ceil": ceil_log2_exponent,
    "floor": floor_exponent,
}


def e8m0_byte(e) -> np.ndarray:
    """UE8M0 byte of an exponent in [-127, 127]."""
    e = np.asarray(e, dtype=np.int64)
    if np.any((e < EXP_MIN) | (e > EXP_MAX)):
        raise ValueError("exponent outside the UE8M0 range")
    return (e + E8M0_BIAS).astype(np.uint8)
