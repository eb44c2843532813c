"""Pins of the 4-bit probability operand (oracle.attention.p4_quantize,
roundup_e2m1 and the forward's ``p_format="nvfp4"``), against what the
NVFP4 element format and the pages' log-domain rule fix ([Summary, §3.5.2
Softmax Throughput and MMA Scheduling]; [Reading, 4.4] second bullet):

* the E2M1 grid: the eight magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6 and ties to
  the even code at every midpoint;
* the scale rule by search: the smallest e with max <= 6 2^e;
* the codes by exhaustive nearest search over the grid per element;
* a hand example; invariance of the codes under a power-of-two shift of a
  row (what lets the forward quantize against its running row maximum);
* the closed form of the forward when every visible probability is equal.
"""

import numpy as np
import pytest

from oracle import attention as A
from oracle import formats
from oracle.quant import quantize_qkv

GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])     # E2M1 magnitudes, code index 0..7


def test_e2m1_grid_and_ties_to_even():
    # the grid points round to themselves
    np.testing.assert_array_equal(formats.e2m1_round(GRID), GRID)
    np.testing.assert_array_equal(formats.e2m1_round(-GRID), -GRID)
    # a midpoint goes to the neighbour whose code index is even
    mids = (GRID[:-1] + GRID[1:]) / 2
    want = np.where(np.arange(7) % 2 == 0, GRID[:-1], GRID[1:])
    np.testing.assert_array_equal(formats.e2m1_round(mids), want)
    # just off a midpoint: the nearer point
    eps = 1e-9
    np.testing.assert_array_equal(formats.e2m1_round(mids - eps), GRID[:-1])
    np.testing.assert_array_equal(formats.e2m1_round(mids + eps), GRID[1:])


def test_roundup_e2m1_by_search():
    rng = np.random.default_rng(7)
    a = np.concatenate([np.ldexp(rng.uniform(0.5, 1.0, 4000), rng.integers(-40, 40, 4000)),
                        np.ldexp(6.0, np.arange(-20, 20)), np.ldexp(1.5, np.arange(-20, 20)),
                        np.nextafter(np.ldexp(6.0, np.arange(-20, 20)), np.inf)])
    got = A.roundup_e2m1(a)
    for ai, gi in zip(a, got):
        e = -200
        while ai > 6.0 * 2.0 ** e:
            e += 1
        assert gi == e, (ai, gi, e)


def _p4_by_search(x, valid):
    out = np.zeros_like(x)
    for r in range(x.shape[0]):
        for g0 in range(0, x.shape[1], A.P4_GROUP):
            idx = [j for j in range(g0, min(g0 + A.P4_GROUP, x.shape[1])) if valid[r, j]]
            amax = max([x[r, j] for j in idx], default=0.0)
            if amax <= 0:
                continue
            e = -300
            while amax > 6.0 * 2.0 ** e:
                e += 1
            for j in idx:
                v = x[r, j] / 2.0 ** e
                dist = np.abs(GRID - v)
                best = np.flatnonzero(dist == dist.min())
                k = best[0] if len(best) == 1 else best[best % 2 == 0][0]   # tie: even code
                out[r, j] = formats.e4m3_round(GRID[k] * 2.0 ** e)
    return out


def test_p4_quantize_matches_exhaustive_search():
    rng = np.random.default_rng(11)
    for trial in range(20):
        rows, keys = 5, int(rng.integers(1, 70))
        x = np.ldexp(rng.uniform(0, 1, (rows, keys)), rng.integers(-12, 9, (rows, keys)))
        x[rng.uniform(size=x.shape) < 0.1] = 0.0
        # exact midpoints of some group scale, to exercise the ties
        x[:, ::7] = np.ldexp(rng.choice([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], (rows, len(range(0, keys, 7)))), 2)
        valid = rng.uniform(size=x.shape) < 0.85
        np.testing.assert_array_equal(A.p4_quantize(x, valid), _p4_by_search(x, valid), err_msg=f"trial {trial}")


def test_p4_hand_example():
    x = np.array([[6, 5, 4.5, 3.2, 2.9, 1.2, 0.8, 0.3, 0.24, 0.26, 0, 0.75, 1.25, 1.75, 2.5, 3.5]], float)
    want = np.array([[6, 4, 4, 3, 3, 1, 1, 0.5, 0, 0.5, 0, 1, 1, 2, 2, 4]], float)
    np.testing.assert_array_equal(A.p4_quantize(x, np.ones_like(x, bool)), want)
    # a masked element takes no part in the group's scale
    valid = np.ones_like(x, bool)
    valid[0, 0] = False          # without the 6, the largest is 5: scale 2^0 still (5 <= 6)
    np.testing.assert_array_equal(A.p4_quantize(x, valid)[0, 1:], want[0, 1:])
    valid[0, [0, 1, 2, 3, 4, 15]] = False   # largest visible 2.5 <= 6 x 2^-1: scale 2^-1
    got = A.p4_quantize(x, valid)[0]
    # x / 0.5 = 2.4, 1.6, .6, .48, .52, 0, 1.5, 2.5 (tie: 2), 3.5 (tie: 4), 5 (tie: 4)
    want2 = np.array([0, 0, 0, 0, 0, 1.0, 0.75, 0.25, 0.25, 0.25, 0, 0.75, 1.0, 2.0, 2.0, 0])
    np.testing.assert_array_equal(got, want2)


def test_p4_codes_shift_with_the_row_maximum():
    # values whose 4-bit results stay inside E4M3's range at every shift, so
    # the carry into E4M3 is exact
    rng = np.random.default_rng(3)
    x = np.ldexp(rng.uniform(0.5, 1.0, (8, 64)), rng.integers(-1, 6, (8, 64)))
    valid = rng.uniform(size=x.shape) < 0.9
    base = A.p4_quantize(x, valid)
    for k in (-3, -1, 1, 2):
        np.testing.assert_array_equal(A.p4_quantize(np.ldexp(x, k), valid), np.ldexp(base, k))


def test_p4_error_and_tight_scale():
    rng = np.random.default_rng(5)
    x = np.ldexp(rng.uniform(0.0, 1.0, (16, 96)), 8)
    valid = np.ones_like(x, bool)
    q = A.p4_quantize(x, valid)
    for g0 in range(0, 96, 16):
        seg, qs = x[:, g0:g0 + 16], q[:, g0:g0 + 16]
        e = A.roundup_e2m1(seg.max(axis=1))
        step = np.ldexp(1.0, e)[:, None]          # half of the grid's widest gap (2) times 2^e
        assert np.all(np.abs(qs - seg) <= step)
        top = qs.max(axis=1)
        assert np.all(top >= np.ldexp(3.0, e)) and np.all(top <= np.ldexp(6.0, e))


@pytest.mark.parametrize("hadamard", [False, True])
def test_p4_forward_closed_form_uniform_probabilities(hadamard):
    """Q = 0: every visible score is 0, P = 1 for every visible key, which
    the 4-bit operand holds exactly (256 = 4 x 2^6); with V rows of one
    magnitude per block the fold factors are 1, so O_i is the mean of the
    dequantized V rows j <= i (as on the 8-bit path), and l_i = i + 1."""
    rng = np.random.default_rng(9)
    L, d = 70, 64
    q = np.zeros((L, d))
    k = rng.standard_normal((L, d))
    v = np.where(rng.uniform(size=(L, d)) < 0.5, -1.0, 1.0) * 0.75
    do = rng.standard_normal((L, d))
    cu = [0, L]
    num = A.Numerics(p_format="nvfp4", hadamard=hadamard, round_outputs=False)
    res = A.training_call(q[:, None, :], k[:, None, :], v[:, None, :], do[:, None, :], cu, num)
    qt = quantize_qkv(q[:, None, :], k[:, None, :], v[:, None, :], cu, hadamard)
    vd = qt["v"][:, 0]
    want = np.cumsum(vd, axis=0) / np.arange(1, L + 1)[:, None]
    np.testing.assert_allclose(res["o"][:, 0], want, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(res["row_sum"][0], np.arange(1, L + 1))
    # the same call on the 8-bit operand gives the same O
    res8 = A.training_call(q[:, None, :], k[:, None, :], v[:, None, :], do[:, None, :], cu,
                           A.Numerics(hadamard=hadamard, round_outputs=False))
    np.testing.assert_array_equal(res["o"], res8["o"])


def test_p4_span_covers_brute_force_evaluations():
    """Every value the 4-bit operand takes when each element of a row moves
    inside its relative interval lies within the span ``_p4_span`` reports
    (brute force over sampled points of the intervals)."""
    from oracle.decisions import _p4_span
    rng = np.random.default_rng(21)
    x = np.ldexp(rng.uniform(0.5, 1.0, (6, 48)), rng.integers(-8, 9, (6, 48)))
    # put some group maxima right at a scale boundary and elements at midpoints
    x[:, 0] = np.ldexp(6.0, 3)
    x[:, 17] = np.ldexp(2.5, 2)
    valid = rng.uniform(size=x.shape) < 0.9
    rel = 1e-3
    span = _p4_span(x * (1 - rel), x * (1 + rel), valid)
    ref = A.p4_quantize(x, valid)
    for t in np.linspace(-1, 1, 9):
        for u in np.linspace(-1, 1, 5):
            y = x * (1 + rel * np.where(np.arange(48) % 2 == 0, t, u)[None, :])
            got = A.p4_quantize(y, valid)
            assert np.all(np.abs(got - ref) <= span + 0.0), (t, u)
    assert np.any(span > 0)        # the boundary cases do open a span
