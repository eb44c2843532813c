"""Pins of the oracle's number formats and exponent rules against things other
than the oracle itself: torch's own casts, closed-form invariants and the
format tables."""

import json
import os

import numpy as np
import pytest
import torch

from oracle import formats

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def all_bf16_values():
    bits = np.arange(1 << 16, dtype=np.uint32) << 16
    v = bits.view(np.float32)
    return v[np.isfinite(v)].astype(np.float64)


def test_e4m3_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = formats.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    np.testing.assert_array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(ours[ok], ref[ok])
    assert formats.e4m3_decode(np.uint8(0x7E)) == formats.E4M3_MAX == 448.0


@pytest.mark.parametrize("scale_exp", list(range(-20, 21, 4)) + [-9, -6, 1, 3, 8])
def test_e4m3_encode_matches_torch_every_bf16(scale_exp):
    """Every finite bf16 value times 2**scale_exp, in range, against torch's
    round-to-nearest-even cast (bits compared, sign of zero included)."""
    x = np.ldexp(all_bf16_values(), scale_exp)
    x = x[np.abs(x) <= 464.0]          # 464 is the largest value that rounds to 448
    ours = formats.e4m3_encode(x)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert x.size > 1000
    np.testing.assert_array_equal(ours, ref)


def test_e4m3_rounding_examples():
    # ties to even between neighbours, subnormal step 2**-9, largest 448
    cases = {1.0625: 1.0, 1.1875: 1.25, 2.0 ** -10: 0.0, 3 * 2.0 ** -10: 2.0 ** -8,
             464.0: 448.0, 0.015625: 0.015625, -2.0 ** -11: -0.0}
    for x, want in cases.items():
        got = float(formats.e4m3_round(x))
        assert got == want and np.signbit(got) == np.signbit(want), (x, got, want)
    with pytest.raises(OverflowError):
        formats.e4m3_round(470.0)
    assert formats.e4m3_round(470.0, saturate=True) == 448.0
    assert formats.e4m3_encode(-2.0 ** -11) == 0x80


def test_e2m1_table_and_ties():
    np.testing.assert_array_equal(formats.e2m1_decode(np.arange(8, dtype=np.uint8)),
                                  [0, .5, 1, 1.5, 2, 3, 4, 6])
    ties = {0.25: 0.0, 0.75: 1.0, 1.25: 1.0, 1.75: 2.0, 2.5: 2.0, 3.5: 4.0, 5.0: 4.0,
            7.0: 6.0, -0.25: -0.0, -5.0: -4.0}
    for x, want in ties.items():
        assert float(formats.e2m1_round(x)) == want, x
    codes = formats.e2m1_encode(np.array([0.75, -3.0]))
    assert codes.tolist() == [2, 8 | 5]


def test_bf16_and_fp16_rounding_match_library_casts():
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(200000) * 10.0 ** rng.integers(-30, 30, 200000),
                        rng.standard_normal(1000) * 1e-40])
    ours = formats.bf16_round(x.astype(np.float32).astype(np.float64))
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(ours, ref.astype(np.float64))
    y = rng.standard_normal(200000) * 10.0 ** rng.integers(-8, 4, 200000)
    np.testing.assert_array_equal(formats.fp16_round(y), y.astype(np.float16).astype(np.float64))


def test_roundup_exponent_is_tight_and_never_clamps():
    """For every nonzero amax: 224 < amax * 2**-e <= 448 (never clamps, and one
    exponent lower would clamp)."""
    rng = np.random.default_rng(3)
    samples = list(np.ldexp(rng.uniform(1, 2, 5000), rng.integers(-60, 60, 5000)))
    for k in range(-40, 40):
        samples += [448.0 * 2.0 ** k, np.nextafter(448.0 * 2.0 ** k, np.inf),
                    1.75 * 2.0 ** k, np.nextafter(1.75 * 2.0 ** k, np.inf), 2.0 ** k]
    for a in samples:
        e = formats.roundup_exponent(a)
        s = a * 2.0 ** -e
        assert 224.0 < s <= 448.0, (a, e, s)
        assert formats.e4m3_round(a * 2.0 ** -e) <= 448.0
    assert formats.roundup_exponent(0.0) == -127
    assert formats.roundup_exponent(448.0) == 0
    assert formats.roundup_exponent(448.0001) == 1
    assert formats.roundup_exponent(1e-300) == -127          # UE8M0 lower clamp
    # closed form from the fp32 bits: amax = m 2**k, m in [1,2): e = k-8 if m <= 1.75 else k-7
    for a in samples[:2000]:
        m, ex = np.frexp(a)
        m, k = 2 * m, ex - 1
        assert formats.roundup_exponent(a) == (k - 8 if m <= 1.75 else k - 7)


def test_floor_rule_clamps_and_ceil_rule_wastes():
    # the microscaling reference floor rule lets the scaled max exceed 448
    e = formats.floor_exponent(500.0)
    assert 500.0 * 2.0 ** -e > 448.0
    assert formats.e4m3_round(500.0 * 2.0 ** -e, saturate=True) == 448.0
    # ceil(log2) - 8 never clamps but can sit a bit below the tight rule
    assert formats.ceil_log2_exponent(300.0) == 1 and formats.roundup_exponent(300.0) == 0


def test_page_facts_fixture():
    """Facts the pages state about the formats (tests/golden/page_facts.json)."""
    with open(os.path.join(GOLDEN, "page_facts.json")) as f:
        facts = json.load(f)["facts"]
    assert facts["e4m3_max"]["value"] == formats.E4M3_MAX
    mags = formats.E2M1_MAGNITUDES[1:]
    assert min(mags[1:] / mags[:-1]) == pytest.approx(facts["e2m1_min_adjacent_ratio"]["value"])
    assert facts["e2m1_magnitude_count"]["value"] == len(formats.E2M1_MAGNITUDES)
