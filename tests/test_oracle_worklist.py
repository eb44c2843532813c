"""Pins of the oracle's work list and NVFP4 operands."""

import numpy as np
import pytest

from oracle import formats, nvfp4, worklist
from precision_causal_attention_hadamard_amd import workloads as W


def touched_pairs_bruteforce(L, bq, bk):
    """(q tile, k tile) pairs with at least one causal (j <= i) element."""
    pairs = set()
    for i in range(L):
        for j in range(i + 1):
            pairs.add((i // bq, j // bk))
    return pairs


@pytest.mark.parametrize("L", [1, 17, 64, 100, 129, 300])
@pytest.mark.parametrize("bq,bk", [(128, 64), (64, 128), (64, 64), (32, 128)])
def test_costs_equal_bruteforce_tile_counts(L, bq, bk):
    pairs = touched_pairs_bruteforce(L, bq, bk)
    for t in range(-(-L // bq)):
        assert worklist.fwd_cost(t, L, bq, bk) == sum(1 for p in pairs if p[0] == t)
    for u in range(-(-L // bk)):
        assert worklist.bwd_cost(u, L, bq, bk) == sum(1 for p in pairs if p[1] == u)


def test_worklist_is_sorted_permutation():
    cu = [0, 17, 300, 300, 1500, 1600]
    items = worklist.fwd_items(cu, 3, 128, 64)
    costs = [it[3] for it in items]
    assert costs == sorted(costs, reverse=True)
    keys = {(d, t, h) for d, t, h, _ in items}
    assert len(keys) == len(items) == 3 * (1 + 3 + 0 + 10 + 1)
    b = worklist.bwd_items(cu, 3, 64, 128)
    assert len(b) == 3 * (1 + 3 + 0 + 10 + 1)
    assert len({(d, t, h) for d, t, h, _ in b}) == len(b)
    # backward: the pages' order too -- cost descending, then document, tile, head
    bc = [c for _, _, _, c in b]
    assert bc == sorted(bc, reverse=True)
    assert b == sorted(b, key=lambda it: (-it[3], it[0], it[1], it[2]))


def test_backward_list_interleaves_documents_by_cost():
    """Cost descending across documents: the cheap last tile of a long
    document comes after the costliest tile of a shorter one (a document-
    grouped order would fail this)."""
    cu = [0, 1024, 1024 + 300]          # 8 key tiles (16 query tiles) and 3 key tiles (5 query tiles)
    b = [(d, t) for d, t, h, c in worklist.bwd_items(cu, 1, 64, 128)]
    assert b.index((1, 0)) < b.index((0, 7))
    assert b[:2] == [(0, 0), (0, 1)]
    assert [c for *_, c in worklist.bwd_items(cu, 1, 64, 128)] == [16, 14, 12, 10, 8, 6, 5, 4, 3, 2, 1]


def test_skew_rule():
    assert worklist.is_skewed([0, 8192] + [8192 + 256 * (i + 1) for i in range(224)])
    assert not worklist.is_skewed([0, 4096, 8192])


def test_nvfp4_round_up_scale_and_exact_dequant():
    wl = W.small_packed(12, [40], heads=2, head_dim=64)
    x = wl.q.float().numpy()
    codes, scales, t, deq = nvfp4.quantize_nvfp4(x)
    assert t == np.float32(np.max(np.abs(x))) / np.float32(2688.0)
    g = x.reshape(40, 2, 4, 16)
    gmax = np.abs(g).max(-1)
    # the scale is an E4M3 value, never below what the group needs, and the
    # next smaller E4M3 value would be below it (round-up, tight)
    need = (gmax.astype(np.float64) / np.float64(np.float32(6 * np.float64(t)))).astype(np.float32)
    assert np.all(scales >= need)
    np.testing.assert_array_equal(formats.e4m3_round(scales), scales)
    vals = np.unique(formats.e4m3_decode(np.arange(0x7F, dtype=np.uint8)))
    for s, n in zip(scales.ravel()[:50], need.ravel()[:50]):
        below = vals[vals < s]
        assert below.size == 0 or below.max() < n
    # dequantized = code value * s * t, and |x / (s t)| <= 6 (no clamp needed)
    assert np.all(np.abs(x / (scales[..., None].repeat(16, -1).reshape(40, 2, 64) * t)) <= 6.0 + 1e-6)
    # every code*scale product is an fp16-exact number (the GPU expands NVFP4
    # into fp16 exactly): at most 6 significant bits
    prod = formats.e2m1_decode(codes) * np.repeat(scales, 16, axis=-1)
    np.testing.assert_array_equal(formats.fp16_round(prod), prod)
    np.testing.assert_allclose(deq, prod * np.float64(t))


def test_nvfp4_slice_with_tensor_amax_equals_slice_of_tensor():
    """Groups are per token: quantizing a block of rows with the whole
    tensor's max-abs reproduces those rows of the whole-tensor quantization
    (what the full-size sampled parity checks rely on)."""
    rng = np.random.default_rng(7)
    x = rng.standard_normal((96, 3, 64)).astype(np.float32)
    x[40, 1, 5] = 37.0                          # the tensor maximum lies outside the slice
    full = nvfp4.quantize_nvfp4(x)
    sl = slice(50, 90)
    part = nvfp4.quantize_nvfp4(x[sl, 1:], amax=np.max(np.abs(x)))
    assert part[2] == full[2]
    np.testing.assert_array_equal(part[0], full[0][sl, 1:])
    np.testing.assert_array_equal(part[1], full[1][sl, 1:])
    # without the tensor amax the slice gets its own (different) tensor scale
    assert nvfp4.quantize_nvfp4(x[sl, 1:])[2] != full[2]
