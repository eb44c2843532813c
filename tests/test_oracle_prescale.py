"""Pins of the oracle's dQ accumulator prescale sigma ([Reading, 4.4] third
bullet; the optional causal dQ scale of the [Summary] bullets): a hand
example, the fp16 range it is chosen for (every partial sum of dQ scaled by
2^-sigma stays below 2^15, also on an adversarial input at the bound), and
causality of the causal variant."""

import numpy as np
import pytest

from oracle import attention as A
from oracle import formats
from oracle.quant import quantize_qkv, quantize_token_blocks
from precision_causal_attention_hadamard_amd import workloads as W


def test_hand_example():
    # one document of 70 tokens (blocks of 32, 32, 6), one head, d = 64
    do_exp = np.array([[-3] * 32 + [-5] * 32 + [-1] * 6])
    k_exp = np.array([[2] * 32 + [7] * 32 + [4] * 6])
    v_exp = np.array([[-2] * 32 + [-6] * 32 + [0] * 6])
    got = A.dq_prescale(do_exp, k_exp, v_exp, [0, 70], 64)
    # document maxima: E_K = 7, E_V = 0; log2 d = 6
    np.testing.assert_array_equal(got[0], do_exp[0] + 7 + 0 + 6 + 13)
    got_c = A.dq_prescale(do_exp, k_exp, v_exp, [0, 70], 64, causal_dq_scale=True)
    np.testing.assert_array_equal(got_c[0, :32], -3 + 2 - 2 + 19)
    np.testing.assert_array_equal(got_c[0, 32:64], -5 + 7 - 2 + 19)
    np.testing.assert_array_equal(got_c[0, 64:], -1 + 7 + 0 + 19)
    # grouped heads: query heads 0, 1 read key/value head 0
    got_g = A.dq_prescale(np.vstack([do_exp, do_exp + 1]), k_exp, v_exp, [0, 70], 64)
    np.testing.assert_array_equal(got_g[1], got_g[0] + 1)
    # two documents: each takes its own maxima
    got_2 = A.dq_prescale(do_exp, k_exp, v_exp, [0, 40, 70], 64)
    assert got_2[0, 0] == -3 + 7 - 2 + 19 and got_2[0, 69] == -1 + 7 + 0 + 19


def partial_sums_fit_fp16(q, k, v, do, cu, hadamard, causal_dq_scale=False, exact=False):
    """Every prefix (over key tiles of 128) of sum_j dS~_ij K~_j times
    2^-sigma_i is below 2^15 in magnitude."""
    num = A.Numerics(hadamard=hadamard, exact=exact)
    gran = "token" if exact else "block"
    qt = quantize_qkv(q, k, v, cu, hadamard, granularity=gran)
    _, do_exp, dod = quantize_token_blocks(do, cu, granularity=gran)
    d = q.shape[2]
    sig = A.dq_prescale(do_exp, qt["k_exp"], qt["v_exp"], cu, d, causal_dq_scale, exact)
    s32, c32 = A.scale_constants(d, None)
    worst = -np.inf
    for s, e in zip(cu[:-1], cu[1:]):
        for h in range(q.shape[1]):
            fw = A.forward_doc(qt["q"][s:e, h], qt["k"][s:e, h], qt["v"][s:e, h], qt["v_key"][s:e, h],
                               qt["v_exp"][h, s:e], qt["v_key_exp"][h, s:e], c32, num)
            if exact:
                fw["q_exp_tok"], fw["k_exp_tok"] = qt["q_exp"][h, s:e], qt["k_exp"][h, s:e]
            bw = A.backward_doc(fw, qt["q"][s:e, h], qt["k"][s:e, h], qt["v"][s:e, h], qt["v_key"][s:e, h],
                                dod[s:e, h], formats.bf16_round(fw["o"]), s32, num)
            L = e - s
            for u0 in range(0, L, 128):
                part = bw["dsq"][:, :u0 + 128] @ qt["k"][s:s + min(L, u0 + 128), h]
                worst = max(worst, float(np.max(np.abs(part) * np.ldexp(1.0, -sig[h, s:e])[:, None])))
    return worst


@pytest.mark.parametrize("causal_dq_scale", [False, True])
def test_partial_sums_stay_in_fp16_range(causal_dq_scale):
    wl = W.small_packed(61, [300, 70], heads=2, head_dim=128, outlier_scale=20.0, hadamard=True)
    q, k, v, do = [t.float().numpy().astype(np.float64) for t in (wl.q, wl.k, wl.v, wl.do)]
    worst = partial_sums_fit_fp16(q, k, v, do, wl.cu_seqlens, True, causal_dq_scale)
    assert 0 < worst < 2.0 ** 15
    assert worst > 2.0 ** -10           # and not wastefully far below it


def test_partial_sums_at_the_adversarial_bound():
    """All codes at the largest magnitude with aligned signs: the bound is
    approached, not exceeded."""
    L, d = 96, 64
    rng = np.random.default_rng(3)
    sgn = np.sign(rng.standard_normal(d))
    q = np.zeros((L, 1, d))
    k = np.ones((L, 1, d)) * sgn
    v = np.tile(np.where(np.arange(L) % 2, 1.0, -1.0)[:, None, None], (1, 1, d)) * sgn
    do = np.ones((L, 1, d)) * sgn
    worst = partial_sums_fit_fp16(q, k, v, do, [0, L], False)
    assert worst < 2.0 ** 15


def test_exact_option_prescale_is_per_token_prefix():
    L = 40
    do_exp = np.zeros((1, L), np.int64)
    k_exp = np.arange(L)[None, :] % 7
    v_exp = -(np.arange(L)[None, :] % 5)
    got = A.dq_prescale(do_exp, k_exp, v_exp, [0, L], 128, exact=True)
    want = np.maximum.accumulate(k_exp[0]) + np.maximum.accumulate(v_exp[0]) + 7 + 13
    np.testing.assert_array_equal(got[0], want)


def test_causal_prescale_ignores_later_blocks():
    wl = W.small_packed(62, [200], heads=1, head_dim=64)
    q, k, v, do = [t.float().numpy().astype(np.float64) for t in (wl.q, wl.k, wl.v, wl.do)]
    qt = quantize_qkv(q, k, v, wl.cu_seqlens)
    _, do_exp, _ = quantize_token_blocks(do, wl.cu_seqlens)
    a = A.dq_prescale(do_exp, qt["k_exp"], qt["v_exp"], wl.cu_seqlens, 64, True)
    k2, v2 = k.copy(), v.copy()
    k2[130:] *= 2.0 ** 12
    v2[130:] *= 2.0 ** 12
    qt2 = quantize_qkv(q, k2, v2, wl.cu_seqlens)
    b = A.dq_prescale(do_exp, qt2["k_exp"], qt2["v_exp"], wl.cu_seqlens, 64, True)
    np.testing.assert_array_equal(a[:, :128], b[:, :128])       # blocks 0-3 end before token 130
    assert np.all(b[:, 160:] > a[:, 160:])
    c = A.dq_prescale(do_exp, qt2["k_exp"], qt2["v_exp"], wl.cu_seqlens, 64, False)
    assert np.all(c[:, :128] > a[:, :128])                      # the default sees the whole document
