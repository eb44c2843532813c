"""Pins of the decision bounds (oracle/decisions.py) against brute-force
emulation of admissible evaluations, on the CPU.

* Scores evaluated in fp32 in random orders (sequential sums of the exact
  products) and scores moved anywhere inside the stated bound: every E4M3
  code of P 2^8 that changes stays inside the stated span, the resulting bf16
  O stays inside the O allowance, and D moves by at most e(D).
* The dQ row under a shift of D: at zero shift it is the oracle's row bit for
  bit; under the shift a change of the stored O produces, it is the row the
  oracle's own backward computes from that O; and every payload a dense scan
  of shifts reaches is reached at one of the listed shifts.
* The near-tie behind one GPU-observed P^ difference is flagged.
"""

import numpy as np
import pytest

from oracle import attention as A
from oracle import decisions as DC
from oracle import formats, quant
from precision_causal_attention_hadamard_amd import workloads as W


def doc_head(wl, doc, h, exact=False):
    """Quantized operands, forward record and allowances of one (document, head)."""
    q, k, v, do = [t.float().numpy().astype(np.float64) for t in (wl.q, wl.k, wl.v, wl.do)]
    num = A.Numerics(hadamard=wl.hadamard, exact=exact)
    s32, c32 = A.scale_constants(wl.head_dim, None)
    gran = "token" if exact else "block"
    qt = quant.quantize_qkv(q, k, v, wl.cu_seqlens, wl.hadamard, granularity=gran)
    _, _, dod = quant.quantize_token_blocks(do, wl.cu_seqlens, granularity=gran)
    hk = h // (wl.heads // wl.kv_heads)
    s, e = wl.cu_seqlens[doc], wl.cu_seqlens[doc + 1]
    ops = dict(q=qt["q"][s:e, h], k=qt["k"][s:e, hk], v=qt["v"][s:e, hk], vk=qt["v_key"][s:e, hk],
               vx=qt["v_exp"][hk, s:e], vkx=qt["v_key_exp"][hk, s:e], do=dod[s:e, h])
    fw = A.forward_doc(ops["q"], ops["k"], ops["v"], ops["vk"], ops["vx"], ops["vkx"], c32, num)
    fw["v_exp_key"] = ops["vkx"]
    if exact:
        fw["q_exp_tok"], fw["k_exp_tok"] = qt["q_exp"][h, s:e], qt["k_exp"][hk, s:e]
    al = DC.doc_head_allowances(fw, ops["q"], ops["k"], ops["v"], ops["vk"], ops["do"], num, c32)
    return ops, fw, al, num, s32, c32


def peff_from_scores(S, fw, ops, c32, rng):
    """The forward's decisions on a given fp32 score matrix, with the exp2
    evaluated to within 4 ulp."""
    L = S.shape[0]
    valid, diag = fw["valid"], fw["diag"]
    sp = formats.fp32_round(S * float(c32))
    m = fw["m"]
    p = np.where(valid, np.exp2(np.where(valid, sp - m[:, None], 0.0)), 0.0)
    p = p * (1 + rng.uniform(-4, 4, p.shape) * DC.U)
    l = p.sum(axis=1) * (1 + rng.uniform(-1, 1, L) * DC.gamma(L))
    if np.array_equal(diag, valid):      # exact option: the all-tile fold (pinned by test_oracle_exact)
        f = fw["fold"]
    else:
        e_ref = quant.fold_reference(ops["vkx"], True)
        f = np.where(diag, np.ldexp(1.0, np.minimum(ops["vkx"][None, :] - e_ref[:, None], 0)), 1.0)
    pe = np.where(diag, np.ldexp(formats.e4m3_round(np.ldexp(p * f, 8)), -8) / f,
                  np.ldexp(formats.e4m3_round(np.ldexp(p, 8)), -8))
    pe = np.where(valid, pe, 0.0)
    o = (np.where(diag, 0.0, pe) @ ops["v"] + np.where(diag, pe, 0.0) @ ops["vk"]) / l[:, None]
    return pe, o


def random_order_fp32_scores(qd, kd, rng):
    """S in fp32: the d exact products added one by one in a random order."""
    terms = qd[:, None, :] * kd[None, :, :]
    acc = np.zeros(terms.shape[:2], np.float32)
    for c in rng.permutation(qd.shape[1]):
        acc = (acc + terms[:, :, c].astype(np.float32)).astype(np.float32)
    return acc.astype(np.float64)


CASES = {
    "outliers_hadamard_d128": lambda: W.small_packed(42, [300, 211], heads=6, head_dim=128,
                                                     outlier_scale=20.0, hadamard=True, kv_heads=2),
    "plain_d64": lambda: W.small_packed(7, [150], heads=2, head_dim=64),
}


@pytest.mark.parametrize("exact", [False, True], ids=["default", "exact"])
@pytest.mark.parametrize("case", list(CASES))
def test_admissible_scores_stay_inside_the_bounds(case, exact):
    wl = CASES[case]()
    doc, h = (1, 3) if case.startswith("outliers") else (0, 1)
    ops, fw, al, num, s32, c32 = doc_head(wl, doc, h, exact)
    rng = np.random.default_rng(5)
    S0 = ops["q"] @ ops["k"].T
    e_s = DC.gamma(wl.head_dim) * (np.abs(ops["q"]) @ np.abs(ops["k"]).T) + DC.U * np.abs(S0)
    o_ref = formats.bf16_round(fw["o"])
    D_ref = np.sum(ops["do"] * o_ref, axis=1)
    changed = 0
    for trial in range(6):
        if trial < 2:
            S = random_order_fp32_scores(ops["q"], ops["k"], rng)
        else:   # anywhere inside the bound, extremes half of the time
            u = rng.uniform(-1, 1, S0.shape)
            if trial % 2:
                u = np.sign(u)
            S = S0 + u * e_s
        assert np.all(np.abs(S - S0) <= e_s * (1 + 1e-9))
        pe, o = peff_from_scores(S, fw, ops, c32, rng)
        dpe = np.abs(pe - fw["peff"])
        assert np.all(dpe <= al["p_span"] * (1 + 1e-12)), float((dpe - al["p_span"]).max())
        changed += int(np.count_nonzero(dpe))
        ob = formats.bf16_round(o)
        assert np.all(np.abs(ob - o_ref) <= al["o"] * (1 + 1e-12)), float((np.abs(ob - o_ref) - al["o"]).max())
        dD = np.abs(np.sum(ops["do"] * ob, axis=1) - D_ref)
        assert np.all(dD <= al["e_D"] * (1 + 1e-12) + 1e-12)
    if case.startswith("outliers"):
        assert changed > 0          # the bound is exercised, not vacuous


def test_the_observed_near_ties_are_flagged():
    """A decision behind a GPU difference of a grouped-head workload: a
    probability with P 2^8 = 136.0002, 1.7e-6 above the E4M3 rounding
    boundary 136 between the codes 128 and 144; the fp32 bound admits both."""
    wl = W.small_packed(43, [129, 64, 31, 250], heads=4, head_dim=128, kv_heads=1)
    ops, fw, al, *_ = doc_head(wl, 0, 1)
    x = fw["p"][73, 35] * 256
    assert 136.0 < x < 136.001
    assert al["p_span"][73, 35] == pytest.approx(16 / 256)
    assert al["o"][73].max() > 0


def dq_evaluator(wl, doc, h, exact=False):
    ops, fw, al, num, s32, c32 = doc_head(wl, doc, h, exact)
    o_out = formats.bf16_round(fw["o"])
    kexp = None
    if exact:
        kexp = fw["k_exp_tok"]
    ev = DC.DqUnderDShift(fw, ops["k"], ops["v"], ops["vk"], ops["do"], o_out, s32, num, kexp)
    return ops, fw, al, num, s32, ev, o_out


def oracle_dq(fw, ops, o_in, s32, num):
    bw = A.backward_doc(fw, ops["q"], ops["k"], ops["v"], ops["vk"], ops["do"], o_in, s32, num)
    dq = bw["dq"]
    if num.hadamard:
        from oracle.hadamard import rotate_back_fp64
        dq = rotate_back_fp64(dq)
    return formats.bf16_round(dq)


@pytest.mark.parametrize("exact", [False, True], ids=["default", "exact"])
@pytest.mark.parametrize("case", list(CASES))
def test_dq_row_at_zero_shift_is_the_oracle_row(case, exact):
    wl = CASES[case]()
    doc, h = (1, 3) if case.startswith("outliers") else (0, 1)
    ops, fw, al, num, s32, ev, o_out = dq_evaluator(wl, doc, h, exact)
    want = oracle_dq(fw, ops, o_out, s32, num)
    for i in range(0, want.shape[0], 7):
        np.testing.assert_array_equal(ev.row(i, 0.0), want[i], err_msg=f"row {i}")


@pytest.mark.parametrize("exact", [False, True], ids=["default", "exact"])
def test_dq_row_under_shift_is_the_backward_of_the_shifted_o(exact):
    """Change one element of the stored O in one row per 32-row block (so no
    two changed rows share a dS block): the oracle's backward from that O
    gives, row by row, exactly the evaluator's row at the D shift the change
    makes."""
    wl = CASES["outliers_hadamard_d128"]()
    ops, fw, al, num, s32, ev, o_out = dq_evaluator(wl, 1, 3, exact)
    rng = np.random.default_rng(13)
    L = o_out.shape[0]
    rows = [b + int(rng.integers(0, min(32, L - b))) for b in range(0, L, 32)]
    o1 = o_out.copy()
    shift = {}
    for i in rows:
        ch = int(rng.integers(0, o_out.shape[1]))
        step = np.ldexp(1.0, int(np.floor(np.log2(abs(o_out[i, ch]) + 1e-30))) - 7) * float(rng.choice([-3, -1, 1, 3]))
        o1[i, ch] = o_out[i, ch] + step
        shift[i] = float(np.sum(ops["do"][i] * o1[i]) - np.sum(ops["do"][i] * o_out[i]))
    want = oracle_dq(fw, ops, o1, s32, num)
    moved = 0
    for i in rows:
        got = ev.row(i, shift[i])
        np.testing.assert_array_equal(got, want[i], err_msg=f"row {i}")
        moved += not np.array_equal(got, ev.row(i, 0.0))
    assert moved > 0


@pytest.mark.parametrize("exact", [False, True], ids=["default", "exact"])
def test_listed_shifts_reach_every_payload_of_a_dense_scan(exact):
    wl = CASES["outliers_hadamard_d128"]()
    ops, fw, al, num, s32, ev, o_out = dq_evaluator(wl, 1, 3, exact)
    rng = np.random.default_rng(17)
    for i in rng.choice(np.arange(40, o_out.shape[0]), 6, replace=False):
        eD = max(float(al["e_D"][i]), 1e-3)
        listed = {ev.row_payload(i, a).tobytes() for a in ev.shifts(i, -eD, eD)}
        dense = {ev.row_payload(i, a).tobytes() for a in np.linspace(-eD, eD, 801)}
        assert dense <= listed, (i, len(dense - listed))
        assert len(listed) > 1
