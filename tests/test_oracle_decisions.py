"""Pins of the decision bounds (oracle/decisions.py) against brute-force
emulation of admissible evaluations, on the CPU.

* Scores evaluated in fp32 in random orders (sequential sums of the exact
  products) and scores moved anywhere inside the stated bound: every E4M3
  code of P 2^8 that changes stays inside the stated span, the resulting bf16
  O stays inside the O allowance, and D moves by at most e(D).
* A shift of the stored O moves the oracle's own (unquantized-dS) dQ exactly
  along the stated direction, by the shift of D.
* dS evaluated from admissible P, l, dP and D: every dS^ code that changes is
  a listed decision and moves inside its listed range (blocks whose exponent
  the bound leaves open are excluded and counted).
* The near-tie behind one GPU-observed difference is flagged.
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
    al = DC.doc_head_allowances(fw, ops["q"], ops["k"], ops["q"], ops["k"], ops["v"], ops["vk"], ops["do"],
                                s32, c32, num)
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


def test_dq_moves_along_the_stated_direction_under_a_shift_of_o():
    wl = CASES["outliers_hadamard_d128"]()
    ops, fw, al, num, s32, c32 = doc_head(wl, 0, 4)
    rng = np.random.default_rng(9)
    num_c = A.Numerics(hadamard=True, quantize_ds=False)
    o0 = formats.bf16_round(fw["o"])
    rows = rng.choice(o0.shape[0], 5, replace=False)
    o1 = o0.copy()
    for i in rows:
        ch = rng.choice(o0.shape[1], 3, replace=False)
        o1[i, ch] += rng.choice([-1, 1], 3) * np.ldexp(1.0, np.floor(np.log2(np.abs(o0[i, ch]) + 1e-30)).astype(int) - 7)
    args = (ops["q"], ops["k"], ops["v"], ops["vk"], ops["do"])
    b0 = A.backward_doc(fw, *args, o0, s32, num_c)
    b1 = A.backward_doc(fw, *args, o1, s32, num_c)
    dD = np.sum(ops["do"] * (o1 - o0), axis=1)
    want = dD[:, None] * al["dq_dir"]
    np.testing.assert_allclose(b1["dq"] - b0["dq"], want, rtol=1e-9, atol=1e-12 * np.abs(b0["dq"]).max())
    assert np.count_nonzero(np.abs(b1["dq"] - b0["dq"]).max(axis=1) > 0) == len(rows)


@pytest.mark.parametrize("exact", [False, True], ids=["default", "exact"])
@pytest.mark.parametrize("case", list(CASES))
def test_admissible_ds_codes_are_listed_decisions(case, exact):
    wl = CASES[case]()
    doc, h = (1, 3) if case.startswith("outliers") else (0, 1)
    ops, fw, al, num, s32, c32 = doc_head(wl, doc, h, exact)
    rng = np.random.default_rng(11)
    L, d = ops["q"].shape
    valid, diag, p, l = fw["valid"], fw["diag"], fw["p"], fw["l"]
    o_out = formats.bf16_round(fw["o"])
    ref = A.backward_doc(fw, ops["q"], ops["k"], ops["v"], ops["vk"], ops["do"], o_out, s32, num)
    D = np.sum(ops["do"] * o_out, axis=1)
    if exact:       # every pair uses the per-key V codes (the forward's diag covers all visible pairs)
        assert np.array_equal(diag, valid)
    dp = np.where(diag, ops["do"] @ ops["vk"].T, ops["do"] @ ops["v"].T)
    dp_abs = np.where(diag, np.abs(ops["do"]) @ np.abs(ops["vk"]).T, np.abs(ops["do"]) @ np.abs(ops["v"]).T)
    listed = {n_: {(int(r), int(c_)): (lo, hi) for r, c_, lo, hi in
                   zip(al[f"ds{n_}_rows"], al[f"ds{n_}_cols"], al[f"ds{n_}_lo"], al[f"ds{n_}_hi"])}
              for n_ in ("q", "k")}
    changed = 0
    for trial in range(6):
        sgn = (lambda shape: np.sign(rng.uniform(-1, 1, shape))) if trial % 2 else \
              (lambda shape: rng.uniform(-1, 1, shape))
        p_a = p * (1 + sgn(p.shape) * al["rel_p"])
        l_a = l * (1 + sgn(l.shape) * al["rel_l"])
        e_dpd = DC.gamma(d + 1) * (np.abs(D)[:, None] + dp_abs) + \
            DC.gamma(d) * np.sum(np.abs(ops["do"] * o_out), axis=1)[:, None]
        dpd = dp - D[:, None] + sgn(dp.shape) * e_dpd
        ds = np.where(valid, (p_a / l_a[:, None]) * dpd * (1 + sgn(dp.shape) * 3 * DC.U), 0.0)
        for n_, ref_q in (("q", ref["dsq"]), ("k", ref["dsq_k"])):
            if exact:
                e_fold = fw["k_exp_tok"] if n_ == "q" else fw["q_exp_tok"]
                dsq = A._ds_exact(ds, valid, e_fold, n_ == "q", "roundup")
                fold = np.ldexp(1.0, e_fold)[None, :] if n_ == "q" else np.ldexp(1.0, e_fold)[:, None]
                g0, g1 = (1, 32) if n_ == "q" else (32, 1)
            else:
                dsq = A._ds_quantize(ds, valid, "roundup")
                fold, (g0, g1) = 1.0, (32, 32)
            # groups whose exponent moved are outside what the list covers
            same_exp = np.ones_like(valid)
            for i0 in range(0, L, g0):
                for j0 in range(0, L, g1):
                    v = valid[i0:i0 + g0, j0:j0 + g1]
                    if v.any():
                        a0 = np.abs(np.where(v, (ref["ds"] * fold)[i0:i0 + g0, j0:j0 + g1], 0)).max()
                        a1 = np.abs(np.where(v, (ds * fold)[i0:i0 + g0, j0:j0 + g1], 0)).max()
                        same_exp[i0:i0 + g0, j0:j0 + g1] = formats.roundup_exponent(a0) == formats.roundup_exponent(a1)
            delta = dsq - ref_q
            ii, jj = np.nonzero((delta != 0) & same_exp)
            for i, j in zip(ii, jj):
                assert (i, j) in listed[n_], (n_, trial, i, j, ds[i, j], ref["ds"][i, j])
                lo, hi = listed[n_][(i, j)]
                assert lo * (1 + 1e-12) - 1e-300 <= delta[i, j] <= hi * (1 + 1e-12) + 1e-300
            changed += len(ii)
    assert changed > 0


def test_the_observed_near_ties_are_flagged():
    """Two decisions behind GPU differences of grouped-head workloads: a
    probability with P 2^8 = 136.0002, 1.7e-6 above the E4M3 rounding
    boundary 136 between the codes 128 and 144, and a dS scaled by its block
    exponent to 84.00003, 3.4e-7 above the boundary 84 between 80 and 88; the
    fp32 bound admits both codes of each."""
    wl = W.small_packed(43, [129, 64, 31, 250], heads=4, head_dim=128, kv_heads=1)
    ops, fw, al, *_ = doc_head(wl, 0, 1)
    x = fw["p"][73, 35] * 256
    assert 136.0 < x < 136.001
    assert al["p_span"][73, 35] == pytest.approx(16 / 256)
    assert al["o"][73].max() > 0
    wl2 = W.small_packed(41, [1, 17, 45, 100, 33, 64, 130, 2], heads=4, head_dim=64, kv_heads=2)
    ops2, fw2, al2, *_ = doc_head(wl2, 6, 1)
    k_ = [n for n, (r, c_) in enumerate(zip(al2["dsq_rows"], al2["dsq_cols"])) if (r, c_) == (30, 20)]
    assert len(k_) == 1
    assert (al2["dsq_lo"][k_[0]], al2["dsq_hi"][k_[0]]) == (-8 * 2.0 ** -6, 0.0)
