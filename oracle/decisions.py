"""Decision bounds of the attention call (oracle; test infrastructure).

The method accumulates S = Q~ K~^T, dP = dO~ V~^T, D, the softmax
denominator l and the output products in fp32 ([Summary] opening paragraphs;
[Reading, 4.1], [Reading, 4.3]); the order of that accumulation is not fixed,
and matrix cores do not add a product's terms one by one.  Any fp32 evaluation
of a sum of n exact terms x_k is within gamma_n * sum |x_k| of the exact sum,
gamma_n = n u / (1 - n u), u = 2**-24 (the standard error bound of floating
point summation in any order: Higham, "Accuracy and Stability of Numerical
Algorithms", ch. 3 and 4).  The attention oracle evaluates every such sum
exactly and rounds once, which is one admissible result.

Where the interval of values that bound admits straddles a rounding boundary
of a quantized decision -- the E4M3 code of P 2^8 (with the diagonal fold),
the bf16 rounding of O, the E4M3 code of dS -- more than one result is
correct.  A P^ or O decision moves a row of O, and through
D_i = sum_d dO~_id O_id it shifts every dS_ij of the row in the same
direction, so dQ_i moves along a known direction; the P^ decision also
enters dV directly.  A dS^ decision moves dQ_i along K~_j and dK_j along
Q~_i by at most the code range it admits.  ``allowances`` returns these, so
a comparison can hold every element to its tolerance plus what the
alternative decisions explain (tests/decision_compare.py fits them, each
coefficient bounded).  The continuous fp32 differences are left to the
tolerance.

Bounds used (per (document, head), vectorised; e = error, rel = relative):
* S: e <= gamma_d sum_k |q~_ik k~_jk| + u |S| (the oracle rounds once);
* S' = fp32(S c) adds 2 u |S'|; P = 2^(S' - m) from a hardware exp2:
  rel <= 2^(c e_S + 2u|S'|) (1 + 4 u) - 1; the integer row maximum is taken as
  equal on both sides (a different one scales every P of the row by an exact
  power of two, which leaves O and dS unchanged outside E4M3 subnormals);
* P^: the code span of [x (1 - rel), x (1 + rel)], x = P 2^8 f;
* l = sum P: rel <= (1 + max rel(P) over the row)(1 + gamma_L) - 1;
* O (before bf16): w = (1 + rel(l)) sum_j span(P^)_ij |V_j| / l_i
  + gamma_L (|P^| |V|)_i / l_i + (rel(l) + u) |O_i|; the bf16 span of
  [O - w, O + w] is the O allowance (the rounding of O to bf16 is itself a
  decision: D is formed from the stored bf16 O);
* D: e(D_i) = sum_d |dO~_id| allowance(O)_id;
* dV_j: sum_i (1 + rel(l_i)) span(P^)_ij / l_i |dO~_i|, then the span of the
  final bf16 rounding.
A shift of D_i by delta moves dQ_i by delta times the row's direction
g_i = -s32 sum_j (P_ij / l_i) K~_j (rotated back with the Hadamard option),
before dS^ re-rounding; ``allowances`` returns g and e(D), and a comparison
fits one coefficient |a_i| <= e(D_i) per row and holds the remainder to the
tolerance.
"""

from __future__ import annotations

import numpy as np

from . import formats
from .attention import Numerics, forward_doc, scale_constants
from .quant import BLOCK, doc_bounds, fold_reference, quantize_qkv, quantize_token_blocks

U = 2.0 ** -24


def gamma(n: int) -> float:
    """gamma_n = n u / (1 - n u) for fp32 summation of n terms."""
    return n * U / (1.0 - n * U)


def _span(rounder, lo, hi):
    """Width of the set of values ``rounder`` maps [lo, hi] to (monotone)."""
    return np.abs(rounder(hi) - rounder(lo))


def _e4m3_span(lo, hi):
    return _span(formats.e4m3_round, lo, hi)


def _bf16_span(x, w):
    return _span(formats.bf16_round, x - w, x + w)


def doc_head_allowances(fw, qs, ks, qd, kd, vblk, vkey, dod, s32, c32, num: Numerics):
    """Allowances of one (document, head).  qs, ks: score operands; qd, kd:
    the dQ/dK operands; vblk, vkey, dod as for forward_doc/backward_doc.
    Returns the O allowance (after its bf16 span), e(D) per row, the dQ
    direction of a D shift (unrotated) and the dV width before its bf16
    rounding."""
    L, d = qd.shape
    valid, diag = fw["valid"], fw["diag"]
    p, l, peff = fw["p"], fw["l"], fw["peff"]
    c = float(c32)
    # scores
    S = qs @ ks.T
    e_s = gamma(d) * (np.abs(qs) @ np.abs(ks).T) + U * np.abs(S)
    sp = fw["sp"]
    w_sp = c * e_s + 2 * U * np.abs(sp)
    rel_p = np.where(valid, np.exp2(w_sp) * (1 + 4 * U) - 1.0, 0.0)
    # P^ decisions (diagonal pairs are folded, then unfolded)
    if num.quantize_p:
        f = fw["fold"]                      # the forward's fold factor of every pair (1 off the fold)
        x = np.ldexp(p * f, 8)
        span_pe = np.where(valid, np.ldexp(_e4m3_span(x * (1 - rel_p), x * (1 + rel_p)), -8) / f, 0.0)
    else:
        span_pe = rel_p * p
    rel_l = (1 + np.max(rel_p, axis=1, initial=0.0)) * (1 + gamma(L)) - 1
    # O before bf16
    av_off, av_dia = np.abs(vblk), np.abs(vkey)
    flips = (np.where(diag, 0.0, span_pe) @ av_off + np.where(diag, span_pe, 0.0) @ av_dia) / l[:, None]
    acc = (np.where(diag, 0.0, np.abs(peff)) @ av_off + np.where(diag, np.abs(peff), 0.0) @ av_dia) / l[:, None]
    o = fw["o"]
    w_o = flips * (1 + rel_l[:, None]) + gamma(L) * acc + (rel_l[:, None] + U) * np.abs(o)
    o_span = _bf16_span(o, w_o) if num.round_outputs else w_o
    # backward: the decisions above shift D, hence every dS of the row
    e_D = np.sum(np.abs(dod) * o_span, axis=1)
    g = -float(s32) * (np.where(valid, p / l[:, None], 0.0) @ kd)
    dv = ((span_pe * (1 + rel_l[:, None])) / l[:, None]).T @ np.abs(dod)
    res = dict(o=o_span, e_D=e_D, dq_dir=g, dv=dv, p_span=span_pe, rel_p=rel_p, rel_l=rel_l)
    if num.quantize_ds:
        res.update(_ds_decisions(fw, dod, vblk, vkey, rel_p, rel_l, num))
    return res


def _ds_decisions(fw, dod, vblk, vkey, rel_p, rel_l, num: Numerics):
    """dS^ codes that admissible evaluations may round either way.

    dS = fp32(fp32(P 2^8 2^-8/l) (dP - D)) with dP - D accumulated in fp32 from
    -D: e(dP - D) <= gamma_(d+1) (|D| + sum |dO~ V|) + gamma_d sum |dO~ O|
    (the D shift the O decisions allow is fitted as one coherent direction
    and not spread over every code of the row again); with
    g = (1 + rel(P))(1 + rel(l)), e(dS) <= |dS| (g (1 + 3u) - 1) + g P/l
    e(dP - D).  An element whose interval [dS - e, dS + e], scaled by its
    block's exponent, holds an E4M3 rounding boundary is returned with the
    range of dS^ values the interval maps to (relative to the oracle's
    dS^).  The block exponent itself is counted as ambiguous when the block
    max-abs interval straddles a power of two (reported, not spanned)."""
    L, d = dod.shape
    p, l, valid, diag = fw["p"], fw["l"], fw["valid"], fw["diag"]
    o_out = formats.bf16_round(fw["o"]) if num.round_outputs else fw["o"]
    D = np.sum(dod * o_out, axis=1)
    dp = np.where(diag, dod @ vkey.T, dod @ vblk.T)
    dp_abs = np.where(diag, np.abs(dod) @ np.abs(vkey).T, np.abs(dod) @ np.abs(vblk).T)
    ds = np.where(valid, (p / l[:, None]) * (dp - D[:, None]), 0.0)
    e_dpd = (gamma(d + 1) * (np.abs(D)[:, None] + dp_abs)
             + gamma(d) * np.sum(np.abs(dod * o_out), axis=1)[:, None])
    grow = (1 + rel_p) * (1 + rel_l[:, None])
    e_ds = np.where(valid, np.abs(ds) * (grow * (1 + 3 * U) - 1) + (p / l[:, None]) * grow * e_dpd, 0.0)
    payloads = {"q": (None, True), "k": (None, False)}
    if num.exact:
        payloads = {"q": (fw["k_exp_tok"], True), "k": (fw["q_exp_tok"], False)}
    res = {}
    blocks_ambiguous = 0
    for name, (e_fold, by_rows) in payloads.items():
        if not num.exact and name == "k":
            res["k"] = res["q"]             # one payload serves both products
            continue
        sc = np.ones(L) if e_fold is None else np.ldexp(1.0, np.asarray(e_fold, dtype=np.int64))
        fold = sc[None, :] if by_rows else sc[:, None]
        xs, es = ds * fold, e_ds * fold
        if num.exact and not by_rows:
            xs, es, vt = xs.T, es.T, valid.T
        else:
            vt = valid
        rows, cols, lo, hi = [], [], [], []
        # groups: 32 x 32 blocks (default), or one row x 32 along the contraction axis (exact)
        gr = 1 if num.exact else BLOCK
        for i0 in range(0, L, gr):
            for j0 in range(0, L, BLOCK):
                v = vt[i0:i0 + gr, j0:j0 + BLOCK]
                if not v.any():
                    continue
                x = np.where(v, xs[i0:i0 + gr, j0:j0 + BLOCK], 0.0)
                ex = np.where(v, es[i0:i0 + gr, j0:j0 + BLOCK], 0.0)
                amax, emax = np.abs(x).max(), ex.max()
                eb = formats.roundup_exponent(amax)
                if formats.roundup_exponent(max(amax - emax, 0.0)) != formats.roundup_exponent(amax + emax):
                    blocks_ambiguous += 1
                q0 = np.ldexp(formats.e4m3_round(np.ldexp(x, -eb)), eb)
                ql = np.ldexp(formats.e4m3_round(np.ldexp(x - ex, -eb), saturate=True), eb)
                qh = np.ldexp(formats.e4m3_round(np.ldexp(x + ex, -eb), saturate=True), eb)
                gi, gj = np.nonzero(v & (ql != qh))
                dlo, dhi = (ql - q0)[gi, gj], (qh - q0)[gi, gj]
                ti, tj = gi + i0, gj + j0
                i_, j_ = (tj, ti) if (num.exact and not by_rows) else (ti, tj)
                fl = sc[j_] if by_rows else sc[i_]     # remove the fold: deltas of the unfolded dS
                rows.append(i_)
                cols.append(j_)
                lo.append(dlo / fl)
                hi.append(dhi / fl)
        res[name] = (rows, cols, lo, hi)
    cat = (lambda a, t: np.concatenate(a).astype(t) if a else np.zeros(0, t))
    out = {"ds_blocks_ambiguous": blocks_ambiguous}
    for name, (rows, cols, lo, hi) in res.items():
        out[f"ds{name}_rows"], out[f"ds{name}_cols"] = cat(rows, np.int64), cat(cols, np.int64)
        out[f"ds{name}_lo"], out[f"ds{name}_hi"] = cat(lo, np.float64), cat(hi, np.float64)
    return out


def allowances(q, k, v, do, cu_seqlens, num: Numerics | None = None):
    """Decision bounds of the whole call (see the module docstring): ``o``
    ``[T, H, d]`` and ``dv`` ``[T, Hk, d]`` per-element allowances; ``e_D``
    ``[T, H]``, the bound of the admissible shift of D per query row;
    ``dq_dir`` ``[T, H, d]``, the change of dQ per unit shift of D; and
    ``ds_q`` / ``ds_k``, the codes of the dS^ payload of dQ / of dK that
    admissible evaluations may round either way (one payload serves both
    unless the exact option is on): query token ``tq`` and head ``h``, key
    token ``tk`` and key/value head ``hk``, the range [lo, hi] of the change
    of the effective dS value, and ``vec``, the change of the dQ row (of the
    dK row) per unit change of it."""
    num = num or Numerics()
    q = np.asarray(q, dtype=np.float64)
    T, H, d = q.shape
    Hk = np.asarray(k).shape[1]
    group = H // Hk
    s32, c32 = scale_constants(d, num.softmax_scale)
    gran = "token" if num.exact else num.granularity
    qt = quantize_qkv(q, k, v, cu_seqlens, num.hadamard, num.rule, gran)
    _, _, do_deq = quantize_token_blocks(do, cu_seqlens, num.rule, gran)
    qs_all, ks_all = qt["q"], qt["k"]
    if num.path == "mixed":
        from .nvfp4 import quantize_nvfp4
        qa, ka = num.nvfp4_amax if num.nvfp4_amax is not None else (None, None)
        *_, qs_all = quantize_nvfp4(qt["q_rot"], qa)
        *_, ks_all = quantize_nvfp4(qt["k_rot"], ka)
    from .hadamard import rotate_back_fp64
    out = dict(o=np.zeros((T, H, d)), dq_dir=np.zeros((T, H, d)), e_D=np.zeros((T, H)))
    amb = {n_: {k_: [] for k_ in ("tq", "h", "tk", "hk", "lo", "hi", "vec")} for n_ in ("q", "k")}
    blocks_ambiguous = 0
    dv_w = np.zeros((T, Hk, d))
    dv_raw = np.zeros((T, Hk, d))
    for s, e in doc_bounds(cu_seqlens):
        if e == s:
            continue
        sl = slice(s, e)
        for h in range(H):
            hk = h // group
            fw = forward_doc(qs_all[sl, h], ks_all[sl, hk], qt["v"][sl, hk], qt["v_key"][sl, hk],
                             qt["v_exp"][hk, sl], qt["v_key_exp"][hk, sl], c32, num)
            fw["v_exp_key"] = qt["v_key_exp"][hk, sl]
            if num.exact:
                fw["q_exp_tok"], fw["k_exp_tok"] = qt["q_exp"][h, sl], qt["k_exp"][hk, sl]
            a = doc_head_allowances(fw, qs_all[sl, h], ks_all[sl, hk], qt["q"][sl, h], qt["k"][sl, hk],
                                    qt["v"][sl, hk], qt["v_key"][sl, hk], do_deq[sl, h], s32, c32, num)
            out["o"][sl, h] = a["o"]
            out["e_D"][sl, h] = a["e_D"]
            out["dq_dir"][sl, h] = rotate_back_fp64(a["dq_dir"]) if num.hadamard else a["dq_dir"]
            dv_w[sl, hk] += a["dv"]
            dv_raw[sl, hk] += (fw["peff"] / fw["l"][:, None]).T @ do_deq[sl, h]
            if "dsq_rows" in a:
                for name, vec_src, vec_idx in (("q", qt["k"][sl, hk], "cols"), ("k", qt["q"][sl, h], "rows")):
                    r, cidx = a[f"ds{name}_rows"], a[f"ds{name}_cols"]
                    vecs = vec_src[cidx if vec_idx == "cols" else r]
                    if num.hadamard:
                        vecs = rotate_back_fp64(vecs)
                    e_ = amb[name]
                    e_["tq"].append(r + s)
                    e_["h"].append(np.full(len(r), h))
                    e_["tk"].append(cidx + s)
                    e_["hk"].append(np.full(len(r), hk))
                    e_["lo"].append(a[f"ds{name}_lo"])
                    e_["hi"].append(a[f"ds{name}_hi"])
                    e_["vec"].append(float(s32) * vecs)
                blocks_ambiguous += a["ds_blocks_ambiguous"]
    out["dv"] = _bf16_span(dv_raw, dv_w) if num.round_outputs else dv_w
    for n_ in ("q", "k"):
        out[f"ds_{n_}"] = {k_: (np.concatenate(v_) if v_ else np.zeros((0, d) if k_ == "vec" else 0))
                           for k_, v_ in amb[n_].items()}
    out["ds_blocks_ambiguous"] = blocks_ambiguous
    return out
