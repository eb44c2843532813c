"""Decision bounds of the attention call (oracle; test infrastructure).

The method accumulates S = Q~ K~^T, the softmax denominator l and the output
products in fp32 ([Summary] opening paragraphs; [Reading, 4.1], [Reading,
4.3]); the order of that accumulation is not fixed.  Any fp32 evaluation of a
sum of n exact terms x_k is within gamma_n * sum |x_k| of the exact sum,
gamma_n = n u / (1 - n u), u = 2**-24 (the standard bound of floating-point
summation in any order: Higham, "Accuracy and Stability of Numerical
Algorithms", ch. 3 and 4).  The attention oracle evaluates every such sum
exactly and rounds once, which is one admissible result.

Where the interval of values that bound admits straddles a rounding boundary
of a quantized decision -- the E4M3 code of P 2^8 (with the diagonal fold),
the bf16 rounding of O -- more than one result is correct.  ``allowances``
returns, per element, how far those decisions can move O and dV, and per
query row the bound e(D) of the shift they allow in D_i = sum_d dO~_id O_id
(D is formed from the stored bf16 O, [Summary, §3.3]).

A shift of D_i moves every dS_ij = P_ij / l_i (dP_ij - D_i) of row i, and the
dS^ codes of the row are re-rounded with it: a code near an E4M3 rounding
boundary can take the neighbouring value, which moves dQ_i by a whole code
step times K~_j.  ``DqUnderDShift`` evaluates the oracle's dQ row with D_i
replaced by D_i + a, everything else unchanged, and lists shifts at which the
row's codes change, so a comparison can look for an admissible shift
(|a| <= e(D_i)) that reproduces a given row.  Its list of shifts may miss
some (it considers exponents near the unshifted ones), and the other rows of
a 32 x 32 dS block are held at their unshifted values; both can only make
such a comparison stricter.

Bounds used (per (document, head), vectorised; e = error, rel = relative):
* S: e <= gamma_d sum_k |q~_ik k~_jk| + u |S| (the oracle rounds once);
* S' = fp32(S c) adds 2 u |S'|; P = 2^(S' - m) from a hardware exp2:
  rel <= 2^(c e_S + 2u|S'|) (1 + 4 u) - 1; the integer row maximum is taken as
  equal on both sides (a different one scales every P of the row by an exact
  power of two, which leaves O and dS unchanged outside E4M3 subnormals);
* P^: the code span of [x (1 - rel), x (1 + rel)], x = P 2^8 f (for the 4-bit
  operand also over the group scales the group's interval maxima allow);
* l = sum P: rel <= (1 + max rel(P) over the row)(1 + gamma_L) - 1;
* O (before bf16): w = (1 + rel(l)) sum_j span(P^)_ij |V_j| / l_i
  + gamma_L (|P^| |V|)_i / l_i + (rel(l) + u) |O_i|; the bf16 span of
  [O - w, O + w] is the O allowance;
* D: e(D_i) = sum_d |dO~_id| allowance(O)_id;
* dV_j: sum_i (1 + rel(l_i)) span(P^)_ij / l_i |dO~_i|, then the span of the
  final bf16 rounding.
The matrix cores' measured error can exceed gamma_n (their 64-term dot
products are not rounded once); a bound that is too tight only makes the
comparison stricter.
"""

from __future__ import annotations

import numpy as np

from . import formats
from .attention import Numerics, forward_doc, scale_constants
from .hadamard import rotate_back_fp64
from .quant import BLOCK, doc_bounds, quantize_qkv, quantize_token_blocks

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


def _p4_span(lo, hi, valid):
    """Width of the values the 4-bit probability operand (p4_quantize) can
    give an element whose value lies in [lo, hi] while every element of its
    group lies in its own interval: the group scale is one of the round-up
    exponents of the group's smallest and largest possible maxima, and under
    each scale the E2M1 rounding (then the E4M3 carry) is monotone."""
    from .attention import P4_GROUP, roundup_e2m1
    out = np.zeros_like(lo)
    n = lo.shape[1]
    for g0 in range(0, n, P4_GROUP):
        sl = slice(g0, min(g0 + P4_GROUP, n))
        v = valid[:, sl]
        a_lo = np.where(v, lo[:, sl], 0.0).max(axis=1)
        a_hi = np.where(v, hi[:, sl], 0.0).max(axis=1)
        qmin = np.full(lo[:, sl].shape, np.inf)
        qmax = np.full(lo[:, sl].shape, -np.inf)
        for a in (a_lo, a_hi):
            nz = a > 0
            e = np.where(nz, roundup_e2m1(np.where(nz, a, 1.0)), 0)[:, None]
            q_lo = np.where(nz[:, None], formats.e4m3_round(np.ldexp(formats.e2m1_round(np.ldexp(lo[:, sl], -e)), e)), 0.0)
            q_hi = np.where(nz[:, None], formats.e4m3_round(np.ldexp(formats.e2m1_round(np.ldexp(hi[:, sl], -e)), e)), 0.0)
            qmin = np.minimum(qmin, q_lo)
            qmax = np.maximum(qmax, q_hi)
        out[:, sl] = np.where(v, qmax - qmin, 0.0)
    return out


def doc_head_allowances(fw, qs, ks, vblk, vkey, dod, num: Numerics, c32):
    """Allowances of one (document, head).  qs, ks: score operands; vblk,
    vkey, dod as for forward_doc/backward_doc.  Returns the O allowance
    (after its bf16 span), e(D) per row, the dV width before its bf16
    rounding and the P^ span."""
    L, d = qs.shape
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
        if num.p_format == "nvfp4":
            span_pe = np.where(valid, np.ldexp(_p4_span(x * (1 - rel_p), x * (1 + rel_p), valid), -8) / f, 0.0)
        else:
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
    e_D = np.sum(np.abs(dod) * o_span, axis=1)
    dv = ((span_pe * (1 + rel_l[:, None])) / l[:, None]).T @ np.abs(dod)
    return dict(o=o_span, e_D=e_D, dv=dv, p_span=span_pe, rel_p=rel_p, rel_l=rel_l)


class DqUnderDShift:
    """dQ rows of one (document, head) when D_i is replaced by D_i + a.

    Built from the oracle's own forward record and backward operands; row
    ``i`` at shift ``a`` is the oracle's dQ_i (bf16, rotated back with the
    Hadamard option) computed with dS_ij = (P_ij / l_i)(dP_ij - (D_i + a)),
    re-quantized by the payload rule of dQ: one round-up exponent per 32 x 32
    block taken over the block's valid entries, the other 31 rows of the
    block unshifted; with the exact option, K's per-token exponent folded in
    and one exponent per (row, 32 keys)."""

    def __init__(self, fw, kd, vblk, vkey, dod, o_out, s32, num: Numerics, k_exp_tok=None):
        self.p = fw["p"].astype(np.float32)          # fp32 values, kept exactly
        self.l = fw["l"]
        self.valid = fw["valid"]
        self.dp = np.where(fw["diag"], dod @ vkey.T, dod @ vblk.T)
        self.D = np.sum(dod * o_out, axis=1)
        self.kd = kd
        self.s32 = float(s32)
        self.num = num
        self.k_exp = None if k_exp_tok is None else np.asarray(k_exp_tok, np.int64)

    def _ds_rows(self, r0, r1, shift=None):
        p = self.p[r0:r1].astype(np.float64)
        D = self.D[r0:r1] if shift is None else self.D[r0:r1] + shift
        return np.where(self.valid[r0:r1], (p / self.l[r0:r1, None]) * (self.dp[r0:r1] - D[:, None]), 0.0)

    def row_payload(self, i, a):
        """Effective dS^ values of row i (the dQ payload) at shift a."""
        ex_rule = formats.EXPONENT_RULES[self.num.rule]
        sat = self.num.rule == "floor"      # only the floor rule can overflow (the oracle clamps it)
        x = self._ds_rows(i, i + 1, np.array([a]))[0]
        v = self.valid[i]
        L = x.shape[0]
        out = np.zeros(L)
        if self.k_exp is not None:        # exact option: per (row, 32 keys), K exponent folded in
            sc = np.ldexp(1.0, self.k_exp)
            xf = x * sc
            for j0 in range(0, L, BLOCK):
                vv = v[j0:j0 + BLOCK]
                if not vv.any():
                    continue
                seg = np.where(vv, xf[j0:j0 + BLOCK], 0.0)
                e = ex_rule(np.max(np.abs(seg)))
                q = np.ldexp(formats.e4m3_decode(formats.e4m3_encode(np.ldexp(seg, -e), saturate=sat)), e)
                out[j0:j0 + BLOCK] = np.where(vv, q, 0.0) / sc[j0:j0 + BLOCK]
            return out
        b0 = i // BLOCK * BLOCK
        others = self._ds_rows(b0, min(b0 + BLOCK, L))
        others[i - b0] = 0.0
        vb = self.valid[b0:min(b0 + BLOCK, L)]
        for j0 in range(0, L, BLOCK):
            vv = v[j0:j0 + BLOCK]
            if not vv.any():
                continue
            m_other = np.max(np.abs(np.where(vb[:, j0:j0 + BLOCK], others[:, j0:j0 + BLOCK], 0.0)))
            seg = np.where(vv, x[j0:j0 + BLOCK], 0.0)
            e = ex_rule(max(m_other, np.max(np.abs(seg))))
            q = np.ldexp(formats.e4m3_decode(formats.e4m3_encode(np.ldexp(seg, -e), saturate=sat)), e)
            out[j0:j0 + BLOCK] = np.where(vv, q, 0.0)
        return out

    def row(self, i, a):
        """dQ_i at shift a, as the oracle's output (bf16 unless outputs are
        left unrounded)."""
        dq = self.s32 * (self.row_payload(i, a) @ self.kd)
        if self.num.hadamard:
            dq = rotate_back_fp64(dq[None, :])[0]
        return formats.bf16_round(dq) if self.num.round_outputs else dq

    def shifts(self, i, lo, hi):
        """Candidate shifts in [lo, hi]: 0, the ends, and one point between
        consecutive shifts at which an element of row i crosses an E4M3
        rounding midpoint or a power-of-two exponent threshold (at the
        unshifted exponent of its group and one binade either side)."""
        x0 = self._ds_rows(i, i + 1)[0]
        v = self.valid[i] & (self.p[i] > 0)
        slope = np.where(v, self.p[i].astype(np.float64) / self.l[i], 0.0)   # x(a) = x0 - slope a
        L = x0.shape[0]
        events = []
        mids = _E4M3_MIDPOINTS
        for j0 in range(0, L, BLOCK):
            jj = np.flatnonzero(v[j0:j0 + BLOCK]) + j0
            if not len(jj):
                continue
            sc = np.ldexp(1.0, self.k_exp[jj]) if self.k_exp is not None else np.ones(len(jj))
            e0 = formats.EXPONENT_RULES[self.num.rule](np.max(np.abs(x0[jj] * sc)))
            for e in (e0 - 1, e0, e0 + 1):
                # x(a) sc 2^-e = m  <=>  a = (x0 - m 2^e / sc) / slope
                lo_v = (x0[jj] - slope[jj] * hi) * sc * np.ldexp(1.0, -e)
                hi_v = (x0[jj] - slope[jj] * lo) * sc * np.ldexp(1.0, -e)
                for k, j in enumerate(jj):
                    a_, b_ = np.searchsorted(mids, [lo_v[k], hi_v[k]])
                    ms = mids[a_:b_]
                    if len(ms):
                        events.append((x0[j] - np.ldexp(ms, e) / sc[k]) / slope[j])
                    for thr in (448.0, -448.0, 224.0, -224.0):
                        if lo_v[k] <= thr <= hi_v[k]:
                            events.append(np.array([(x0[j] - np.ldexp(thr, e) / sc[k]) / slope[j]]))
        ev = np.concatenate(events) if events else np.zeros(0)
        ev = np.unique(np.clip(ev, lo, hi))
        pts = np.concatenate([[0.0, lo, hi], (ev[1:] + ev[:-1]) / 2 if len(ev) > 1 else [], ev])
        pts = pts[(pts >= lo) & (pts <= hi)]
        return pts[np.argsort(np.abs(pts), kind="stable")]


def _e4m3_midpoints():
    mags = np.unique(formats.e4m3_decode(np.arange(256, dtype=np.uint8)))
    mags = mags[np.isfinite(mags)]
    vals = np.unique(np.concatenate([-mags, mags]))
    return (vals[1:] + vals[:-1]) / 2


_E4M3_MIDPOINTS = _e4m3_midpoints()


def allowances(q, k, v, do, cu_seqlens, num: Numerics | None = None):
    """Decision bounds of the whole call (see the module docstring): ``o``
    ``[T, H, d]`` and ``dv`` ``[T, Hk, d]`` per-element allowances; ``e_D``
    ``[T, H]``, the bound of the admissible shift of D per query row;
    ``dq_rows``, a ``DqUnderDShift`` per (document start, head); ``docs``,
    the (start, end) of every non-empty document."""
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
    out = dict(o=np.zeros((T, H, d)), e_D=np.zeros((T, H)), dq_rows={},
               docs=[(s, e) for s, e in doc_bounds(cu_seqlens) if e > s])
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
            a = doc_head_allowances(fw, qs_all[sl, h], ks_all[sl, hk], qt["v"][sl, hk], qt["v_key"][sl, hk],
                                    do_deq[sl, h], num, c32)
            out["o"][sl, h] = a["o"]
            out["e_D"][sl, h] = a["e_D"]
            dv_w[sl, hk] += a["dv"]
            dv_raw[sl, hk] += (fw["peff"] / fw["l"][:, None]).T @ do_deq[sl, h]
            o_out = formats.bf16_round(fw["o"]) if num.round_outputs else fw["o"]
            out["dq_rows"][(s, h)] = DqUnderDShift(fw, qt["k"][sl, hk], qt["v"][sl, hk], qt["v_key"][sl, hk],
                                                   do_deq[sl, h], o_out, s32, num,
                                                   qt["k_exp"][hk, sl] if num.exact else None)
    out["dv"] = _bf16_span(dv_raw, dv_w) if num.round_outputs else dv_w
    return out


