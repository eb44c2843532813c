"""Forward and backward of the causal block-scaled attention call (oracle;
test infrastructure).

This is not exact attention: quantization is part of the result, so the
algorithm is followed step by step -- the method's quantization rules, then
attention on the dequantized operands.  Matrix products of dequantized E4M3
operands are exact in fp64 (every product of two E4M3 values of one block pair
is a multiple of 2**-18 of the pair's scale and the sums stay below 2**25 of it,
well inside 53 bits); everything else is fp64 rounded once to the precision the
method fixes.  Work is done per (document, head); nothing crosses a document.

Readings of points the pages leave open (each a numbered reading in the
design notes):

* Scores ``S' = fp32(fp32(Q~ K~^T) * c)`` with ``c = fp32(softmax_scale *
  log2 e)``; ``softmax_scale = 1/sqrt(d)`` by default.
* Row-max scaling: the row maximum of S' is rounded up to an integer ``m``,
  and ``P = fp32(exp2(S' - m))`` lies in (0, 1].  The backward must replay
  the forward's tiling, diagonal decisions, exponential evaluation and
  row-max scaling ([Summary, §3.3 Forward-Backward Numerical Consistency];
  [Reading, 4.3]); with an integer maximum every online-softmax rescale is a
  power of two, so the probabilities relative to the final maximum are the
  ones both passes see.
* The probability operand uses the fixed exponent -8 (the round-up rule
  applied to P's bound of 1): ``P^ = E4M3(P * 2**8) * 2**-8``; it is a
  constant, so one payload serves P^V and P^T dO.
* Diagonal pairs are those whose query and key lie in the same doc-local
  32-token block; there V uses per-key codes, and each key's exponent is
  folded along the contraction (key) axis into P before P is quantized
  ([Summary], opening paragraphs: per-key V scales with a K-fold on diagonal
  tiles as a causal-leak limit; [News, "Key design choices"]: per-key scale
  folding).  The fold is taken relative to the largest per-key exponent among
  the keys the query may see in its block,
  ``e_ref(i) = max{e_key(j) : blk(j) = blk(i), j <= i}``, so
  ``f_ij = 2**(e_key(j) - e_ref(i)) <= 1`` and
  ``P_eff = E4M3(P * f * 2**8) * 2**-8 / f``.  Nothing in this product then
  depends on a later key.  (A fold relative to the block exponent, switch
  ``fold="block"``, still depends on later keys of the block, because a
  smaller ``f`` pushes more entries into E4M3's subnormal range.)  Defining
  "diagonal" at block level makes the decision identical for every tiling.
* The softmax denominator ``l`` and dS use the unquantized P; O and dV use
  the quantized P^ ([Reading, 4.3] lists P^ as the replayed quantity).
* D is built from the same quantized dO as dP and the bf16 output
  ([Summary, §3.3]; [Reading, 4.3]).
* dS gets one round-up exponent per doc-local 32 x 32 block from the block's
  max-abs ([Summary, §3.3], second bullet; [Reading, 4.3]).
* dQ and dK use the same token-block Q~ and K~ payloads as the forward.  With
  the Hadamard rotation on, both are rotated back (the normalised matrix is
  symmetric and orthogonal).
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import formats
from .hadamard import rotate_back_fp64
from .quant import BLOCK, doc_bounds, fold_reference, quantize_qkv, quantize_token_blocks

LOG2E = float(np.log2(np.e))
P_EXP = -8          # fixed exponent of the probability operand


@dataclass
class Numerics:
    """Switches of the oracle.  The defaults are the method."""
    quantize_operands: bool = True   # E4M3 Q, K, V, dO (False: identity codecs)
    quantize_p: bool = True          # E4M3 probability operand
    quantize_ds: bool = True         # E4M3 dS with 32x32 block exponents
    round_outputs: bool = True       # bf16 O, dQ, dK, dV
    rule: str = "roundup"            # exponent rule: roundup | ceil | floor
    granularity: str = "block"       # operand scales: block | tensor | token
    hadamard: bool = False
    causal: bool = True
    path: str = "mxfp8"              # "mxfp8", or "mixed" (NVFP4 scores)
    fold: str = "causal"             # diagonal V: causal | block | none (block codes)
    softmax_scale: float | None = None
    nvfp4_amax: tuple | None = None  # (Q, K) tensor max-abs when the inputs are a slice
    exact: bool = False              # the exact option (see exact_fold_reference, _ds_exact)
    p_format: str = "e4m3"           # probability operand of O: e4m3 | nvfp4 (p4_quantize)


def scale_constants(d: int, softmax_scale: float | None):
    """fp32 softmax scale and fp32 ``c = softmax_scale * log2(e)``."""
    s32 = np.float32(1.0 / np.sqrt(d)) if not softmax_scale or softmax_scale <= 0 \
        else np.float32(softmax_scale)
    c32 = np.float32(np.float64(s32) * LOG2E)
    return s32, c32


def _out(x, num: Numerics):
    return formats.bf16_round(x) if num.round_outputs else np.asarray(x, dtype=np.float64)


def ds_block_quantize(ds: np.ndarray, valid: np.ndarray, rule: str = "roundup"):
    """dS^ of one (document, head) ([Summary, §3.3], second bullet; [Reading,
    4.3]): the document-local 32 x 32 blocks (query block I, key block J) of
    dS each get one exponent, the round-up exponent of the block's max-abs
    taken over its valid entries (masked entries count as 0), and every valid
    entry becomes E4M3(dS 2^-e) 2^e.  Returns ``(dS^, e)`` with ``e[I, J]``
    the exponent of block (I, J), or -128 where the block holds no valid
    entry (such blocks stay zero).  ``ds`` may be a rectangular slice whose
    first row and column start blocks."""
    Lr, Lc = ds.shape
    out = np.zeros_like(ds)
    exps = np.full((-(-Lr // BLOCK), -(-Lc // BLOCK)), -128, dtype=np.int64)
    ex_rule = formats.EXPONENT_RULES[rule]
    for bi, i0 in enumerate(range(0, Lr, BLOCK)):
        for bj, j0 in enumerate(range(0, Lc, BLOCK)):
            blk = ds[i0:i0 + BLOCK, j0:j0 + BLOCK]
            v = valid[i0:i0 + BLOCK, j0:j0 + BLOCK]
            if not v.any():
                continue
            e = ex_rule(np.max(np.abs(np.where(v, blk, 0.0))))
            exps[bi, bj] = e
            q = formats.e4m3_encode(np.ldexp(np.where(v, blk, 0.0), -e), saturate=(rule == "floor"))
            out[i0:i0 + BLOCK, j0:j0 + BLOCK] = np.where(
                v, np.ldexp(formats.e4m3_decode(q), e), 0.0)
    return out, exps


def _ds_quantize(ds: np.ndarray, valid: np.ndarray, rule: str):
    """dS^ values alone (see ds_block_quantize)."""
    return ds_block_quantize(ds, valid, rule)[0]


def exact_fold_reference(v_exp_key, L: int):
    """Exact option: fold reference of every (query i, key j) pair, the
    largest per-key V exponent among the keys of j's 32-token block that i
    may see: ``max{e_key(j') : blk(j') = blk(j), j' <= i}`` ([Summary] opening
    paragraphs and [Reading, 4.2]: per-key V scales folded into P; the exact
    option applies the fold to every tile).  Entries with j > i are unused."""
    e = np.asarray(v_exp_key, dtype=np.int64)
    ref = np.zeros((L, L), dtype=np.int64)
    for j0 in range(0, L, BLOCK):
        cm = np.maximum.accumulate(e[j0:j0 + BLOCK])          # prefix max inside block J
        n = len(cm)
        i = np.arange(L)
        idx = np.clip(i - j0, 0, n - 1)                         # last key of J that query i sees
        ref[:, j0:j0 + n] = cm[idx][:, None]
    return ref


def _ds_exact(ds, valid, e_fold, rows: bool, rule: str):
    """Exact option: a dS payload for one product.  ``e_fold`` ([L] per-token
    exponent) is folded into dS along the product's contraction axis -- the
    key's K exponent for dQ (``rows``: groups are one query row x 32 keys),
    the query's Q exponent for dK (groups are one key x 32 queries) -- and the
    folded values are quantized with one round-up exponent per group (the
    per-query-row dS exponent of [Reading, 4.2]/[Summary]; a group of 32 along
    the contraction axis is the microscaling block of the product).  Returns
    the effective dS value each product uses (fold removed)."""
    L = ds.shape[0]
    ex_rule = formats.EXPONENT_RULES[rule]
    scale = np.ldexp(1.0, np.asarray(e_fold, dtype=np.int64))
    x = ds * (scale[None, :] if rows else scale[:, None])
    out = np.zeros_like(ds)
    if not rows:
        x, valid_t = x.T, valid.T
    else:
        valid_t = valid
    for r in range(L):
        for c0 in range(0, L, BLOCK):
            v = valid_t[r, c0:c0 + BLOCK]
            if not v.any():
                continue
            seg = np.where(v, x[r, c0:c0 + BLOCK], 0.0)
            e = ex_rule(np.max(np.abs(seg)))
            q = formats.e4m3_decode(formats.e4m3_encode(np.ldexp(seg, -e), saturate=(rule == "floor")))
            out[r, c0:c0 + BLOCK] = np.where(v, np.ldexp(q, e), 0.0)
    if not rows:
        out = out.T
    return out / (scale[None, :] if rows else scale[:, None])


P4_GROUP = 16       # keys per group of the 4-bit probability operand


def roundup_e2m1(a):
    """Smallest integer e with a <= 6 * 2^e, for a > 0 (elementwise): the
    round-up scale rule of the token-block exponent with E2M1's largest
    magnitude 6 in place of E4M3's 448.  With a = M 2^k, M in [1, 2): since
    6 * 2^e = 1.5 * 2^(e + 2), e = k - 2 when M <= 1.5, else k - 1."""
    m, k = np.frexp(np.asarray(a, dtype=np.float64))     # a = m 2^k, m in [0.5, 1)
    return np.where(2.0 * m <= 1.5, k - 3, k - 2).astype(np.int64)


def p4_quantize(x, valid):
    """4-bit probability operand, log-domain NVFP4 ([Summary, §3.5.2 Softmax
    Throughput and MMA Scheduling]; [Reading, 4.4] second bullet): the pages
    quantize P to NVFP4 by taking each group's largest exponent and
    subtracting, so the group scale is a power of two and no element is
    divided.  ``x``: [rows, keys] fp64, nonnegative (P 2^8 times the diagonal
    fold); ``valid``: the visible pairs.  Groups are 16 consecutive keys from
    the document start, per row.  Per group, e = roundup_e2m1 of the largest
    visible x (a group with none, or only zeros, is all zero); each visible
    element becomes E2M1_RNE(x 2^-e) 2^e (at most 6 2^e, so nothing saturates),
    and that value enters the FP8 product as an E4M3 number (exact but below
    E4M3's range).  Returns the values (0 where not visible)."""
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    n = x.shape[1]
    for g0 in range(0, n, P4_GROUP):
        sl = slice(g0, min(g0 + P4_GROUP, n))
        seg = np.where(valid[:, sl], x[:, sl], 0.0)
        amax = seg.max(axis=1)
        nz = amax > 0
        e = np.where(nz, roundup_e2m1(np.where(nz, amax, 1.0)), 0)
        q = formats.e2m1_round(np.ldexp(seg, -e[:, None]))
        out[:, sl] = np.where(valid[:, sl], np.ldexp(q, e[:, None]), 0.0)
    return formats.e4m3_round(out)


def forward_doc(qd, kd, vblk, vkey, v_exp_blk, v_exp_key, c32, num: Numerics):
    """Forward of one (document, head).

    qd, kd: dequantized score operands ``[L, d]`` fp64 (E4M3 token-block, or
    NVFP4 on the mixed path); vblk, vkey: dequantized V ``[L, d]`` fp64.  v_exp_blk, v_exp_key:
    int ``[L]`` exponents of V's block and per-key scales.
    Returns a dict with fp32 S', integer row max ``m``, fp32 P, fp32 ``l``,
    the effective probability operand ``peff`` and the diagonal mask.
    """
    L = qd.shape[0]
    i = np.arange(L)
    valid = (i[None, :] <= i[:, None]) if num.causal else np.ones((L, L), bool)
    s = formats.fp32_round(qd @ kd.T)                       # exact sum -> fp32
    sp = (s.astype(np.float32) * c32).astype(np.float64)    # fp32 product
    m = np.ceil(np.max(np.where(valid, sp, -np.inf), axis=1)) if L else np.zeros(0)
    p = formats.fp32_round(np.exp2(np.where(valid, sp - m[:, None], -np.inf)))
    l = formats.fp32_round(p.sum(axis=1))
    blk = i // BLOCK
    diag = (blk[:, None] == blk[None, :]) & valid
    if num.fold == "none":               # block codes on the diagonal too
        diag = np.zeros_like(diag)
    e_ref = fold_reference(v_exp_key, num.causal)
    if num.fold == "block":
        e_ref = v_exp_blk
    if num.exact:
        # every visible pair uses the per-key (per-token) V codes, folded into
        # P against the reference of its (query, key block)
        diag = valid.copy()
        e_ref2 = exact_fold_reference(v_exp_key, L)
    else:
        e_ref2 = np.broadcast_to(e_ref[:, None], (L, L))
    if num.quantize_p:
        f = np.where(diag, np.ldexp(1.0, np.minimum(v_exp_key[None, :] - e_ref2, 0)), 1.0)
        if num.p_format == "nvfp4":
            # one 4-bit operand over every visible pair (the fold applied first)
            peff = np.ldexp(p4_quantize(np.ldexp(p * f, -P_EXP), valid), P_EXP) / f
        else:
            p_off = np.ldexp(formats.e4m3_round(np.ldexp(p, -P_EXP)), P_EXP)
            p_dia = np.ldexp(formats.e4m3_round(np.ldexp(p * f, -P_EXP)), P_EXP) / f
            peff = np.where(diag, p_dia, p_off)
    else:
        peff = p
    o = (np.where(diag, 0.0, peff) @ vblk + np.where(diag, peff, 0.0) @ vkey) / l[:, None]
    return dict(sp=sp, m=m.astype(np.int64), p=p, l=l, peff=peff, diag=diag,
                valid=valid, o=o, fold=f if num.quantize_p else None)


def backward_doc(fw, qd, kd, vblk, vkey, dod, o_out, s32, num: Numerics):
    """Backward of one (document, head) given the forward record ``fw``,
    the dequantized dO ``dod`` and the bf16 output ``o_out``."""
    p, l, peff, diag, valid = fw["p"], fw["l"], fw["peff"], fw["diag"], fw["valid"]
    D = np.sum(dod * o_out, axis=1)                                   # fp64
    dp = np.where(diag, dod @ vkey.T, dod @ vblk.T)
    ds = np.where(valid, (p / l[:, None]) * (dp - D[:, None]), 0.0)
    if num.exact and num.quantize_ds:
        # exact option: one payload per product, each with the other operand's
        # per-token exponent folded in and one exponent per 32 along its
        # contraction axis (fw carries the per-token Q and K exponents)
        dsq = _ds_exact(ds, valid, fw["k_exp_tok"], True, num.rule)
        dsq_k = _ds_exact(ds, valid, fw["q_exp_tok"], False, num.rule)
    else:
        dsq = _ds_quantize(ds, valid, num.rule) if num.quantize_ds else ds
        dsq_k = dsq
    dv = (peff / l[:, None]).T @ dod
    dq = float(s32) * (dsq @ kd)
    dk = float(s32) * (dsq_k.T @ qd)
    nz = valid & (ds != 0)
    zeroed = int(np.count_nonzero(nz & (dsq == 0)))
    return dict(D=D, ds=ds, dsq=dsq, dsq_k=dsq_k, dq=dq, dk=dk, dv=dv,
                ds_nonzero=int(np.count_nonzero(nz)), ds_zeroed=zeroed)


def dq_prescale(do_exp, k_exp, v_exp, cu_seqlens, head_dim: int, causal_dq_scale: bool = False,
                exact: bool = False):
    """Power-of-two prescale of the fp16 dQ accumulator ([Reading, 4.4] third
    bullet: dQ partials are reduced in FP16 after a data-dependent power-of-two
    scale; [Summary] bullets on the optional causal dQ scale).  For query
    token i of a document, with exponents as integers ([H, T] for dO, [Hk, T]
    for K and V; query head h reads key/value head h // (H / Hk)):

        sigma_i = e_dO(i) + E_V + E_K + log2(d) + 13

    E_V, E_K: the largest V and K exponents over the document (default), over
    the tokens j <= i (``causal_dq_scale``, or per token with the exact
    option, whose exponents are per token).  Since every |dS~_ij| sums to at
    most 2.2 d 448^2 2^(e_dO + E_V) over a row (P / l sums to 1, |dP - D| is
    at most twice a d-term dot product of codes, E4M3 rounding adds 1/16) and
    |K~| <= 448 2^E_K, every partial sum of sum_j dS~_ij K~_j scaled by
    2^-sigma stays below 2^15, inside fp16.  Returns int64 [H, T]."""
    do_exp = np.asarray(do_exp, np.int64)
    k_exp = np.asarray(k_exp, np.int64)
    v_exp = np.asarray(v_exp, np.int64)
    H, T = do_exp.shape
    group = H // k_exp.shape[0]
    lg = int(np.log2(head_dim))
    out = np.zeros((H, T), dtype=np.int64)
    for s, e in doc_bounds(cu_seqlens):
        if e == s:
            continue
        for h in range(H):
            ek, ev = k_exp[h // group, s:e], v_exp[h // group, s:e]
            if causal_dq_scale or exact:
                # (block exponents repeat over a block, so this is the max over blocks J <= I)
                ek, ev = np.maximum.accumulate(ek), np.maximum.accumulate(ev)
            else:
                ek, ev = np.full(e - s, ek.max()), np.full(e - s, ev.max())
            out[h, s:e] = do_exp[h, s:e] + ek + ev + lg + 13
    return out


def training_call(q, k, v, do, cu_seqlens, num: Numerics | None = None):
    """Quantize, forward and backward of the whole packed call.

    q, do: ``[T, H, d]``; k, v: ``[T, Hk, d]`` with Hk dividing H -- grouped
    query attention when Hk < H: query head h reads key/value head
    h // (H / Hk), and the dK, dV of a key/value head are the sums over its
    query heads, rounded once ([Reading, 5.2] lists GQA variants among the measured
    workloads; [Reading, 6.3] its deterministic reduction).  All hold bf16
    values.  Returns a dict with the quantized payloads (codes and exponents,
    bit-comparable), the forward statistics ``row_max`` (int) and ``row_sum``
    (fp32) in ``[H, T]``, ``D`` in ``[H, T]``, and the outputs O, dQ, dK, dV as
    fp64 arrays holding bf16 values (or unrounded values when
    ``round_outputs`` is off).
    """
    num = num or Numerics()
    q = np.asarray(q, dtype=np.float64)
    T, H, d = q.shape
    Hk = np.asarray(k).shape[1]
    if H % Hk:
        raise ValueError("key/value heads must divide query heads")
    group = H // Hk
    s32, c32 = scale_constants(d, num.softmax_scale)
    gran = "token" if num.exact else num.granularity      # exact option: per-token operand scales
    if num.exact and num.path != "mxfp8":
        raise ValueError("the exact option is defined for the MXFP8 path")
    if num.quantize_operands:
        qt = quantize_qkv(q, k, v, cu_seqlens, num.hadamard, num.rule, gran)
        do_codes, do_exp, do_deq = quantize_token_blocks(do, cu_seqlens, num.rule, gran)
        qs_all, ks_all = qt["q"], qt["k"]
        if num.path == "mixed":
            from .nvfp4 import quantize_nvfp4
            qa, ka = num.nvfp4_amax if num.nvfp4_amax is not None else (None, None)
            *_, qs_all = quantize_nvfp4(qt["q_rot"], qa)
            *_, ks_all = quantize_nvfp4(qt["k_rot"], ka)
        elif num.path != "mxfp8":
            raise ValueError(num.path)
    else:
        from .hadamard import fwht_fp32
        q32 = np.asarray(q, np.float32)
        k32 = np.asarray(k, np.float32)
        if num.hadamard:
            q32, k32 = fwht_fp32(q32), fwht_fp32(k32)
        z = np.zeros((H, T), dtype=np.int64)
        zk = np.zeros((Hk, T), dtype=np.int64)
        v64 = np.asarray(v, dtype=np.float64)
        qt = dict(q=q32.astype(np.float64), k=k32.astype(np.float64), v=v64, v_key=v64,
                  v_exp=zk, v_key_exp=zk)
        do_codes, do_exp, do_deq = None, z, np.asarray(do, dtype=np.float64)
        qs_all, ks_all = qt["q"], qt["k"]

    o = np.zeros((T, H, d))
    dq = np.zeros((T, H, d))
    dk_sum = np.zeros((T, Hk, d))     # unrounded sums over the query heads of a group
    dv_sum = np.zeros((T, Hk, d))
    row_max = np.zeros((H, T), dtype=np.int64)
    row_sum = np.zeros((H, T), dtype=np.float64)
    Dst = np.zeros((H, T))
    ds_nonzero = ds_zeroed = 0
    for s, e in doc_bounds(cu_seqlens):
        if e == s:
            continue
        for h in range(H):
            sl = slice(s, e)
            hk = h // group
            fw = forward_doc(qs_all[sl, h], ks_all[sl, hk], qt["v"][sl, hk], qt["v_key"][sl, hk],
                             qt["v_exp"][hk, sl], qt["v_key_exp"][hk, sl], c32, num)
            o_out = _out(fw["o"], num)
            if num.exact:
                fw["q_exp_tok"], fw["k_exp_tok"] = qt["q_exp"][h, sl], qt["k_exp"][hk, sl]
            bw = backward_doc(fw, qt["q"][sl, h], qt["k"][sl, hk], qt["v"][sl, hk],
                              qt["v_key"][sl, hk], do_deq[sl, h], o_out, s32, num)
            o[sl, h] = o_out
            row_max[h, sl] = fw["m"]
            row_sum[h, sl] = fw["l"]
            Dst[h, sl] = bw["D"]
            dqh, dkh = bw["dq"], bw["dk"]
            if num.hadamard:
                dqh, dkh = rotate_back_fp64(dqh), rotate_back_fp64(dkh)
            dq[sl, h] = _out(dqh, num)
            dk_sum[sl, hk] += dkh
            dv_sum[sl, hk] += bw["dv"]
            ds_nonzero += bw["ds_nonzero"]
            ds_zeroed += bw["ds_zeroed"]
    dk, dv = _out(dk_sum, num), _out(dv_sum, num)
    res = dict(o=o, dq=dq, dk=dk, dv=dv, row_max=row_max, row_sum=row_sum, D=Dst,
               do_codes=do_codes, do_exp=do_exp,
               ds_zero_fraction=(ds_zeroed / ds_nonzero) if ds_nonzero else 0.0)
    if num.quantize_operands:
        res.update({k_: qt[k_] for k_ in ("q_codes", "q_exp", "k_codes", "k_exp", "v_codes",
                                          "v_exp", "v_key_codes", "v_key_exp", "v_ref_exp")})
    return res
