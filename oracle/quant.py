"""Operand quantization of the attention training call (oracle; test infrastructure).

Layouts: per-token tensors are ``[T, H, d]`` (packed documents, no padding);
per-token metadata is ``[H, T]``.  Documents are given by ``cu_seqlens``
(``[0, L_0, L_0 + L_1, ..., T]``).

Rules followed:

* Token-block scaling: one power-of-two exponent per 32 consecutive tokens of
  one document times the full head dimension, per head.  Because the exponent
  is shared by the whole 32 x d block, codes and scales stay valid under
  transpose, so one E4M3 payload serves both matrix orientations
  ([Summary, §3.1 Token-Block Scaling]; [Reading, 4.1]).
* Blocks are counted from each document's start and never cross a document
  boundary (document-local scales; [Reading, 4.4] packed layout and
  [Reading, part 八] third insight; [News, "Key design choices"]).  A
  document's last block may be shorter than 32 tokens.  Every token carries
  its block's exponent ([Summary, §3.6.2 Load-Balanced Scheduling]: per-token
  scale metadata).
* The exponent is rounded up so that the block maximum never clamps
  ([Summary, §3.2 Causally Safe Scales]); see ``formats.roundup_exponent``.
* V additionally gets one exponent per key, used on diagonal blocks where the
  per-key scale is folded along the contraction axis into P
  ([Summary, abstract paragraph on causal leakage]; [News, "Key design
  choices"]: per-key scale folding).
"""

from __future__ import annotations

import numpy as np

from . import formats
from .hadamard import fwht_fp32

BLOCK = 32


def doc_bounds(cu_seqlens) -> list[tuple[int, int]]:
    cu = [int(c) for c in cu_seqlens]
    if cu[0] != 0 or any(b < a for a, b in zip(cu, cu[1:])):
        raise ValueError("cu_seqlens must start at 0 and be non-decreasing")
    return list(zip(cu[:-1], cu[1:]))


def doc_blocks(start: int, end: int) -> list[tuple[int, int]]:
    """Token ranges of the 32-token blocks of one document, from its start."""
    return [(b, min(b + BLOCK, end)) for b in range(start, end, BLOCK)]


def local_block_index(cu_seqlens) -> np.ndarray:
    """blk(i): document-local block index of every packed token."""
    T = int(cu_seqlens[-1])
    out = np.zeros(T, dtype=np.int64)
    for s, e in doc_bounds(cu_seqlens):
        out[s:e] = (np.arange(s, e) - s) // BLOCK
    return out


def _encode(scaled: np.ndarray, rule: str) -> np.ndarray:
    # Only the microscaling floor rule can overflow; its reference conversion
    # clamps to the largest finite value.
    return formats.e4m3_encode(scaled, saturate=(rule == "floor"))


def quantize_token_blocks(x, cu_seqlens, rule: str = "roundup",
                          granularity: str = "block"):
    """Quantize ``x`` ([T, H, d], values exact in fp32) to E4M3 codes.

    ``granularity``: ``"block"`` (the method: 32 doc-local tokens x d per
    head), ``"tensor"`` (one exponent for the whole tensor -- the leak worst
    case, a positive control for the causality probe) or ``"token"`` (one
    exponent per token and head).

    Returns ``(codes u8 [T,H,d], exps int64 [H,T], deq fp64 [T,H,d])`` where
    ``deq = value(code) * 2**exp`` exactly.
    """
    x = np.asarray(x, dtype=np.float64)
    T, H, d = x.shape
    ex_rule = formats.EXPONENT_RULES[rule]
    exps = np.zeros((H, T), dtype=np.int64)
    if granularity == "tensor":
        exps[:] = ex_rule(np.max(np.abs(x)) if x.size else 0.0)
    elif granularity == "token":
        for h in range(H):
            for t in range(T):
                exps[h, t] = ex_rule(np.max(np.abs(x[t, h])))
    elif granularity == "block":
        for s, e in doc_bounds(cu_seqlens):
            for bs, be in doc_blocks(s, e):
                for h in range(H):
                    exps[h, bs:be] = ex_rule(np.max(np.abs(x[bs:be, h, :])))
    else:
        raise ValueError(granularity)
    scale = np.ldexp(1.0, -exps.T)[:, :, None]          # 2**-e per (t, h)
    codes = _encode(x * scale, rule)
    deq = formats.e4m3_decode(codes) * np.ldexp(1.0, exps.T)[:, :, None]
    return codes, exps, deq


def quantize_per_key(v, rule: str = "roundup"):
    """Per-key V quantization: ``e_key(j) = roundup(max_d |V_jd|)`` for every
    (token, head), codes ``E4M3(V_j * 2**-e_key(j))``."""
    v = np.asarray(v, dtype=np.float64)
    T, H, d = v.shape
    ex_rule = formats.EXPONENT_RULES[rule]
    exps = np.zeros((H, T), dtype=np.int64)
    for h in range(H):
        for t in range(T):
            exps[h, t] = ex_rule(np.max(np.abs(v[t, h])))
    codes = _encode(v * np.ldexp(1.0, -exps.T)[:, :, None], rule)
    deq = formats.e4m3_decode(codes) * np.ldexp(1.0, exps.T)[:, :, None]
    return codes, exps, deq


def fold_reference(e_key, causal: bool = True):
    """Per query: the largest per-key V exponent among the keys of its own
    32-token block that it may see (all keys of the block when not causal)."""
    e_key = np.asarray(e_key, dtype=np.int64)
    out = np.empty_like(e_key)
    for b0 in range(0, e_key.shape[0], BLOCK):
        seg = e_key[b0:b0 + BLOCK]
        out[b0:b0 + BLOCK] = np.maximum.accumulate(seg) if causal else seg.max()
    return out


def quantize_qkv(q, k, v, cu_seqlens, hadamard: bool = False, rule: str = "roundup",
                 granularity: str = "block"):
    """The fused forward-side quantization: optional Hadamard rotation of Q and
    K rows (fp32), then token-block E4M3 codes for Q, K, V and per-key codes
    for V ([Reading, 4.4] fused quantizer; [Summary, §4.3 Ablation Study])."""
    q32 = np.asarray(q, dtype=np.float32)
    k32 = np.asarray(k, dtype=np.float32)
    if hadamard:
        q32 = fwht_fp32(q32)
        k32 = fwht_fp32(k32)
    out = {}
    out["q_codes"], out["q_exp"], out["q"] = quantize_token_blocks(q32, cu_seqlens, rule, granularity)
    out["k_codes"], out["k_exp"], out["k"] = quantize_token_blocks(k32, cu_seqlens, rule, granularity)
    out["v_codes"], out["v_exp"], out["v"] = quantize_token_blocks(v, cu_seqlens, rule, granularity)
    out["v_key_codes"], out["v_key_exp"], out["v_key"] = quantize_per_key(v, rule)
    ref = np.zeros_like(out["v_key_exp"])
    for s, e in doc_bounds(cu_seqlens):
        for h in range(ref.shape[0]):
            ref[h, s:e] = fold_reference(out["v_key_exp"][h, s:e])
    out["v_ref_exp"] = ref          # per query: fold reference of the diagonal P V
    out["q_rot"], out["k_rot"] = q32.astype(np.float64), k32.astype(np.float64)
    return out
