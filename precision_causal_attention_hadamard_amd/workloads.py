"""Seeded synthetic inputs for the attention training call.

This module only draws random numbers and rounds them to bf16; it holds none
of the method's arithmetic, so both the HIP path and the CPU oracle can take
their inputs from it.

Recipe (the pages' kernel benchmarks use synthetic packed workloads with 16
heads and head dim 128; no dataset is involved):

* every tensor is drawn as fp32 N(0, 1) from ``numpy.random.default_rng(seed)``
  (PCG64) and rounded to bf16 (round-to-nearest-even);
* draw order: Q, K, V, dO, then structure (outlier channels, document
  lengths);
* layout ``[T, H, d]``, packed documents described by ``cu_seqlens``.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

SEED_BASE = 20261100


@dataclass
class Workload:
    name: str
    q: torch.Tensor            # bf16 [T, H, d] on the CPU
    k: torch.Tensor
    v: torch.Tensor
    do: torch.Tensor
    cu_seqlens: list
    heads: int
    head_dim: int
    hadamard: bool = False
    path: int = 0              # 0 = MXFP8, 1 = mixed NVFP4 scores
    causal_dq_scale: bool = False
    notes: dict = field(default_factory=dict)

    @property
    def kv_heads(self) -> int:
        return int(self.k.shape[1])

    @property
    def total_tokens(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def doc_lens(self) -> list:
        return [b - a for a, b in zip(self.cu_seqlens, self.cu_seqlens[1:])]

    @property
    def has_outliers(self) -> bool:
        return bool(self.notes.get("outlier_scale"))

    def causal_pairs(self) -> int:
        """Number of (query, key) pairs the causal call computes, all heads."""
        return self.heads * sum(L * (L + 1) // 2 for L in self.doc_lens)

    def flops(self) -> int:
        """Algorithmic FLOPs of forward (2 products) + backward (5 products),
        each 2*d per causal pair: 14 * d * pairs."""
        return 14 * self.head_dim * self.causal_pairs()


def _bf16(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def draw_tensors(rng, T: int, H: int, d: int, outlier_scale: float = 0.0, kv_heads: int = 0):
    """Q, K, V, dO as bf16; optional outlier channels drawn after the tensors.
    K and V carry ``kv_heads`` heads (0 = H; fewer for grouped query attention)."""
    Hk = kv_heads or H
    raw = [rng.standard_normal((T, h, d), dtype=np.float32) for h in (H, Hk, Hk, H)]
    if outlier_scale:
        n_out = max(1, int(round(0.01 * d)))
        for x in raw:
            for h in range(x.shape[1]):
                ch = rng.choice(d, size=n_out, replace=False)
                x[:, h, ch] *= np.float32(outlier_scale)
    return [_bf16(x) for x in raw]


def lognormal_fill(rng, total: int, median: float = 1024.0, sigma: float = 1.0,
                   lo: int = 17, hi: int = 8192) -> list:
    """Document lengths filling ``total`` tokens: lengths
    ``round(exp(N(ln median, sigma)))`` clipped to [lo, hi] are appended while
    they fit; the remainder becomes the last document, merged into the
    previous one when it is shorter than ``lo``."""
    lens = []
    left = total
    while True:
        L = int(np.clip(np.round(np.exp(rng.normal(np.log(median), sigma))), lo, hi))
        if L > left:
            break
        lens.append(L)
        left -= L
    if left:
        if left < lo and lens:
            lens[-1] += left
        else:
            lens.append(left)
    return lens


def _cu(lens) -> list:
    return [0] + list(np.cumsum(lens).astype(int).tolist())


def config(k: int, seed: int | None = None, kv_heads: int = 0) -> Workload:
    """The five workloads of the call (k = 1..5).  ``kv_heads`` (0 = one per
    query head) gives the grouped-query variant: K and V drawn with that many
    heads, everything else as in the plain workload."""
    seed = SEED_BASE + k if seed is None else seed
    rng = np.random.default_rng(seed)

    def wl(name, q, kk, v, do, cu, heads, d, **kw):
        if kv_heads and kv_heads != heads:
            name = name.replace(f"_h{heads}_", f"_h{heads}_kv{kv_heads}_")
        return Workload(name, q, kk, v, do, cu, heads, d, **kw)

    if k == 1:   # tiny: one 256-token document, 2 heads, head dim 64
        q, kk, v, do = draw_tensors(rng, 256, 2, 64, kv_heads=kv_heads)
        return wl("tiny_1x256_h2_d64", q, kk, v, do, [0, 256], 2, 64)
    if k == 2:   # batch 2 x 4096, 16 heads, d 128, 1% outlier channels x20, Hadamard on
        q, kk, v, do = draw_tensors(rng, 8192, 16, 128, outlier_scale=20.0, kv_heads=kv_heads)
        return wl("batched_2x4096_h16_d128_outliers_hadamard", q, kk, v, do,
                  [0, 4096, 8192], 16, 128, hadamard=True, notes={"outlier_scale": 20.0})
    if k == 3:   # packed 4 rows x 16384, lognormal documents
        q, kk, v, do = draw_tensors(rng, 65536, 16, 128, kv_heads=kv_heads)
        lens = []
        for _ in range(4):
            lens += lognormal_fill(rng, 16384)
        return wl("packed_4x16384_lognormal_h16_d128", q, kk, v, do, _cu(lens), 16, 128)
    if k == 4:   # long context 32768: two 12288-token docs + lognormal shorts
        q, kk, v, do = draw_tensors(rng, 32768, 16, 128, kv_heads=kv_heads)
        lens = [12288, 12288] + lognormal_fill(rng, 8192)
        return wl("long_1x32768_h16_d128", q, kk, v, do, _cu(lens), 16, 128)
    if k == 5:   # mixed path, shapes of config 2, no outliers
        q, kk, v, do = draw_tensors(rng, 8192, 16, 128, kv_heads=kv_heads)
        return wl("mixed_2x4096_h16_d128", q, kk, v, do, [0, 4096, 8192], 16, 128, path=1)
    raise ValueError(k)


# The pages' packed kernel-benchmark shapes beside the five workloads above
# (16 heads, head dim 128, N(0, 1), MXFP8, Hadamard off): equal-length batches
# and the two skewed calls, one 8192-token document followed by 32 or 224
# documents of 256 tokens.
PAGES_SHAPES = {
    "equal_4x4096": [4096] * 4,
    "equal_16x1024": [1024] * 16,
    "equal_16x4096": [4096] * 16,
    "equal_64x1024": [1024] * 64,
    "skew_8192_32x256": [8192] + [256] * 32,
    "skew_8192_224x256": [8192] + [256] * 224,
}


def pages_shape(name: str, seed: int = SEED_BASE + 600, kv_heads: int = 0) -> Workload:
    """One of ``PAGES_SHAPES`` with inputs drawn by the recipe above."""
    lens = PAGES_SHAPES[name]
    rng = np.random.default_rng(seed)
    q, kk, v, do = draw_tensors(rng, int(sum(lens)), 16, 128, kv_heads=kv_heads)
    kvs = f"_kv{kv_heads}" if kv_heads and kv_heads != 16 else ""
    return Workload(f"{name}_h16{kvs}_d128", q, kk, v, do, _cu(lens), 16, 128)


def small_packed(seed: int, doc_lens, heads: int = 2, head_dim: int = 64,
                 outlier_scale: float = 0.0, hadamard: bool = False, path: int = 0,
                 kv_heads: int = 0) -> Workload:
    """A small packed workload for parity tests (documents off 32-alignment);
    ``kv_heads`` < ``heads`` gives grouped query attention."""
    rng = np.random.default_rng(seed)
    T = int(sum(doc_lens))
    q, kk, v, do = draw_tensors(rng, T, heads, head_dim, outlier_scale, kv_heads)
    kvs = f"_kv{kv_heads}" if kv_heads and kv_heads != heads else ""
    return Workload(f"packed_{'_'.join(map(str, doc_lens))}_h{heads}{kvs}_d{head_dim}", q, kk, v, do,
                    _cu(doc_lens), heads, head_dim, hadamard=hadamard, path=path,
                    notes={"outlier_scale": outlier_scale} if outlier_scale else {})


def extreme_rows(seed: int, doc_lens, heads: int = 2, head_dim: int = 64, logit: float = 150.0) -> Workload:
    """Rows whose scores all sit far above or far below zero: K rows are
    beta u + N(0, 0.3^2) noise with u the all-ones vector, and each query row is
    s beta u + N(0, 0.3^2) noise with s = +1, -1 or 0 in runs of 32 rows (one
    32-token block each, cycling +1, 0, -1, 0), beta chosen so that
    beta^2 d log2(e) / sqrt(d) = ``logit``: scores of the s = +1 rows lie near
    +logit and of the s = -1 rows near -logit in log2 units."""
    rng = np.random.default_rng(SEED_BASE + 700 + seed)
    T = int(sum(doc_lens))
    d = head_dim
    beta = float(np.sqrt(logit * np.sqrt(d) / (d * np.log2(np.e))))
    sign = np.array([1.0, 0.0, -1.0, 0.0], dtype=np.float32)[(np.arange(T) // 32) % 4]
    noise = lambda: rng.normal(0.0, 0.3, size=(T, heads, d)).astype(np.float32)
    k = beta + noise()
    q = sign[:, None, None] * beta + noise()
    v = rng.standard_normal((T, heads, d), dtype=np.float32)
    do = rng.standard_normal((T, heads, d), dtype=np.float32)
    return Workload(f"extreme_rows_{'_'.join(map(str, doc_lens))}_h{heads}_d{d}", _bf16(q), _bf16(k), _bf16(v),
                    _bf16(do), _cu(doc_lens), heads, d, notes={"logit": logit})


def saved_forward_state(seed: int, T: int, H: int, d: int):
    """Stand-ins for the forward's saved outputs, for tests of the backward's
    preparation stage on its own: O bf16 ``[T, H, d]`` drawn N(0, 1), the
    integer row maximum int32 ``[H, T]`` uniform in [-4, 12] and the row sum
    fp32 ``[H, T]`` uniform in [1, 64]."""
    rng = np.random.default_rng(SEED_BASE + 900 + seed)
    o = _bf16(rng.standard_normal((T, H, d), dtype=np.float32))
    row_max = torch.from_numpy(rng.integers(-4, 13, size=(H, T)).astype(np.int32))
    row_sum = torch.from_numpy(rng.uniform(1.0, 64.0, size=(H, T)).astype(np.float32))
    return o, row_max, row_sum


def e4m3_sweep(shifts=range(-20, 21), head_dim: int = 128) -> Workload:
    """Every finite bf16 value times every power of two 2^k (k in ``shifts``)
    that stays inside the E4M3 range of a 32-token block scaled by 2^k: each
    block holds one anchor of magnitude 448 * 2^k (so its exponent is k) and
    then bf16 values v with |v| <= 448 * 2^k, in increasing order of their
    bit patterns.  One head; Q = K = V = dO; one document per shift so that
    blocks never mix shifts."""
    bits = np.arange(1 << 16, dtype=np.uint32)
    vals = (bits << 16).view(np.float32)
    vals = vals[np.isfinite(vals)]
    rows, lens = [], []
    per_row = head_dim
    for k in shifts:
        anchor = np.float32(448.0 * 2.0 ** k)
        v = vals[np.abs(vals) <= anchor]
        n_tok = -(-len(v) // (31 * per_row))            # 31 value rows + 1 anchor row per block
        pad = np.zeros(n_tok * 31 * per_row - len(v), np.float32)
        body = np.concatenate([v, pad]).reshape(n_tok, 31, per_row)
        blocks = np.concatenate([np.full((n_tok, 1, per_row), anchor, np.float32), body], axis=1)
        rows.append(blocks.reshape(-1, per_row))
        lens.append(blocks.shape[0] * 32)
    x = np.concatenate(rows)[:, None, :]
    t = _bf16(x)
    return Workload(f"e4m3_sweep_{len(lens)}shifts", t, t.clone(), t.clone(), t.clone(), _cu(lens), 1, head_dim)
