"""Longest-first work list of the packed call (oracle; test infrastructure).

The pages build the schedule once per microbatch on the GPU: items are sorted
by cost, longest first, and handed to a persistent grid; skewed loads (longest
document at least 4x the mean) fetch work dynamically
([Summary, §3.6.2 Load-Balanced Scheduling]; [Reading, 4.4], last bullet).
The cost model and tie-break are not given; the reading taken
here:

* forward item = (document, query tile t, head); cost = number of key tiles
  the causal query tile touches: ``floor((min((t+1)*Bq, L) - 1) / Bk) + 1``;
* backward item = (document, key tile u, head); cost = number of query tiles
  at or after the key tile: ``ceil(L/Bq) - floor(u*Bk/Bq)``;
* both lists: cost descending, then document, tile, head ascending (the
  pages sort the work items by cost, costliest first).
Every key is unique, so exactly one order is correct.
"""

from __future__ import annotations

from .quant import doc_bounds


def _cdiv(a: int, b: int) -> int:
    return -(-a // b)


def fwd_cost(t: int, L: int, bq: int, bk: int, causal: bool = True) -> int:
    if not causal:
        return _cdiv(L, bk)
    return (min((t + 1) * bq, L) - 1) // bk + 1


def bwd_cost(u: int, L: int, bq: int, bk: int, causal: bool = True) -> int:
    if not causal:
        return _cdiv(L, bq)
    return _cdiv(L, bq) - (u * bk) // bq


def fwd_items(cu_seqlens, heads: int, bq: int, bk: int, causal: bool = True):
    """Sorted forward work list as (doc, tile, head, cost) tuples."""
    items = []
    for doc, (s, e) in enumerate(doc_bounds(cu_seqlens)):
        L = e - s
        for t in range(_cdiv(L, bq)):
            c = fwd_cost(t, L, bq, bk, causal)
            items.extend((doc, t, h, c) for h in range(heads))
    return sorted(items, key=lambda it: (-it[3], it[0], it[1], it[2]))


def bwd_items(cu_seqlens, heads: int, bq: int, bk: int, causal: bool = True):
    """Sorted backward work list as (doc, key tile, head, cost) tuples."""
    items = []
    for doc, (s, e) in enumerate(doc_bounds(cu_seqlens)):
        L = e - s
        for u in range(_cdiv(L, bk)):
            c = bwd_cost(u, L, bq, bk, causal)
            items.extend((doc, u, h, c) for h in range(heads))
    return sorted(items, key=lambda it: (-it[3], it[0], it[1], it[2]))


def is_skewed(cu_seqlens) -> bool:
    """Skew test of the pages: longest document >= 4 x the mean length."""
    lens = [e - s for s, e in doc_bounds(cu_seqlens)]
    if not lens or sum(lens) == 0:
        return False
    return max(lens) * len(lens) >= 4 * sum(lens)
