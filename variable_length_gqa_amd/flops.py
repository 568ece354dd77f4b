"""Algorithmic work of the attention forward pass.

A (query, key) pair is "visible" when the key is inside the query row's mask
(causal: key position <= query position, with the queries aligned to the end
of the keys; window W: only the W most recent keys).  Each visible pair costs
2*D multiply-adds in Q.K^T and 2*D in P.V, i.e. 4*D floating-point operations
per head; masked pairs inside computed tiles and skipped tiles do not count.
"""

from __future__ import annotations

import numpy as np


def visible_pairs(Lq: int, Lk: int, causal: bool, window: int = 0) -> int:
    """Number of (query, key) pairs one head of one sequence attends to."""
    if Lq <= 0 or Lk <= 0:
        return 0
    i = np.arange(Lq, dtype=np.int64)
    off = Lk - Lq
    if causal or window > 0:
        hi = np.minimum(Lk - 1, i + off)
    else:
        hi = np.full(Lq, Lk - 1, dtype=np.int64)
    if window > 0:
        lo = np.maximum(0, i + off - window + 1)
    else:
        lo = np.zeros(Lq, dtype=np.int64)
    return int(np.maximum(0, hi - lo + 1).sum())


def attention_flops(lengths_q, lengths_k, num_heads: int, head_dim: int, causal: bool,
                    window: int = 0) -> int:
    """4*D FLOPs per visible pair, summed over sequences and query heads."""
    pairs = sum(visible_pairs(a, b, causal, window) for a, b in zip(lengths_q, lengths_k))
    return 4 * head_dim * num_heads * pairs


def io_bytes(total_q: int, total_k: int, num_heads: int, num_kv_heads: int, head_dim: int,
             elem_bytes: int, out_bytes: int | None = None) -> int:
    """Q, K, V read once, O and the F32 LSE written once."""
    ob = elem_bytes if out_bytes is None else out_bytes
    return (total_q * num_heads * head_dim * (elem_bytes + ob)
            + 2 * total_k * num_kv_heads * head_dim * elem_bytes
            + total_q * num_heads * 4)


def visible_key_span(Lq: int, Lk: int, causal: bool, window: int = 0) -> int:
    """Number of key positions visible to at least one query row: the keys a
    pass that reads each needed K/V row once must fetch."""
    if Lq <= 0 or Lk <= 0:
        return 0
    off = Lk - Lq
    hi = min(Lk - 1, Lq - 1 + off) if (causal or window > 0) else Lk - 1
    lo = max(0, off - window + 1) if window > 0 else 0
    return max(0, hi - lo + 1)
