"""Pure-Python brute force for tiny inputs (math.fsum, no NumPy arithmetic).

TEST INFRASTRUCTURE ONLY: never imported by the product path.

An independent second writing of the definition, used to pin the NumPy oracle
on tiny ragged inputs.  It does not reuse the mask helper of ``attention``: the
visibility rule is spelled out again here, row by row.

Sources: realizar 0.8.4, src/gguf/inference/forward/attention.rs, IMP-111b
``standard_single_head_attention`` (dot products, scale, per-row softmax,
weighted sum of V) with the max-subtracted softmax of IMP-111a
``standard_softmax``; masks and head mapping as in boostr varlen_attention.rs
(``VarLenAttentionOps``) and boostr flash.rs ("Sliding window").
"""

from __future__ import annotations

import math


def attention_one_row(qi, keys, values, visible, scale):
    """Softmax-weighted mean of ``values`` over the ``visible`` key indices.

    Returns (o: list[float], lse: float); an empty visible set gives zeros and
    -inf.
    """
    D = len(values[0]) if values else len(qi)
    if not visible:
        return [0.0] * D, -math.inf
    scores = {j: scale * math.fsum(qi[d] * keys[j][d] for d in range(len(qi))) for j in visible}
    m = max(scores.values())
    w = {j: math.exp(scores[j] - m) for j in visible}
    l = math.fsum(w.values())
    o = [math.fsum(w[j] * values[j][d] for j in visible) / l for d in range(D)]
    return o, m + math.log(l)


def visible_keys(i, Lq, Lk, causal, window):
    """Key indices row i may attend to, listed one by one."""
    last = i + (Lk - Lq)  # the query's own position among the keys
    out = []
    for j in range(Lk):
        if (causal or window > 0) and j > last:
            continue
        if window > 0 and j < last - window + 1:
            continue
        out.append(j)
    return out


def varlen(q, k, v, lengths_q, lengths_k, num_heads, num_kv_heads, causal, window=0,
           scale=None):
    """Nested-list varlen attention: q[t][h][d], k/v[t][kvh][d] -> (O, LSE)."""
    G = num_heads // num_kv_heads
    D = len(q[0][0]) if q else len(k[0][0])
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    O = [[[0.0] * D for _ in range(num_heads)] for _ in range(len(q))]
    LSE = [[-math.inf] * num_heads for _ in range(len(q))]
    sq = sk = 0
    for Lq, Lk in zip(lengths_q, lengths_k):
        for h in range(num_heads):
            kvh = h // G
            keys = [k[sk + j][kvh] for j in range(Lk)]
            vals = [v[sk + j][kvh] for j in range(Lk)]
            for i in range(Lq):
                o, l = attention_one_row(q[sq + i][h], keys, vals,
                                         visible_keys(i, Lq, Lk, causal, window), scale)
                O[sq + i][h] = o
                LSE[sq + i][h] = l
        sq += Lq
        sk += Lk
    return O, LSE
