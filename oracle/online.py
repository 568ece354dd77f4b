"""Tiled online-softmax attention in float64 (the recurrence the fused kernel runs).

TEST INFRASTRUCTURE ONLY: never imported by the product path.

realizar 0.8.4, src/gguf/inference/forward/attention.rs, IMP-111a
``online_softmax`` and IMP-111b ``tiled_single_head_attention``: for each query
row keep a running maximum m, a running denominator l and a running weighted
sum o; for each key tile take the tile maximum, and when it raises m rescale l
and o by exp(m_old - m_new); then add exp(s - m) and exp(s - m) * v of the tile;
at the end divide o by l.  Here the masks of the boostr pages are added
(masked keys are simply absent from a tile) and the maximum is "safe": a row
that has seen no visible key yet keeps m = -inf and l = 0 and is never rescaled
(the page guards the rescale by a positive running sum for the same reason).

Its pin is equality with the materialised definition in ``attention``, the
same check the realizar page uses its standard implementation for.
"""

from __future__ import annotations

import math

import numpy as np


def tiled_head(qh, kh, vh, causal, window, tile, scale=None):
    """O [Lq, D] and LSE [Lq] of one (sequence, head) by the tiled recurrence."""
    qh, kh, vh = (np.asarray(x, dtype=np.float64) for x in (qh, kh, vh))
    Lq, D = qh.shape
    Lk = kh.shape[0]
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    off = Lk - Lq
    O = np.zeros((Lq, vh.shape[1]))
    LSE = np.full((Lq,), -math.inf)
    for i in range(Lq):
        hi = Lk - 1 if not (causal or window > 0) else min(Lk - 1, i + off)
        lo = 0 if window <= 0 else max(0, i + off - window + 1)
        m, l = -math.inf, 0.0
        o = np.zeros(vh.shape[1])
        for t0 in range(0, Lk, tile):
            js = [j for j in range(t0, min(Lk, t0 + tile)) if lo <= j <= hi]
            if not js:
                continue
            s = np.array([scale * float(qh[i] @ kh[j]) for j in js])
            m_new = max(m, float(s.max()))
            if m_new > m and l > 0.0:
                r = math.exp(m - m_new)
                l *= r
                o *= r
            m = m_new
            w = np.exp(s - m)
            l += float(w.sum())
            o += w @ vh[js]
        if l > 0.0:
            O[i] = o / l
            LSE[i] = m + math.log(l)
    return O, LSE
