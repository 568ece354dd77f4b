"""Packing of padded batches into the varlen layout, written out plainly.

TEST INFRASTRUCTURE ONLY (see the package docstring).

boostr 0.2.0 varlen_attention.rs ("Variable-length Flash Attention"): sequences
of different lengths are packed into one buffer instead of being padded, and
sequence b occupies rows cu_seqlens[b] .. cu_seqlens[b+1] ("Cumulative sequence
lengths": cu_seqlens[0] = 0, cu_seqlens[i] = sum of the lengths of sequences
0..i-1).  The offsets are those of a CSR layout, built as a cumulative sum with
a leading zero (boostr's MoE dispatch page builds its expert offsets the same
way).  Pure data movement: every result here is exact.
"""

from __future__ import annotations

import numpy as np

from .attention import cu_seqlens_from_lengths  # noqa: F401  (the prefix sum)


def pack(padded: np.ndarray, lengths) -> np.ndarray:
    """padded [B, S, ...] -> packed [sum(lengths), ...]: row s < lengths[b] of
    sequence b goes to row cu[b] + s."""
    padded = np.asarray(padded)
    lengths = [int(n) for n in lengths]
    if len(lengths) != padded.shape[0]:
        raise ValueError("one length per batch entry")
    if any(n < 0 or n > padded.shape[1] for n in lengths):
        raise ValueError("lengths must lie in [0, S]")
    return np.concatenate([padded[b, :n] for b, n in enumerate(lengths)]
                          + [np.zeros((0,) + padded.shape[2:], padded.dtype)], axis=0)


def unpack(packed: np.ndarray, cu_seqlens, max_seqlen: int) -> np.ndarray:
    """packed [T, ...] -> padded [B, max_seqlen, ...] with zeros after each
    sequence's last row (the inverse of ``pack`` on the valid rows)."""
    packed = np.asarray(packed)
    cu = [int(c) for c in np.asarray(cu_seqlens)]
    B = len(cu) - 1
    out = np.zeros((B, max_seqlen) + packed.shape[1:], packed.dtype)
    for b in range(B):
        n = cu[b + 1] - cu[b]
        if n < 0 or n > max_seqlen:
            raise ValueError("sequence lengths must lie in [0, max_seqlen]")
        out[b, :n] = packed[cu[b]:cu[b + 1]]
    return out
