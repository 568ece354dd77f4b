"""The attention backward pass written out from its definition, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.

The pages fix the interface (boostr 0.2.0 varlen_attention.rs,
``varlen_attention_bwd``: dout, q, k, v, the forward output and logsumexp,
cu_seqlens, returning ``(dq, dk, dv)`` with dk/dv shaped like k/v under GQA;
boostr flash.rs, ``flash_attention_bwd``: the dense layout with causal and
sliding-window masks, "gradients with same shapes as inputs") but not the
arithmetic.  What is computed here is the gradient of the forward definition
(``oracle.attention``) for a scalar loss whose gradient with respect to O is
``dout``:

  per sequence, query head h (kv head h // G) and visible pair (i, j):
      P_ij  = exp(s_ij - LSE_i),  s_ij = scale <q_i, k_j>      (softmax weights)
      dv_j  = sum_i P_ij dO_i                                   (O_i = sum_j P_ij v_j)
      dP_ij = <dO_i, v_j>
      dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik)                   (softmax Jacobian)
      dq_i  = scale sum_j dS_ij k_j
      dk_j  = scale sum_i dS_ij q_i
  and dk, dv of a kv head are summed over the G query heads that share it.
  Rows with no visible key contribute nothing.

The weights are recomputed from q and k (max-subtracted softmax, as in the
forward oracle); the forward output and LSE a kernel receives are not used
here, so this is the exact gradient of the exact forward.  It is pinned by
central finite differences of the forward oracle (tests/test_oracle_pins.py).
"""

from __future__ import annotations

import math
from typing import Iterable

import numpy as np

from .attention import (ROW_BLOCK, _check_heads, _map_units, allowed_keys, as_f64, as_np)


def attend_rows_bwd(qrows: np.ndarray, K: np.ndarray, V: np.ndarray, dOrows: np.ndarray,
                    rows: np.ndarray, Lq: int, Lk: int, causal: bool, window: int,
                    scale: float):
    """Gradients from the query rows ``rows`` of one (sequence, head).

    Returns (dq [n, D] for those rows, dk [Lk, D] and dv [Lk, D] contributions
    of those rows).  Masked scores are -inf, as in the forward oracle.
    """
    n, D = qrows.shape
    if n == 0 or Lk == 0:
        return np.zeros((n, D)), np.zeros((Lk, D)), np.zeros((Lk, V.shape[1]))
    s = (qrows @ K.T) * scale
    ok = allowed_keys(rows, Lq, Lk, causal, window)
    s = np.where(ok, s, -np.inf)
    m = s.max(axis=1)
    has = np.isfinite(m)
    p = np.exp(s - np.where(has, m, 0.0)[:, None])     # masked: exp(-inf) = 0
    l = p.sum(axis=1)
    P = p / np.where(has, l, 1.0)[:, None]             # softmax weights (0 on empty rows)
    dv = P.T @ dOrows
    dP = dOrows @ V.T
    dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
    dq = scale * (dS @ K)
    dk = scale * (dS.T @ qrows)
    return dq, dk, dv


def _bwd_head(qh, kh, vh, doh, causal, window, scale):
    Lq, Lk = qh.shape[0], kh.shape[0]
    dq = np.zeros(qh.shape)
    dk = np.zeros(kh.shape)
    dv = np.zeros(vh.shape)
    for r0 in range(0, Lq, ROW_BLOCK):
        r1 = min(Lq, r0 + ROW_BLOCK)
        a, b, c = attend_rows_bwd(qh[r0:r1], kh, vh, doh[r0:r1], np.arange(r0, r1), Lq, Lk,
                                  causal, window, scale)
        dq[r0:r1] = a
        dk += b
        dv += c
    return dq, dk, dv


def varlen_attention_bwd(dout, q, k, v, cu_seqlens_q, cu_seqlens_k, num_heads: int,
                         num_kv_heads: int, causal: bool, window: int = 0,
                         scale: float | None = None, workers: int = 1,
                         heads: Iterable[int] | None = None):
    """Packed variable-length backward: returns (dq [total_q,H,D], dk [total_k,Hkv,D],
    dv [total_k,Hkv,D]) in float64.  ``heads`` restricts the query heads that
    contribute (timing samples)."""
    G = _check_heads(num_heads, num_kv_heads)
    qf, kf, vf, dof = as_f64(q), as_f64(k), as_f64(v), as_f64(dout)
    cq = as_np(cu_seqlens_q).astype(np.int64)
    ck = as_np(cu_seqlens_k).astype(np.int64)
    T_q, H, D = qf.shape
    if H != num_heads or kf.shape[1] != num_kv_heads or dof.shape != qf.shape:
        raise ValueError("shapes do not match the head counts")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    B = len(cq) - 1
    dq = np.zeros(qf.shape)
    dk = np.zeros(kf.shape)
    dv = np.zeros(vf.shape)
    heads = list(range(H)) if heads is None else list(heads)

    def unit(b, h):
        kvh = h // G
        return _bwd_head(qf[cq[b]:cq[b + 1], h], kf[ck[b]:ck[b + 1], kvh],
                         vf[ck[b]:ck[b + 1], kvh], dof[cq[b]:cq[b + 1], h], causal, window,
                         scale)

    units = [(b, h) for b in range(B) for h in heads]
    for b, h, a, c, e in _map_units("varlen_bwd", unit, units, workers):
        dq[cq[b]:cq[b + 1], h] = a
        dk[ck[b]:ck[b + 1], h // G] += c
        dv[ck[b]:ck[b + 1], h // G] += e
    return dq, dk, dv


def flash_attention_bwd(dout, q, k, v, num_heads: int, num_kv_heads: int, causal: bool,
                        window: int = 0, scale: float | None = None, workers: int = 1,
                        heads: Iterable[int] | None = None):
    """Dense backward: returns (dq [B,H,S_q,D], dk [B,Hkv,S_k,D], dv [B,Hkv,S_k,D]) in
    float64.  All S_k keys of k/v are attended (the backward of the pages takes no
    kv_seq_len)."""
    G = _check_heads(num_heads, num_kv_heads)
    qf, kf, vf, dof = as_f64(q), as_f64(k), as_f64(v), as_f64(dout)
    B, H, Sq, D = qf.shape
    if H != num_heads or kf.shape[1] != num_kv_heads or dof.shape != qf.shape:
        raise ValueError("shapes do not match the head counts")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    dq = np.zeros(qf.shape)
    dk = np.zeros(kf.shape)
    dv = np.zeros(vf.shape)
    heads = list(range(H)) if heads is None else list(heads)

    def unit(b, h):
        kvh = h // G
        return _bwd_head(qf[b, h], kf[b, kvh], vf[b, kvh], dof[b, h], causal, window, scale)

    units = [(b, h) for b in range(B) for h in heads]
    for b, h, a, c, e in _map_units("dense_bwd", unit, units, workers):
        dq[b, h] = a
        dk[b, h // G] += c
        dv[b, h // G] += e
    return dq, dk, dv
