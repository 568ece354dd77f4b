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

The FP8 backward (boostr flash.rs, ``flash_attention_bwd_fp8``) takes E4M3
codes with per-tensor dequantisation scales for q, k, v, dout and the forward
output (real value = code value * scale) and per-tensor quantisation scales
for dq, dk, dv.  The page says the output's scale serves the preprocessing
step: the row term sum_k P_ik dP_ik, which equals <dO_i, O_i>, is taken from
the stored output (delta_i = <dO_i, o8_i * o_scale>); everything else is the
gradient above on the dequantised inputs, and each gradient is then encoded
as E4M3(g / g_scale), round to nearest even, saturating at +-448.
"""

from __future__ import annotations

import math
from typing import Iterable

import numpy as np

from . import e4m3 as _e4m3
from .attention import (ROW_BLOCK, _check_heads, _map_units, allowed_keys, as_f64, as_np)


def attend_rows_bwd(qrows: np.ndarray, K: np.ndarray, V: np.ndarray, dOrows: np.ndarray,
                    rows: np.ndarray, Lq: int, Lk: int, causal: bool, window: int,
                    scale: float, Orows: np.ndarray | None = None):
    """Gradients from the query rows ``rows`` of one (sequence, head).

    Returns (dq [n, D] for those rows, dk [Lk, D] and dv [Lk, D] contributions
    of those rows).  Masked scores are -inf, as in the forward oracle.  With
    ``Orows`` (a stored forward output) the row term of the softmax Jacobian
    is <dO_i, O_i> from it instead of sum_k P_ik dP_ik.
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
    if Orows is None:
        delta = (P * dP).sum(axis=1, keepdims=True)
    else:
        delta = (dOrows * Orows).sum(axis=1, keepdims=True)
    dS = P * (dP - delta)
    dq = scale * (dS @ K)
    dk = scale * (dS.T @ qrows)
    return dq, dk, dv


def _bwd_head(qh, kh, vh, doh, causal, window, scale, oh=None):
    Lq, Lk = qh.shape[0], kh.shape[0]
    dq = np.zeros(qh.shape)
    dk = np.zeros(kh.shape)
    dv = np.zeros(vh.shape)
    for r0 in range(0, Lq, ROW_BLOCK):
        r1 = min(Lq, r0 + ROW_BLOCK)
        a, b, c = attend_rows_bwd(qh[r0:r1], kh, vh, doh[r0:r1], np.arange(r0, r1), Lq, Lk,
                                  causal, window, scale, None if oh is None else oh[r0:r1])
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


def flash_attention_bwd_fp8(dout8, q8, k8, v8, o8, num_heads: int, num_kv_heads: int,
                            causal: bool, q_scale: float, k_scale: float, v_scale: float,
                            do_scale: float, o_scale: float, dq_scale: float, dk_scale: float,
                            dv_scale: float, workers: int = 1,
                            heads: Iterable[int] | None = None):
    """FP8 dense backward: returns (dq8, dk8, dv8 uint8 E4M3 codes, dq, dk, dv f64).

    dout8, q8, o8 [B,H,S_q,D] and k8, v8 [B,Hkv,S_k,D] are E4M3 codes; the
    real inputs are code * scale.  The row term uses the stored output
    (o8 * o_scale); the gradients are those of ``flash_attention_bwd`` on the
    dequantised inputs (scale 1/sqrt(D), causal or no mask: the page's FP8
    backward takes no window), quantised as E4M3(g / g_scale).
    """
    for name, s in (("q_scale", q_scale), ("k_scale", k_scale), ("v_scale", v_scale),
                    ("do_scale", do_scale), ("o_scale", o_scale), ("dq_scale", dq_scale),
                    ("dk_scale", dk_scale), ("dv_scale", dv_scale)):
        if not (math.isfinite(s) and s > 0):
            raise ValueError(f"{name} must be finite and positive")
    G = _check_heads(num_heads, num_kv_heads)
    qf = _e4m3.decode(as_np(q8)) * float(q_scale)
    kf = _e4m3.decode(as_np(k8)) * float(k_scale)
    vf = _e4m3.decode(as_np(v8)) * float(v_scale)
    dof = _e4m3.decode(as_np(dout8)) * float(do_scale)
    of = _e4m3.decode(as_np(o8)) * float(o_scale)
    B, H, Sq, D = qf.shape
    if H != num_heads or kf.shape[1] != num_kv_heads or dof.shape != qf.shape or \
            of.shape != qf.shape:
        raise ValueError("shapes do not match the head counts")
    scale = 1.0 / math.sqrt(D)
    dq = np.zeros(qf.shape)
    dk = np.zeros(kf.shape)
    dv = np.zeros(vf.shape)
    heads = list(range(H)) if heads is None else list(heads)

    def unit(b, h):
        kvh = h // G
        return _bwd_head(qf[b, h], kf[b, kvh], vf[b, kvh], dof[b, h], causal, 0, scale,
                         of[b, h])

    units = [(b, h) for b in range(B) for h in heads]
    for b, h, a, c, e in _map_units("dense_bwd_fp8", unit, units, workers):
        dq[b, h] = a
        dk[b, h // G] += c
        dv[b, h // G] += e
    return (_e4m3.encode(dq / dq_scale), _e4m3.encode(dk / dk_scale),
            _e4m3.encode(dv / dv_scale), dq, dk, dv)
