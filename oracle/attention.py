"""The attention forward pass written out from its definition, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.

What is computed (the plain definition; nothing is fused or reordered beyond
evaluating independent query rows in blocks):

  for every sequence b, query head h, kv head  kvh = h // (H / Hkv)
  and query row i in [0, Lq_b):
      s_j   = scale * <q_i, k_j>              j in [0, Lk_b),  scale = 1/sqrt(D)
      A_i   = keys row i may see (mask below)
      m     = max_{j in A_i} s_j
      l     = sum_{j in A_i} exp(s_j - m)
      O_i   = sum_{j in A_i} exp(s_j - m) v_j / l
      LSE_i = m + ln(l)                       (natural log)
      A_i empty  ->  O_i = 0,  LSE_i = -inf

  mask, with off = Lk - Lq (queries are the newest Lq positions of the keys):
      causal        : j <= i + off
      window W > 0  : i + off - W + 1 <= j <= i + off   (exactly W keys; the
                      window implies the causal upper bound)

Sources:
  * packed layout q [total_q, H, D], k/v [total_k, Hkv, D], I32 cu_seqlens,
    GQA map kv_head = q_head / (H / Hkv), output + F32 logsumexp:
    boostr 0.2.0, src/ops/traits/attention/varlen_attention.rs,
    ``VarLenAttentionOps`` ("Layout contract", "GQA key/value head mapping",
    "Cumulative sequence lengths").
  * dense layout q [B,H,S_q,D], k/v [B,Hkv,S_k,D], sliding window ("the most
    recent window_size key positions"), ``kv_seq_len`` (loop bound shorter than
    the dim-2 stride), FP8 per-tensor dequant scales and output quant scale:
    boostr, src/ops/traits/attention/flash.rs, ``FlashAttentionOps``
    ("Layout contract", "GQA support", "Sliding window",
    ``flash_attention_fwd`` / "kv_seq_len", ``flash_attention_fwd_fp8``).
  * scale 1/sqrt(head_dim), max-subtracted softmax exp(x - max)/sum, and the
    materialised scores -> softmax -> weights @ V evaluation:
    realizar 0.8.4, src/gguf/inference/forward/attention.rs, IMP-110
    (``parallel_multihead_attention_gpu``) and IMP-111 (``standard_softmax``,
    ``standard_single_head_attention``).
"""

from __future__ import annotations

import math
import os
from typing import Iterable, Sequence

import numpy as np

from . import e4m3 as _e4m3

ROW_BLOCK = 256


# ---------------------------------------------------------------------------
# inputs
# ---------------------------------------------------------------------------

def cu_seqlens_from_lengths(lengths: Sequence[int]) -> np.ndarray:
    """Exclusive prefix sum of the lengths, I32, with a leading zero.

    boostr 0.2.0 varlen_attention.rs, ``VarLenAttentionOps`` "Cumulative
    sequence lengths": cu[0] = 0 and cu[i] = sum of the lengths of sequences
    0..i-1 (so cu has batch_size + 1 entries).
    """
    cu = [0]
    for n in lengths:
        n = int(n)
        if n < 0:
            raise ValueError("sequence lengths must be non-negative")
        cu.append(cu[-1] + n)
    if cu[-1] > np.iinfo(np.int32).max:
        raise ValueError("total tokens overflow I32")
    return np.asarray(cu, dtype=np.int32)


def as_f64(x) -> np.ndarray:
    """Upcast a stored tensor (torch bf16/f16/f32 or numpy) to float64 exactly."""
    if isinstance(x, np.ndarray):
        return x.astype(np.float64)
    import torch  # torch is only used to read bf16/f16 storage

    if isinstance(x, torch.Tensor):
        x = x.detach().cpu()
        if x.dtype in (torch.bfloat16, torch.float16):
            x = x.to(torch.float32)
        return x.to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def as_np(x) -> np.ndarray:
    if isinstance(x, np.ndarray):
        return x
    try:
        import torch

        if isinstance(x, torch.Tensor):
            return x.detach().cpu().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x)


# ---------------------------------------------------------------------------
# the definition for one (sequence, head)
# ---------------------------------------------------------------------------

def allowed_keys(rows: np.ndarray, Lq: int, Lk: int, causal: bool, window: int) -> np.ndarray:
    """Boolean [len(rows), Lk] mask of the keys each query row may see.

    Causal: key j is visible from row i when j <= i + (Lk - Lq) (queries are
    the most recent Lq positions).  Window W > 0: only the most recent W keys,
    i + off - W + 1 <= j <= i + off (boostr flash.rs, "Sliding window").
    """
    rows = np.asarray(rows, dtype=np.int64)[:, None]
    j = np.arange(Lk, dtype=np.int64)[None, :]
    off = Lk - Lq
    ok = np.ones((rows.shape[0], Lk), dtype=bool)
    if causal or window > 0:
        ok &= j <= rows + off
    if window > 0:
        ok &= j >= rows + off - window + 1
    return ok


def attend_rows(qrows: np.ndarray, K: np.ndarray, V: np.ndarray, rows: np.ndarray,
                Lq: int, Lk: int, causal: bool, window: int, scale: float):
    """O and LSE for the query rows ``rows`` of one (sequence, head).

    qrows [n, D], K/V [Lk, D] are float64.  Scores are materialised, masked
    with -inf (the additive-mask convention of boostr flash.rs
    ``AttentionOps``), and put through the max-subtracted softmax of realizar
    IMP-111a ``standard_softmax``; the weights then multiply V
    (``standard_single_head_attention``).
    """
    n, D = qrows.shape
    if n == 0:
        return np.zeros((0, V.shape[1])), np.zeros((0,))
    if Lk == 0:
        return np.zeros((n, V.shape[1])), np.full((n,), -np.inf)
    s = (qrows @ K.T) * scale
    ok = allowed_keys(rows, Lq, Lk, causal, window)
    s = np.where(ok, s, -np.inf)
    m = s.max(axis=1)
    has = np.isfinite(m)
    m_safe = np.where(has, m, 0.0)
    p = np.exp(s - m_safe[:, None])          # masked entries: exp(-inf) = 0
    l = p.sum(axis=1)
    with np.errstate(invalid="ignore", divide="ignore"):
        O = np.where(has[:, None], (p @ V) / np.where(has, l, 1.0)[:, None], 0.0)
        lse = np.where(has, m_safe + np.log(np.where(has, l, 1.0)), -np.inf)
    return O, lse


def _attend_head(qh: np.ndarray, kh: np.ndarray, vh: np.ndarray, causal: bool,
                 window: int, scale: float):
    Lq, Lk = qh.shape[0], kh.shape[0]
    O = np.zeros((Lq, vh.shape[1]))
    lse = np.full((Lq,), -np.inf)
    for r0 in range(0, Lq, ROW_BLOCK):
        r1 = min(Lq, r0 + ROW_BLOCK)
        O[r0:r1], lse[r0:r1] = attend_rows(qh[r0:r1], kh, vh, np.arange(r0, r1), Lq, Lk,
                                           causal, window, scale)
    return O, lse


def _check_heads(num_heads: int, num_kv_heads: int):
    if num_heads <= 0 or num_kv_heads <= 0 or num_heads % num_kv_heads != 0:
        raise ValueError("num_heads must be a positive multiple of num_kv_heads")
    return num_heads // num_kv_heads


# ---------------------------------------------------------------------------
# work distribution (a process pool over independent (sequence, head) units)
# ---------------------------------------------------------------------------

_SHARED: dict = {}


def _worker_init():
    try:
        from threadpoolctl import threadpool_limits

        threadpool_limits(1)
    except Exception:  # pragma: no cover
        pass


def _run_unit(args):
    kind, b, h = args
    return (b, h) + _SHARED[kind](b, h)


def _map_units(kind: str, fn, units: list, workers: int):
    if workers <= 1 or len(units) <= 1:
        return [(b, h) + fn(b, h) for (b, h) in units]
    import multiprocessing as mp

    _SHARED[kind] = fn
    try:
        ctx = mp.get_context("fork")
        with ctx.Pool(workers, initializer=_worker_init) as pool:
            return pool.map(_run_unit, [(kind, b, h) for (b, h) in units], chunksize=1)
    finally:
        _SHARED.pop(kind, None)


def default_workers() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


# ---------------------------------------------------------------------------
# the three entry points of the pages
# ---------------------------------------------------------------------------

def varlen_attention_fwd(q, k, v, cu_seqlens_q, cu_seqlens_k, num_heads: int,
                         num_kv_heads: int, causal: bool, window: int = 0,
                         scale: float | None = None, workers: int = 1,
                         heads: Iterable[int] | None = None):
    """Packed variable-length forward: returns (O [total_q,H,D], LSE [total_q,H]).

    boostr 0.2.0 varlen_attention.rs, ``varlen_attention_fwd``: q
    [total_q, H, D], k/v [total_k, Hkv, D], sequence b spans rows
    cu[b]..cu[b+1] of q (cu_seqlens_q) and of k/v (cu_seqlens_k).
    ``heads`` restricts the computation to a subset of query heads (rows of the
    other heads stay 0 / -inf); it exists to time bounded samples.
    """
    G = _check_heads(num_heads, num_kv_heads)
    qf, kf, vf = as_f64(q), as_f64(k), as_f64(v)
    cq = as_np(cu_seqlens_q).astype(np.int64)
    ck = as_np(cu_seqlens_k).astype(np.int64)
    T_q, H, D = qf.shape
    if H != num_heads or kf.shape[1] != num_kv_heads:
        raise ValueError("head counts do not match the tensor shapes")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    B = len(cq) - 1
    O = np.zeros(qf.shape)
    lse = np.full((T_q, H), -np.inf)
    heads = list(range(H)) if heads is None else list(heads)

    def unit(b, h):
        kvh = h // G
        qh = qf[cq[b]:cq[b + 1], h, :]
        kh = kf[ck[b]:ck[b + 1], kvh, :]
        vh = vf[ck[b]:ck[b + 1], kvh, :]
        return _attend_head(qh, kh, vh, causal, window, scale)

    units = [(b, h) for b in range(B) for h in heads]
    for b, h, Ob, lb in _map_units("varlen", unit, units, workers):
        O[cq[b]:cq[b + 1], h, :] = Ob
        lse[cq[b]:cq[b + 1], h] = lb
    return O, lse


def flash_attention_fwd(q, k, v, num_heads: int, num_kv_heads: int, causal: bool,
                        window: int = 0, kv_seq_len: int | None = None,
                        scale: float | None = None, workers: int = 1,
                        heads: Iterable[int] | None = None):
    """Dense forward: returns (O [B,H,S_q,D], LSE [B,H,S_q]).

    boostr flash.rs, ``flash_attention_fwd``: q [B,H,S_q,D], k/v
    [B,Hkv,S_k,D]; with ``kv_seq_len = n`` only the first n key positions are
    attended although the buffer holds S_k of them ("kv_seq_len").
    """
    G = _check_heads(num_heads, num_kv_heads)
    qf, kf, vf = as_f64(q), as_f64(k), as_f64(v)
    B, H, Sq, D = qf.shape
    cap = kf.shape[2]
    n = cap if kv_seq_len is None else int(kv_seq_len)
    if n < 0 or n > cap:
        raise ValueError("kv_seq_len exceeds the key buffer")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    O = np.zeros(qf.shape)
    lse = np.full((B, H, Sq), -np.inf)
    heads = list(range(H)) if heads is None else list(heads)

    def unit(b, h):
        kvh = h // G
        return _attend_head(qf[b, h], kf[b, kvh, :n], vf[b, kvh, :n], causal, window, scale)

    units = [(b, h) for b in range(B) for h in heads]
    for b, h, Ob, lb in _map_units("dense", unit, units, workers):
        O[b, h] = Ob
        lse[b, h] = lb
    return O, lse


def flash_attention_fwd_fp8(q8, k8, v8, num_heads: int, num_kv_heads: int, causal: bool,
                            q_scale: float, k_scale: float, v_scale: float, o_scale: float,
                            workers: int = 1, heads: Iterable[int] | None = None):
    """FP8 forward: returns (o8 codes uint8 [B,H,S_q,D], LSE [B,H,S_q], O f64).

    boostr flash.rs, ``flash_attention_fwd_fp8``: q/k/v are E4M3 codes with
    per-tensor dequantisation scales (real = code value * scale); the result is
    computed at full precision and quantised for output with ``o_scale``
    (o8 = E4M3(O / o_scale), round-to-nearest-even, saturating).  LSE is over
    the scaled scores (scale 1/sqrt(D) applied to the dequantised q.k).
    """
    for name, s in (("q_scale", q_scale), ("k_scale", k_scale), ("v_scale", v_scale),
                    ("o_scale", o_scale)):
        if not (math.isfinite(s) and s > 0):
            raise ValueError(f"{name} must be finite and positive")
    qf = _e4m3.decode(as_np(q8)) * float(q_scale)
    kf = _e4m3.decode(as_np(k8)) * float(k_scale)
    vf = _e4m3.decode(as_np(v8)) * float(v_scale)
    O, lse = flash_attention_fwd(qf, kf, vf, num_heads, num_kv_heads, causal,
                                 workers=workers, heads=heads)
    o8 = _e4m3.encode(O / float(o_scale))
    return o8, lse, O


# ---------------------------------------------------------------------------
# single rows (for sampled checks at full size)
# ---------------------------------------------------------------------------

def varlen_rows(q, k, v, cu_seqlens_q, cu_seqlens_k, num_heads: int, num_kv_heads: int,
                causal: bool, samples, window: int = 0, scale: float | None = None):
    """O and LSE for the listed (sequence b, head h, row i) triples only."""
    G = _check_heads(num_heads, num_kv_heads)
    cq = as_np(cu_seqlens_q).astype(np.int64)
    ck = as_np(cu_seqlens_k).astype(np.int64)
    D = q.shape[-1]
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    outs, lses = [], []
    for (b, h, i) in samples:
        kvh = h // G
        Lq, Lk = int(cq[b + 1] - cq[b]), int(ck[b + 1] - ck[b])
        qi = as_f64(q[int(cq[b]) + i, h, :])[None, :]
        K = as_f64(k[int(ck[b]):int(ck[b + 1]), kvh, :])
        V = as_f64(v[int(ck[b]):int(ck[b + 1]), kvh, :])
        o, l = attend_rows(qi, K, V, np.array([i]), Lq, Lk, causal, window, scale)
        outs.append(o[0])
        lses.append(l[0])
    return np.array(outs), np.array(lses)


def dense_rows(q, k, v, num_heads: int, num_kv_heads: int, causal: bool, samples,
               window: int = 0, kv_seq_len: int | None = None, scale: float | None = None):
    """O and LSE for the listed (batch b, head h, row i) triples of the dense layout."""
    G = _check_heads(num_heads, num_kv_heads)
    Sq, D = q.shape[2], q.shape[3]
    n = k.shape[2] if kv_seq_len is None else int(kv_seq_len)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    outs, lses = [], []
    for (b, h, i) in samples:
        kvh = h // G
        qi = as_f64(q[b, h, i, :])[None, :]
        K = as_f64(k[b, kvh, :n, :])
        V = as_f64(v[b, kvh, :n, :])
        o, l = attend_rows(qi, K, V, np.array([i]), Sq, n, causal, window, scale)
        outs.append(o[0])
        lses.append(l[0])
    return np.array(outs), np.array(lses)


def fp8_rows(q8, k8, v8, num_heads: int, num_kv_heads: int, causal: bool, samples,
             q_scale: float, k_scale: float, v_scale: float, o_scale: float):
    """(o8 codes, O f64, LSE) of the listed (batch b, head h, row i) triples of
    the FP8 entry point; only the needed slices are decoded."""
    G = _check_heads(num_heads, num_kv_heads)
    q8, k8, v8 = as_np(q8), as_np(k8), as_np(v8)
    D = q8.shape[3]
    Sq, Sk = q8.shape[2], k8.shape[2]
    scale = 1.0 / math.sqrt(D)
    outs, lses = [], []
    cache = {}
    for (b, h, i) in samples:
        kvh = h // G
        if (b, kvh) not in cache:
            cache[(b, kvh)] = (_e4m3.decode(k8[b, kvh]) * float(k_scale),
                               _e4m3.decode(v8[b, kvh]) * float(v_scale))
        K, V = cache[(b, kvh)]
        qi = (_e4m3.decode(q8[b, h, i]) * float(q_scale))[None, :]
        o, l = attend_rows(qi, K, V, np.array([i]), Sq, Sk, causal, 0, scale)
        outs.append(o[0])
        lses.append(l[0])
    O = np.array(outs)
    return _e4m3.encode(O / float(o_scale)), O, np.array(lses)
