"""Python entry points over the C ABI: argument marshalling only.

Each function checks shapes and dtypes, allocates ``out`` / ``lse`` with torch
(unless given), and enqueues the HIP kernel on torch's current stream.  Every
step of the computation runs in the HIP library; there is no other path.

Argument order follows the pages' signatures:
  * boostr 0.2.0, src/ops/traits/attention/varlen_attention.rs,
    ``VarLenAttentionOps::varlen_attention_fwd``
  * boostr, src/ops/traits/attention/flash.rs,
    ``FlashAttentionOps::flash_attention_fwd`` / ``flash_attention_fwd_fp8``
The forwards return ``(output, logsumexp)``; the backwards
(``VarLenAttentionOps::varlen_attention_bwd``,
``FlashAttentionOps::flash_attention_bwd`` / ``flash_attention_bwd_fp8``)
return ``(dq, dk, dv)``.
"""

from __future__ import annotations

import os

import torch

from . import _lib

_DTYPE_CODE = {torch.float32: _lib.VLGQA_F32, torch.float16: _lib.VLGQA_F16,
               torch.bfloat16: _lib.VLGQA_BF16}

DEBUG_CHECKS = os.environ.get("VLGQA_DEBUG_CHECKS", "0") not in ("", "0")


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _need(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def _check_device_tensor(name: str, t: torch.Tensor, device):
    _need(isinstance(t, torch.Tensor), f"{name} must be a torch.Tensor")
    _need(t.is_cuda, f"{name} must be a GPU tensor")
    _need(t.device == device, f"{name} is on {t.device}, expected {device}")
    _need(t.is_contiguous(), f"{name} must be contiguous")


def check_cu_seqlens(cu: torch.Tensor, total: int, max_seqlen: int, name: str):
    """Host-side validation of cu_seqlens (copies it to the host; debug use)."""
    c = cu.detach().to("cpu", torch.int64).tolist()
    _need(len(c) >= 1 and c[0] == 0, f"{name}[0] must be 0")
    _need(all(b >= a for a, b in zip(c, c[1:])), f"{name} must be non-decreasing")
    _need(c[-1] == total, f"{name}[-1] = {c[-1]} must equal the packed token count {total}")
    _need(all(b - a <= max_seqlen for a, b in zip(c, c[1:])),
          f"a sequence in {name} is longer than its max_seqlen {max_seqlen}")


def varlen_attention_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                         cu_seqlens_q: torch.Tensor, cu_seqlens_k: torch.Tensor,
                         batch_size: int, num_heads: int, num_kv_heads: int,
                         max_seqlen_q: int, max_seqlen_k: int, head_dim: int, causal: bool,
                         out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                         check_seqlens: bool | None = None):
    """Packed variable-length attention forward -> (out [total_q,H,D], lse [total_q,H] f32)."""
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("cu_seqlens_q", cu_seqlens_q),
                    ("cu_seqlens_k", cu_seqlens_k)):
        _check_device_tensor(name, t, dev)
    _need(q.dtype in _DTYPE_CODE, f"unsupported dtype {q.dtype}")
    _need(k.dtype == q.dtype and v.dtype == q.dtype, "q, k and v must share one dtype")
    _need(cu_seqlens_q.dtype == torch.int32 and cu_seqlens_k.dtype == torch.int32,
          "cu_seqlens must be int32")
    _need(q.dim() == 3 and q.shape[1] == num_heads and q.shape[2] == head_dim,
          "q must be [total_q, num_heads, head_dim]")
    _need(k.dim() == 3 and k.shape[1] == num_kv_heads and k.shape[2] == head_dim,
          "k must be [total_k, num_kv_heads, head_dim]")
    _need(v.shape == k.shape, "v must have the shape of k")
    _need(cu_seqlens_q.numel() == batch_size + 1 and cu_seqlens_k.numel() == batch_size + 1,
          "cu_seqlens must have batch_size + 1 entries")
    total_q, total_k = q.shape[0], k.shape[0]
    if check_seqlens if check_seqlens is not None else DEBUG_CHECKS:
        check_cu_seqlens(cu_seqlens_q, total_q, max_seqlen_q, "cu_seqlens_q")
        check_cu_seqlens(cu_seqlens_k, total_k, max_seqlen_k, "cu_seqlens_k")
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((total_q, num_heads), dtype=torch.float32, device=dev)
    _check_device_tensor("out", out, dev)
    _check_device_tensor("lse", lse, dev)
    _need(out.shape == q.shape and out.dtype == q.dtype, "out must match q")
    _need(lse.shape == (total_q, num_heads) and lse.dtype == torch.float32,
          "lse must be float32 [total_q, num_heads]")
    lib = _lib.load()
    rc = lib.varlen_attention_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens_q),
                                  _ptr(cu_seqlens_k), total_q, total_k, batch_size, num_heads,
                                  num_kv_heads, max_seqlen_q, max_seqlen_k, head_dim,
                                  int(bool(causal)), _DTYPE_CODE[q.dtype], _ptr(out), _ptr(lse),
                                  _stream(dev))
    _lib.check(rc)
    return out, lse


def flash_attention_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, num_heads: int,
                        num_kv_heads: int, head_dim: int, causal: bool, window_size: int = 0,
                        kv_seq_len: int | None = None, out: torch.Tensor | None = None,
                        lse: torch.Tensor | None = None):
    """Dense attention forward -> (out [B,H,S_q,D], lse [B,H,S_q] f32).

    k/v are [B, Hkv, capacity, D]; ``kv_seq_len`` attends to the first n key
    positions only, using dim 2 as the memory stride (None = all of them).
    """
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_device_tensor(name, t, dev)
    _need(q.dtype in _DTYPE_CODE, f"unsupported dtype {q.dtype}")
    _need(k.dtype == q.dtype and v.dtype == q.dtype, "q, k and v must share one dtype")
    _need(q.dim() == 4 and q.shape[1] == num_heads and q.shape[3] == head_dim,
          "q must be [B, num_heads, S_q, head_dim]")
    _need(k.dim() == 4 and k.shape[0] == q.shape[0] and k.shape[1] == num_kv_heads
          and k.shape[3] == head_dim, "k must be [B, num_kv_heads, S_k, head_dim]")
    _need(v.shape == k.shape, "v must have the shape of k")
    _need(window_size >= 0, "window_size must be non-negative")
    B, _, Sq, _ = q.shape
    cap = k.shape[2]
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, num_heads, Sq), dtype=torch.float32, device=dev)
    _check_device_tensor("out", out, dev)
    _check_device_tensor("lse", lse, dev)
    _need(out.shape == q.shape and out.dtype == q.dtype, "out must match q")
    _need(lse.shape == (B, num_heads, Sq) and lse.dtype == torch.float32,
          "lse must be float32 [B, num_heads, S_q]")
    lib = _lib.load()
    rc = lib.flash_attention_fwd(_ptr(q), _ptr(k), _ptr(v), B, num_heads, num_kv_heads, Sq, cap,
                                 head_dim, int(bool(causal)), int(window_size),
                                 -1 if kv_seq_len is None else int(kv_seq_len),
                                 _DTYPE_CODE[q.dtype], _ptr(out), _ptr(lse), _stream(dev))
    _lib.check(rc)
    return out, lse


def decode_workspace_floats(batch: int, num_kv_heads: int, head_dim: int, kv_len: int) -> int:
    """Float32 workspace ``flash_attention_decode`` needs for ``kv_len`` attended keys."""
    n = _lib.load().vlgqa_decode_workspace_floats(batch, num_kv_heads, head_dim, kv_len)
    _need(n >= 0, "negative extent")
    return int(n)


def flash_attention_decode(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, num_heads: int,
                           num_kv_heads: int, head_dim: int, causal: bool, window_size: int = 0,
                           kv_seq_len: int | None = None, out: torch.Tensor | None = None,
                           lse: torch.Tensor | None = None,
                           workspace: torch.Tensor | None = None):
    """Split-KV dense forward for decode shapes -> (out, lse), as flash_attention_fwd.

    Requires S_q * num_heads / num_kv_heads <= 32.  ``workspace`` (float32, at
    least ``decode_workspace_floats(B, Hkv, D, n)`` elements) is allocated when
    not given; a caller decoding step by step can size one for the capacity.
    """
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_device_tensor(name, t, dev)
    _need(q.dtype in (torch.bfloat16, torch.float16), f"unsupported dtype {q.dtype}")
    _need(k.dtype == q.dtype and v.dtype == q.dtype, "q, k and v must share one dtype")
    _need(q.dim() == 4 and q.shape[1] == num_heads and q.shape[3] == head_dim,
          "q must be [B, num_heads, S_q, head_dim]")
    _need(k.dim() == 4 and k.shape[0] == q.shape[0] and k.shape[1] == num_kv_heads
          and k.shape[3] == head_dim, "k must be [B, num_kv_heads, capacity, head_dim]")
    _need(v.shape == k.shape, "v must have the shape of k")
    B, _, Sq, _ = q.shape
    cap = k.shape[2]
    n = cap if kv_seq_len is None else int(kv_seq_len)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, num_heads, Sq), dtype=torch.float32, device=dev)
    _check_device_tensor("out", out, dev)
    _check_device_tensor("lse", lse, dev)
    _need(out.shape == q.shape and out.dtype == q.dtype, "out must match q")
    _need(lse.shape == (B, num_heads, Sq) and lse.dtype == torch.float32,
          "lse must be float32 [B, num_heads, S_q]")
    need = decode_workspace_floats(B, num_kv_heads, head_dim, max(n, 0))
    if workspace is None:
        workspace = torch.empty(max(need, 4), dtype=torch.float32, device=dev)
    _check_device_tensor("workspace", workspace, dev)
    _need(workspace.dtype == torch.float32, "workspace must be float32")
    lib = _lib.load()
    rc = lib.flash_attention_decode(_ptr(q), _ptr(k), _ptr(v), B, num_heads, num_kv_heads, Sq,
                                    cap, head_dim, int(bool(causal)), int(window_size),
                                    -1 if kv_seq_len is None else int(kv_seq_len),
                                    _DTYPE_CODE[q.dtype], _ptr(out), _ptr(lse), _ptr(workspace),
                                    workspace.numel(), _stream(dev))
    _lib.check(rc)
    return out, lse


def flash_attention_decode_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                                   num_heads: int, num_kv_heads: int, head_dim: int, causal: bool,
                                   window_size: int, kv_seq_len: int | None, out: torch.Tensor,
                                   lse: torch.Tensor):
    """flash_attention_decode for callers that cannot allocate: the split-KV
    partials go to the library's static per-GPU scratch instead of a workspace,
    and ``out`` / ``lse`` must be given (nothing is allocated here either).
    Calls that overlap on one GPU share that scratch and race: order them."""
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out), ("lse", lse)):
        _check_device_tensor(name, t, dev)
    _need(q.dtype in (torch.bfloat16, torch.float16), f"unsupported dtype {q.dtype}")
    _need(k.dtype == q.dtype and v.dtype == q.dtype, "q, k and v must share one dtype")
    _need(q.dim() == 4 and q.shape[1] == num_heads and q.shape[3] == head_dim,
          "q must be [B, num_heads, S_q, head_dim]")
    _need(k.dim() == 4 and k.shape[0] == q.shape[0] and k.shape[1] == num_kv_heads
          and k.shape[3] == head_dim, "k must be [B, num_kv_heads, capacity, head_dim]")
    _need(v.shape == k.shape, "v must have the shape of k")
    B, _, Sq, _ = q.shape
    _need(out.shape == q.shape and out.dtype == q.dtype, "out must match q")
    _need(lse.shape == (B, num_heads, Sq) and lse.dtype == torch.float32,
          "lse must be float32 [B, num_heads, S_q]")
    lib = _lib.load()
    rc = lib.flash_attention_decode_noalloc(_ptr(q), _ptr(k), _ptr(v), B, num_heads, num_kv_heads,
                                            Sq, k.shape[2], head_dim, int(bool(causal)),
                                            int(window_size),
                                            -1 if kv_seq_len is None else int(kv_seq_len),
                                            _DTYPE_CODE[q.dtype], _ptr(out), _ptr(lse),
                                            _stream(dev))
    _lib.check(rc)
    return out, lse


def flash_attention_fwd_fp8(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, num_heads: int,
                            num_kv_heads: int, head_dim: int, causal: bool, q_scale: float,
                            k_scale: float, v_scale: float, o_scale: float,
                            out: torch.Tensor | None = None, lse: torch.Tensor | None = None):
    """FP8 (OCP E4M3 codes, uint8 or float8_e4m3fn tensors) dense forward.

    Returns (out uint8 E4M3 codes [B,H,S_q,D], lse [B,H,S_q] f32).
    """
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_device_tensor(name, t, dev)
    ok = (torch.uint8, torch.float8_e4m3fn)
    _need(q.dtype in ok and k.dtype in ok and v.dtype in ok,
          "fp8 inputs must be uint8 or float8_e4m3fn (OCP E4M3 codes)")
    _need(q.dim() == 4 and q.shape[1] == num_heads and q.shape[3] == head_dim,
          "q must be [B, num_heads, S_q, head_dim]")
    _need(k.dim() == 4 and k.shape[0] == q.shape[0] and k.shape[1] == num_kv_heads
          and k.shape[3] == head_dim, "k must be [B, num_kv_heads, S_k, head_dim]")
    _need(v.shape == k.shape, "v must have the shape of k")
    B, _, Sq, _ = q.shape
    if out is None:
        out = torch.empty(q.shape, dtype=torch.uint8, device=dev)
    if lse is None:
        lse = torch.empty((B, num_heads, Sq), dtype=torch.float32, device=dev)
    _check_device_tensor("out", out, dev)
    _check_device_tensor("lse", lse, dev)
    _need(out.shape == q.shape and out.dtype in ok, "out must be a [B,H,S_q,D] fp8 buffer")
    _need(lse.shape == (B, num_heads, Sq) and lse.dtype == torch.float32,
          "lse must be float32 [B, num_heads, S_q]")
    lib = _lib.load()
    rc = lib.flash_attention_fwd_fp8(_ptr(q), _ptr(k), _ptr(v), B, num_heads, num_kv_heads, Sq,
                                     k.shape[2], head_dim, int(bool(causal)), float(q_scale),
                                     float(k_scale), float(v_scale), float(o_scale), _ptr(out),
                                     _ptr(lse), _stream(dev))
    _lib.check(rc)
    return out, lse


_BWD_DTYPES = (torch.bfloat16, torch.float16)


def _check_bwd_common(dout, q, k, v, out, lse, dev):
    for name, t in (("dout", dout), ("q", q), ("k", k), ("v", v), ("out", out), ("lse", lse)):
        _check_device_tensor(name, t, dev)
    _need(q.dtype in _BWD_DTYPES, f"the backward supports bf16 and f16, not {q.dtype}")
    _need(k.dtype == q.dtype and v.dtype == q.dtype and dout.dtype == q.dtype
          and out.dtype == q.dtype, "dout, q, k, v and out must share one dtype")
    _need(dout.shape == q.shape and out.shape == q.shape, "dout and out must have the shape of q")
    _need(v.shape == k.shape, "v must have the shape of k")
    _need(lse.dtype == torch.float32, "lse must be float32")


def bwd_workspace_floats(rows: int, keys: int, num_heads: int, num_kv_heads: int,
                         head_dim: int, e4m3: bool = False) -> int:
    """float32 elements of the backward workspace (the library's own count)."""
    n = _lib.load().vlgqa_bwd_workspace_floats(rows, keys, num_heads, num_kv_heads, head_dim,
                                               int(bool(e4m3)))
    _need(n >= 0, "negative extent")
    return int(n)


def _bwd_outputs(q, k, v, dq, dk, dv, ws, ws_floats, dev):
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if ws is None:
        ws = torch.empty((max(ws_floats, 4),), dtype=torch.float32, device=dev)
    for name, t, like in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        _check_device_tensor(name, t, dev)
        _need(t.shape == like.shape and t.dtype == like.dtype, f"{name} must match its input")
    _check_device_tensor("workspace", ws, dev)
    _need(ws.dtype == torch.float32 and ws.numel() >= ws_floats,
          f"workspace must be float32 with at least {ws_floats} elements")
    return dq, dk, dv, ws


def varlen_attention_bwd(dout: torch.Tensor, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                         output: torch.Tensor, lse: torch.Tensor, cu_seqlens_q: torch.Tensor,
                         cu_seqlens_k: torch.Tensor, batch_size: int, num_heads: int,
                         num_kv_heads: int, max_seqlen_q: int, max_seqlen_k: int, head_dim: int,
                         causal: bool, check_seqlens: bool | None = None,
                         dq: torch.Tensor | None = None, dk: torch.Tensor | None = None,
                         dv: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """Packed variable-length attention backward -> (dq [total_q,H,D], dk, dv [total_k,Hkv,D]).

    ``output`` and ``lse`` are the forward's results for the same inputs.
    dq / dk / dv / workspace (float32, ``bwd_workspace_floats(total_q, total_k,
    ...)`` elements) may be passed preallocated.
    """
    dev = q.device
    _check_bwd_common(dout, q, k, v, output, lse, dev)
    for name, t in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        _check_device_tensor(name, t, dev)
    _need(cu_seqlens_q.dtype == torch.int32 and cu_seqlens_k.dtype == torch.int32,
          "cu_seqlens must be int32")
    _need(q.dim() == 3 and q.shape[1] == num_heads and q.shape[2] == head_dim,
          "q must be [total_q, num_heads, head_dim]")
    _need(k.dim() == 3 and k.shape[1] == num_kv_heads and k.shape[2] == head_dim,
          "k must be [total_k, num_kv_heads, head_dim]")
    _need(cu_seqlens_q.numel() == batch_size + 1 and cu_seqlens_k.numel() == batch_size + 1,
          "cu_seqlens must have batch_size + 1 entries")
    total_q, total_k = q.shape[0], k.shape[0]
    _need(lse.shape == (total_q, num_heads), "lse must be [total_q, num_heads]")
    if check_seqlens if check_seqlens is not None else DEBUG_CHECKS:
        check_cu_seqlens(cu_seqlens_q, total_q, max_seqlen_q, "cu_seqlens_q")
        check_cu_seqlens(cu_seqlens_k, total_k, max_seqlen_k, "cu_seqlens_k")
    dq, dk, dv, ws = _bwd_outputs(q, k, v, dq, dk, dv, workspace,
                                  bwd_workspace_floats(total_q, total_k, num_heads,
                                                       num_kv_heads, head_dim), dev)
    lib = _lib.load()
    rc = lib.varlen_attention_bwd(_ptr(dout), _ptr(q), _ptr(k), _ptr(v), _ptr(output), _ptr(lse),
                                  _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), total_q, total_k,
                                  batch_size, num_heads, num_kv_heads, max_seqlen_q,
                                  max_seqlen_k, head_dim, int(bool(causal)),
                                  _DTYPE_CODE[q.dtype], _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws),
                                  _stream(dev))
    _lib.check(rc)
    return dq, dk, dv


def flash_attention_bwd(dout: torch.Tensor, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                        output: torch.Tensor, lse: torch.Tensor, num_heads: int,
                        num_kv_heads: int, head_dim: int, causal: bool, window_size: int = 0,
                        dq: torch.Tensor | None = None, dk: torch.Tensor | None = None,
                        dv: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """Dense attention backward -> (dq [B,H,S_q,D], dk, dv [B,Hkv,S_k,D]).

    All S_k keys of k/v are attended (the pages' backward takes no kv_seq_len).
    dq / dk / dv / workspace (float32, ``bwd_workspace_floats(B * S_q, B * S_k,
    ...)`` elements) may be passed preallocated.
    """
    dev = q.device
    _check_bwd_common(dout, q, k, v, output, lse, dev)
    _need(q.dim() == 4 and q.shape[1] == num_heads and q.shape[3] == head_dim,
          "q must be [B, num_heads, S_q, head_dim]")
    _need(k.dim() == 4 and k.shape[0] == q.shape[0] and k.shape[1] == num_kv_heads
          and k.shape[3] == head_dim, "k must be [B, num_kv_heads, S_k, head_dim]")
    _need(window_size >= 0, "window_size must be non-negative")
    B, _, Sq, _ = q.shape
    Sk = k.shape[2]
    _need(lse.shape == (B, num_heads, Sq), "lse must be [B, num_heads, S_q]")
    dq, dk, dv, ws = _bwd_outputs(q, k, v, dq, dk, dv, workspace,
                                  bwd_workspace_floats(B * Sq, B * Sk, num_heads, num_kv_heads,
                                                       head_dim), dev)
    lib = _lib.load()
    rc = lib.flash_attention_bwd(_ptr(dout), _ptr(q), _ptr(k), _ptr(v), _ptr(output), _ptr(lse),
                                 B, num_heads, num_kv_heads, Sq, Sk, head_dim,
                                 int(bool(causal)), int(window_size), _DTYPE_CODE[q.dtype],
                                 _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws), _stream(dev))
    _lib.check(rc)
    return dq, dk, dv


def flash_attention_bwd_fp8(dout: torch.Tensor, q: torch.Tensor, k: torch.Tensor,
                            v: torch.Tensor, output: torch.Tensor, lse: torch.Tensor,
                            num_heads: int, num_kv_heads: int, head_dim: int, causal: bool,
                            q_scale: float, k_scale: float, v_scale: float, do_scale: float,
                            o_scale: float, dq_scale: float, dk_scale: float, dv_scale: float,
                            dq: torch.Tensor | None = None, dk: torch.Tensor | None = None,
                            dv: torch.Tensor | None = None,
                            workspace: torch.Tensor | None = None):
    """FP8 (E4M3 codes as uint8) dense backward -> (dq8, dk8, dv8) uint8 codes.

    Inputs are codes with dequantisation scales (real = code * scale); the
    gradients come back as E4M3(g / g_scale).  ``lse`` is the FP8 forward's.
    """
    dev = q.device
    for name, t in (("dout", dout), ("q", q), ("k", k), ("v", v), ("output", output),
                    ("lse", lse)):
        _check_device_tensor(name, t, dev)
    for name, t in (("dout", dout), ("q", q), ("k", k), ("v", v), ("output", output)):
        _need(t.dtype == torch.uint8, f"{name} must hold E4M3 codes as uint8")
    _need(q.dim() == 4 and q.shape[1] == num_heads and q.shape[3] == head_dim,
          "q must be [B, num_heads, S_q, head_dim]")
    _need(k.dim() == 4 and k.shape[0] == q.shape[0] and k.shape[1] == num_kv_heads
          and k.shape[3] == head_dim, "k must be [B, num_kv_heads, S_k, head_dim]")
    _need(v.shape == k.shape, "v must have the shape of k")
    _need(dout.shape == q.shape and output.shape == q.shape,
          "dout and output must have the shape of q")
    B, _, Sq, _ = q.shape
    Sk = k.shape[2]
    _need(lse.dtype == torch.float32 and lse.shape == (B, num_heads, Sq),
          "lse must be float32 [B, num_heads, S_q]")
    ws_floats = bwd_workspace_floats(B * Sq, B * Sk, num_heads, num_kv_heads, head_dim, True)
    dq, dk, dv, ws = _bwd_outputs(q, k, v, dq, dk, dv, workspace, ws_floats, dev)
    lib = _lib.load()
    rc = lib.flash_attention_bwd_fp8(_ptr(dout), _ptr(q), _ptr(k), _ptr(v), _ptr(output),
                                     _ptr(lse), B, num_heads, num_kv_heads, Sq, Sk, head_dim,
                                     int(bool(causal)), float(q_scale), float(k_scale),
                                     float(v_scale), float(do_scale), float(o_scale),
                                     float(dq_scale), float(dk_scale), float(dv_scale),
                                     _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws), ws.numel(),
                                     _stream(dev))
    _lib.check(rc)
    return dq, dk, dv
