"""Python entry points of the packing kernels: argument marshalling only.

boostr 0.2.0 varlen_attention.rs: variable-length sequences packed into one
buffer with I32 cu_seqlens offsets (cu[0] = 0, cu[i] = sum of lengths
0..i-1).  Every step runs in the HIP library on torch's current stream.
"""

from __future__ import annotations

import torch

from . import _lib
from . import attention as _attention
from .attention import _check_device_tensor, _need, _ptr, _stream, check_cu_seqlens


def cu_seqlens(lengths: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """int32 lengths [B] (device) -> int32 cu_seqlens [B+1] (device)."""
    dev = lengths.device
    _check_device_tensor("lengths", lengths, dev)
    _need(lengths.dtype == torch.int32 and lengths.dim() == 1, "lengths must be int32 [B]")
    B = lengths.shape[0]
    if out is None:
        out = torch.empty(B + 1, dtype=torch.int32, device=dev)
    _check_device_tensor("out", out, dev)
    _need(out.dtype == torch.int32 and out.shape == (B + 1,), "out must be int32 [B+1]")
    rc = _lib.load().vlgqa_cu_seqlens(_ptr(lengths), B, _ptr(out), _stream(dev))
    _lib.check(rc)
    return out


def _row_bytes(t: torch.Tensor, lead: int) -> int:
    n = t.element_size()
    for s in t.shape[lead:]:
        n *= s
    return n


def pack(padded: torch.Tensor, cu_seqlens_: torch.Tensor, total: int | None = None,
         out: torch.Tensor | None = None) -> torch.Tensor:
    """padded [B, S, ...] -> packed [total, ...] by cu_seqlens (device int32 [B+1]).

    ``total`` = cu_seqlens[-1]; when it is not given it is read back from the
    device (one synchronising copy).
    """
    dev = padded.device
    _check_device_tensor("padded", padded, dev)
    _check_device_tensor("cu_seqlens", cu_seqlens_, dev)
    _need(padded.dim() >= 2, "padded must be [B, S, ...]")
    B, S = padded.shape[0], padded.shape[1]
    _need(cu_seqlens_.dtype == torch.int32 and cu_seqlens_.shape == (B + 1,),
          "cu_seqlens must be int32 [B+1]")
    if total is None:
        total = int(cu_seqlens_[-1].item())
    if _attention.DEBUG_CHECKS:
        check_cu_seqlens(cu_seqlens_, total, S, "cu_seqlens")
    if out is None:
        out = torch.empty((total,) + tuple(padded.shape[2:]), dtype=padded.dtype, device=dev)
    _check_device_tensor("out", out, dev)
    _need(out.shape == (total,) + tuple(padded.shape[2:]) and out.dtype == padded.dtype,
          "out must be [total, ...] of the padded dtype")
    rc = _lib.load().vlgqa_pack(_ptr(padded), _ptr(cu_seqlens_), B, S, _row_bytes(padded, 2),
                                total, _ptr(out), _stream(dev))
    _lib.check(rc)
    return out


def unpack(packed: torch.Tensor, cu_seqlens_: torch.Tensor, max_seqlen: int,
           out: torch.Tensor | None = None) -> torch.Tensor:
    """packed [total, ...] -> padded [B, max_seqlen, ...], zeros after each sequence."""
    dev = packed.device
    _check_device_tensor("packed", packed, dev)
    _check_device_tensor("cu_seqlens", cu_seqlens_, dev)
    _need(packed.dim() >= 1, "packed must be [total, ...]")
    _need(cu_seqlens_.dtype == torch.int32 and cu_seqlens_.dim() == 1,
          "cu_seqlens must be int32 [B+1]")
    B = cu_seqlens_.shape[0] - 1
    if _attention.DEBUG_CHECKS:
        total = int(cu_seqlens_[-1].item())
        _need(total <= packed.shape[0], f"cu_seqlens[-1] = {total} exceeds the packed rows")
        check_cu_seqlens(cu_seqlens_, total, max_seqlen, "cu_seqlens")
    shape = (B, max_seqlen) + tuple(packed.shape[1:])
    if out is None:
        out = torch.empty(shape, dtype=packed.dtype, device=dev)
    _check_device_tensor("out", out, dev)
    _need(out.shape == shape and out.dtype == packed.dtype, "out must be [B, max_seqlen, ...]")
    rc = _lib.load().vlgqa_unpack(_ptr(packed), _ptr(cu_seqlens_), B, max_seqlen,
                                  _row_bytes(packed, 1), _ptr(out), _stream(dev))
    _lib.check(rc)
    return out
