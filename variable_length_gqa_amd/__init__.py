"""MI355X-native fused attention over packed variable-length sequences.

Entry points (HIP kernels for gfx950 behind a C ABI, see include/vlgqa.h):
  varlen_attention_fwd     packed [total, H, D] with I32 cu_seqlens, GQA, causal
  flash_attention_fwd      dense [B, H, S, D], KV capacity stride, sliding window
  flash_attention_fwd_fp8  dense OCP E4M3 with per-tensor scales
  flash_attention_decode   dense, few queries against a long KV cache (split-KV)
  flash_attention_decode_noalloc  the same without a workspace (library scratch)
      -> (output, logsumexp)
  varlen_attention_bwd     gradients of the packed forward
  flash_attention_bwd      gradients of the dense forward
  flash_attention_bwd_fp8  gradients of the E4M3 forward, as E4M3 codes
      -> (dq, dk, dv)
  packing.cu_seqlens / packing.pack / packing.unpack
                           lengths -> cu_seqlens, padded <-> packed on the device
"""

from .attention import (  # noqa: F401
    decode_workspace_floats,
    flash_attention_bwd,
    flash_attention_bwd_fp8,
    flash_attention_decode,
    flash_attention_decode_noalloc,
    flash_attention_fwd,
    flash_attention_fwd_fp8,
    varlen_attention_bwd,
    varlen_attention_fwd,
)
from . import packing  # noqa: F401
from ._lib import VlgqaError  # noqa: F401

__version__ = "0.1.0"
