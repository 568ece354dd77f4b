"""Plain, slow, CPU reference for the varlen / GQA attention forward pass.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
its Python binding) imports, calls or links anything here; only the tests,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` do.  The
product fails loudly when its HIP library is missing; it never falls back to
this package.

Everything is computed in float64 on the inputs exactly as stored (bf16/f16/f32
are upcast, e4m3 codes are decoded and multiplied by their per-tensor scale).

Sources (the pages this follows):
  * boostr 0.2.0, src/ops/traits/attention/varlen_attention.rs --
    ``VarLenAttentionOps``: packed layout contract, GQA head map, cumulative
    sequence lengths, ``varlen_attention_fwd`` returning ``(output, logsumexp)``.
  * boostr, src/ops/traits/attention/flash.rs -- ``FlashAttentionOps``: dense
    ``[B,H,S,D]`` layout, GQA without repeat_kv, sliding window, ``kv_seq_len``
    over a capacity buffer, FP8 per-tensor scales, F32 logsumexp.
  * realizar 0.8.4, src/gguf/inference/forward/attention.rs -- IMP-111:
    standard softmax, standard (materialised) single-head attention used to
    verify the tiled version, online softmax and tiled single-head attention.

Modules:
  attention  -- the definition, materialised per (sequence, head) in row blocks.
  brute      -- pure-Python triple loop with math.fsum, for tiny inputs.
  online     -- the tiled online-softmax recurrence (realizar IMP-111b) in f64.
  e4m3       -- OCP FP8 E4M3 ("fn") decode and round-to-nearest-even encode.
  backward   -- the gradient of the forward definition (dq, dk, dv), summed
                over the query heads of a GQA group for dk/dv; its FP8 form.
  pack       -- padded [B, S, ...] <-> packed [total, ...] by cu_seqlens.

Parity pins for every function live in ``tests/test_oracle_pins.py``; none of
them compares the oracle with itself.
"""

from .attention import (  # noqa: F401
    cu_seqlens_from_lengths,
    allowed_keys,
    attend_rows,
    varlen_attention_fwd,
    flash_attention_fwd,
    flash_attention_fwd_fp8,
    varlen_rows,
    dense_rows,
    fp8_rows,
)
from .backward import (attend_rows_bwd, varlen_attention_bwd, flash_attention_bwd,  # noqa: F401
                       flash_attention_bwd_fp8)
from . import brute, online, e4m3, pack  # noqa: F401
