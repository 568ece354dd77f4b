"""Seeded synthetic inputs for the attention forward workloads.

Shared by the tests, the benchmark and the smoke check as the ONE module both
the HIP path and the CPU oracle receive inputs from.  It holds no attention
arithmetic: it only draws numbers, casts them to the storage dtype and lays
them out.

Recipe (every workload): values i.i.d. N(0, 1) drawn in float32 from a CPU
``torch.Generator`` seeded with ``1000 + config number``; draw order is the
sequence lengths (when random), then q, k, v; the draws are cast to the
storage dtype with round-to-nearest-even.  FP8 inputs are quantised per tensor
with scale = amax|x| / 448 and codes = E4M3(x / scale) (torch's
round-to-nearest-even cast).

Workloads (names used across the tests and the benchmark):
  varlen_f32_mha    lengths [512,300,128], H=Hkv=4, D=64, f32, non-causal
  varlen_bf16_gqa   16 sequences, lengths uniform in [128, 2048], H=32,
                    Hkv=8, D=128, bf16, causal
  varlen_bf16_long  lengths [8192,4096,2048,2048], H=64, Hkv=8, D=128, bf16,
                    causal (the throughput workload)
  dense_bf16_window [B=4, H=32, S=8192, D=128] queries, Hkv=8, K/V buffers of
                    capacity 16384 with kv_seq_len=8192 (the unused tail is NaN),
                    causal, window 4096
  dense_fp8         [B=8, H=32, S=4096, D=128] E4M3 q, Hkv=8, causal
"""

from __future__ import annotations

from dataclasses import dataclass, field

import torch

E4M3_MAX = 448.0


@dataclass
class Varlen:
    q: torch.Tensor                 # [total_q, H, D]
    k: torch.Tensor                 # [total_k, Hkv, D]
    v: torch.Tensor                 # [total_k, Hkv, D]
    cu_q: torch.Tensor              # int32 [B+1]
    cu_k: torch.Tensor              # int32 [B+1]
    lengths_q: list
    lengths_k: list
    num_heads: int
    num_kv_heads: int
    head_dim: int
    causal: bool
    name: str = ""

    @property
    def batch_size(self):
        return len(self.lengths_q)

    @property
    def max_seqlen_q(self):
        return max(self.lengths_q) if self.lengths_q else 0

    @property
    def max_seqlen_k(self):
        return max(self.lengths_k) if self.lengths_k else 0

    def to(self, device):
        return Varlen(self.q.to(device), self.k.to(device), self.v.to(device),
                      self.cu_q.to(device), self.cu_k.to(device), self.lengths_q,
                      self.lengths_k, self.num_heads, self.num_kv_heads, self.head_dim,
                      self.causal, self.name)


@dataclass
class Dense:
    q: torch.Tensor                 # [B, H, S_q, D]
    k: torch.Tensor                 # [B, Hkv, capacity, D]
    v: torch.Tensor
    num_heads: int
    num_kv_heads: int
    head_dim: int
    causal: bool
    window: int = 0
    kv_seq_len: int | None = None
    name: str = ""
    # fp8 only: per-tensor dequantisation scales (real = code * scale)
    scales: dict = field(default_factory=dict)

    def to(self, device):
        return Dense(self.q.to(device), self.k.to(device), self.v.to(device), self.num_heads,
                     self.num_kv_heads, self.head_dim, self.causal, self.window,
                     self.kv_seq_len, self.name, dict(self.scales))


def _cumsum_i32(lengths):
    out = [0]
    for n in lengths:
        out.append(out[-1] + int(n))
    return torch.tensor(out, dtype=torch.int32)


def _normal(g, shape):
    return torch.randn(shape, generator=g, dtype=torch.float32)


def make_varlen(lengths_q, lengths_k=None, num_heads=4, num_kv_heads=4, head_dim=64,
                dtype=torch.bfloat16, causal=False, seed=0, name="") -> Varlen:
    """Packed q/k/v for the given per-sequence lengths (lengths_k defaults to lengths_q)."""
    lengths_q = [int(n) for n in lengths_q]
    lengths_k = lengths_q if lengths_k is None else [int(n) for n in lengths_k]
    g = torch.Generator().manual_seed(seed)
    Tq, Tk = sum(lengths_q), sum(lengths_k)
    q = _normal(g, (Tq, num_heads, head_dim)).to(dtype)
    k = _normal(g, (Tk, num_kv_heads, head_dim)).to(dtype)
    v = _normal(g, (Tk, num_kv_heads, head_dim)).to(dtype)
    return Varlen(q, k, v, _cumsum_i32(lengths_q), _cumsum_i32(lengths_k), lengths_q,
                  lengths_k, num_heads, num_kv_heads, head_dim, causal, name)


def random_lengths(g, n, lo, hi):
    """n lengths uniform on the integers [lo, hi] (inclusive)."""
    return [int(x) for x in torch.randint(lo, hi + 1, (n,), generator=g)]


def make_dense(batch, num_heads, num_kv_heads, seqlen_q, head_dim, dtype=torch.bfloat16,
               causal=True, window=0, kv_seq_len=None, capacity=None, seed=0,
               tail_fill=float("nan"), name="") -> Dense:
    """Dense q [B,H,S_q,D] and K/V buffers [B,Hkv,capacity,D].

    The first ``kv_seq_len`` positions of K/V hold N(0,1) draws; positions from
    kv_seq_len to capacity hold ``tail_fill`` (NaN by default, so that any read
    of them poisons the result).
    """
    n = seqlen_q if kv_seq_len is None else int(kv_seq_len)
    cap = n if capacity is None else int(capacity)
    g = torch.Generator().manual_seed(seed)
    q = _normal(g, (batch, num_heads, seqlen_q, head_dim)).to(dtype)
    kd = _normal(g, (batch, num_kv_heads, n, head_dim))
    vd = _normal(g, (batch, num_kv_heads, n, head_dim))
    k = torch.full((batch, num_kv_heads, cap, head_dim), tail_fill, dtype=dtype)
    v = torch.full((batch, num_kv_heads, cap, head_dim), tail_fill, dtype=dtype)
    k[:, :, :n] = kd.to(dtype)
    v[:, :, :n] = vd.to(dtype)
    return Dense(q, k, v, num_heads, num_kv_heads, head_dim, causal, window,
                 None if kv_seq_len is None else n, name)


def make_dout(like: torch.Tensor, seed: int) -> torch.Tensor:
    """A seeded N(0,1) output gradient with the shape and dtype of ``like``
    (the incoming gradient of a backward pass)."""
    g = torch.Generator().manual_seed(seed)
    return _normal(g, tuple(like.shape)).to(like.dtype)


def quantize_e4m3(x: torch.Tensor):
    """Per-tensor E4M3 quantisation: (uint8 codes, scale) with scale = amax / 448."""
    amax = float(x.abs().max())
    scale = amax / E4M3_MAX if amax > 0 else 1.0
    codes = (x.to(torch.float32) / scale).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes.contiguous(), scale


def make_dense_fp8(batch, num_heads, num_kv_heads, seqlen, head_dim, causal=True, seed=0,
                   name="") -> Dense:
    """E4M3 q/k/v [B,H(kv),S,D] from N(0,1) draws, with per-tensor scales."""
    g = torch.Generator().manual_seed(seed)
    q = _normal(g, (batch, num_heads, seqlen, head_dim))
    k = _normal(g, (batch, num_kv_heads, seqlen, head_dim))
    v = _normal(g, (batch, num_kv_heads, seqlen, head_dim))
    q8, qs = quantize_e4m3(q)
    k8, ks = quantize_e4m3(k)
    v8, vs = quantize_e4m3(v)
    return Dense(q8, k8, v8, num_heads, num_kv_heads, head_dim, causal, 0, None, name,
                 {"q_scale": qs, "k_scale": ks, "v_scale": vs})


# ---------------------------------------------------------------------------
# the named workloads
# ---------------------------------------------------------------------------

WORKLOADS = ("varlen_f32_mha", "varlen_bf16_gqa", "varlen_bf16_long", "dense_bf16_window",
             "dense_fp8", "dense_bf16_decode")
SEEDS = {name: 1000 + i for i, name in enumerate(WORKLOADS)}


def workload(name: str):
    seed = SEEDS[name]
    if name == "varlen_f32_mha":
        return make_varlen([512, 300, 128], num_heads=4, num_kv_heads=4, head_dim=64,
                           dtype=torch.float32, causal=False, seed=seed, name=name)
    if name == "varlen_bf16_gqa":
        g = torch.Generator().manual_seed(seed)
        lengths = random_lengths(g, 16, 128, 2048)
        # q/k/v continue the same generator stream after the lengths
        Tq = sum(lengths)
        q = _normal(g, (Tq, 32, 128)).to(torch.bfloat16)
        k = _normal(g, (Tq, 8, 128)).to(torch.bfloat16)
        v = _normal(g, (Tq, 8, 128)).to(torch.bfloat16)
        cu = _cumsum_i32(lengths)
        return Varlen(q, k, v, cu, cu.clone(), lengths, list(lengths), 32, 8, 128, True, name)
    if name == "varlen_bf16_long":
        return make_varlen([8192, 4096, 2048, 2048], num_heads=64, num_kv_heads=8,
                           head_dim=128, dtype=torch.bfloat16, causal=True, seed=seed,
                           name=name)
    if name == "dense_bf16_window":
        return make_dense(4, 32, 8, 8192, 128, dtype=torch.bfloat16, causal=True,
                          window=4096, kv_seq_len=8192, capacity=16384, seed=seed, name=name)
    if name == "dense_fp8":
        return make_dense_fp8(8, 32, 8, 4096, 128, causal=True, seed=seed, name=name)
    if name == "dense_bf16_decode":
        # one new query per sequence against 8192 cached keys of a 16384-slot
        # buffer (the head configuration of the dense window workload)
        return make_dense(16, 32, 8, 1, 128, dtype=torch.bfloat16, causal=True, window=0,
                          kv_seq_len=8192, capacity=16384, seed=seed, name=name)
    raise KeyError(name)
