"""GPU parity at sizes beyond the named workloads: one 131072-token sequence
(query and key indices past 2^16, 1024 query tiles, 4096 key tiles) and a
262144-key KV cache for the decode path, on rows the oracle computes one by
one; and the other extreme, 500 sequences of 0-40 tokens."""

import numpy as np
import pytest
import torch

import oracle
import variable_length_gqa_amd as vg
from variable_length_gqa_amd import workloads as W

from .helpers import TOL, assert_close, oracle_workers, to_f64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def test_varlen_single_131072_token_sequence_sampled():
    L = 131072
    x = W.make_varlen([L], num_heads=8, num_kv_heads=1, head_dim=128, dtype=torch.bfloat16,
                      causal=True, seed=700)
    xd = x.to(DEV)
    o, l = vg.varlen_attention_fwd(xd.q, xd.k, xd.v, xd.cu_q, xd.cu_k, 1, 8, 1, L, L, 128, True)
    torch.cuda.synchronize()
    o, l = o.cpu(), l.cpu()
    assert not torch.isnan(o).any() and torch.isfinite(l).all()
    rng = np.random.default_rng(701)
    rows = [0, 1, 127, 128, 65535, 65536, 65537, L - 129, L - 128, L - 1]
    rows += [int(r) for r in rng.integers(0, L, 10)]
    samples = [(0, h, r) for r in rows for h in (0, 7)]
    O, LSE = oracle.varlen_rows(x.q, x.k, x.v, x.cu_q, x.cu_k, 8, 1, True, samples)
    got_o = np.stack([to_f64(o[r, h]) for (_, h, r) in samples])
    got_l = np.array([float(l[r, h]) for (_, h, r) in samples])
    to, tl = TOL[torch.bfloat16]
    assert_close("O", got_o, O, to, torch.bfloat16)
    assert_close("LSE", got_l, LSE, tl)


def test_decode_262144_key_cache():
    n = 262144
    g = torch.Generator().manual_seed(702)
    q = torch.randn(1, 32, 1, 128, generator=g).to(torch.bfloat16)
    kv = W.make_dense(1, 8, 8, 1, 128, dtype=torch.bfloat16, kv_seq_len=n, capacity=n + 1000,
                      seed=703)
    d = W.Dense(q, kv.k, kv.v, 32, 8, 128, True, 0, n)
    dd = d.to(DEV)
    o, l = vg.flash_attention_decode(dd.q, dd.k, dd.v, 32, 8, 128, True, 0, n)
    torch.cuda.synchronize()
    O, L = oracle.flash_attention_fwd(d.q, d.k, d.v, 32, 8, True, 0, n, workers=oracle_workers())
    to, tl = TOL[torch.bfloat16]
    assert_close("O", to_f64(o.cpu()), O, to, torch.bfloat16)
    assert_close("LSE", l.cpu().double().numpy(), L, tl)


@pytest.mark.parametrize("head_dim", [64, 128])
def test_bwd_unsplit_heads_many_short_sequences(head_dim):
    """400 sequences of 0-96 tokens, 8 kv heads of 2 query heads: a grid of
    well over two key-tile workgroups per CU whose loops are all short, so the
    dK / dV workgroups cover the whole head group and store dK and dV directly
    (no partial sums to reduce).  Backward against the oracle on every
    element."""
    g = torch.Generator().manual_seed(707 + head_dim)
    lengths = [int(n) for n in torch.randint(0, 97, (400,), generator=g)]
    H, Hkv, D = 16, 8, head_dim
    x = W.make_varlen(lengths, num_heads=H, num_kv_heads=Hkv, head_dim=D, dtype=torch.bfloat16,
                      causal=True, seed=708 + head_dim)
    xd = x.to(DEV)
    B, mx = len(lengths), max(lengths)
    o, l = vg.varlen_attention_fwd(xd.q, xd.k, xd.v, xd.cu_q, xd.cu_k, B, H, Hkv, mx, mx, D, True)
    dO = W.make_dout(x.q, 709)
    dq, dk, dv = vg.varlen_attention_bwd(dO.to(DEV), xd.q, xd.k, xd.v, o, l, xd.cu_q, xd.cu_k, B,
                                         H, Hkv, mx, mx, D, True)
    torch.cuda.synchronize()
    refs = oracle.varlen_attention_bwd(dO, x.q, x.k, x.v, x.cu_q, x.cu_k, H, Hkv, True,
                                       workers=oracle_workers())
    for name, got, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), refs):
        err = float(np.abs(to_f64(got.cpu()) - ref).max())
        assert err <= 1.5e-2 * float(np.abs(ref).max()), (name, err)


def test_many_tiny_sequences_forward_and_backward():
    """500 sequences of 0-40 tokens (many empty or shorter than one tile) and
    a group of 16 query heads per kv head: forward and backward against the
    oracle on every element."""
    g = torch.Generator().manual_seed(704)
    lengths = [int(n) for n in torch.randint(0, 41, (500,), generator=g)]
    x = W.make_varlen(lengths, num_heads=16, num_kv_heads=1, head_dim=64, dtype=torch.bfloat16,
                      causal=True, seed=705)
    xd = x.to(DEV)
    B, mx = len(lengths), max(lengths)
    o, l = vg.varlen_attention_fwd(xd.q, xd.k, xd.v, xd.cu_q, xd.cu_k, B, 16, 1, mx, mx, 64, True)
    dO = W.make_dout(x.q, 706)
    dq, dk, dv = vg.varlen_attention_bwd(dO.to(DEV), xd.q, xd.k, xd.v, o, l, xd.cu_q, xd.cu_k, B,
                                         16, 1, mx, mx, 64, True)
    torch.cuda.synchronize()
    O, L = oracle.varlen_attention_fwd(x.q, x.k, x.v, x.cu_q, x.cu_k, 16, 1, True,
                                       workers=oracle_workers())
    to, tl = TOL[torch.bfloat16]
    assert_close("O", to_f64(o.cpu()), O, to, torch.bfloat16)
    assert_close("LSE", l.cpu().double().numpy(), L, tl)
    refs = oracle.varlen_attention_bwd(dO, x.q, x.k, x.v, x.cu_q, x.cu_k, 16, 1, True,
                                       workers=oracle_workers())
    for name, got, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), refs):
        err = float(np.abs(to_f64(got.cpu()) - ref).max())
        assert err <= 1.5e-2 * float(np.abs(ref).max()), (name, err)
