"""GPU parity of the split-KV decode entry point against the f64 oracle.

The decode path computes exactly the dense forward (same masks, same O and
LSE), so its oracle is the dense forward oracle.  The K/V buffers hold NaN
past kv_seq_len: any read of them would poison the result.
"""

import math

import pytest
import torch

import oracle
import variable_length_gqa_amd as vg
from variable_length_gqa_amd import workloads as W

from .helpers import TOL, assert_close, f16_large_probability_case, oracle_workers, to_f64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run_decode(d, workspace=None):
    dd = d.to(DEV)
    o, l = vg.flash_attention_decode(dd.q, dd.k, dd.v, d.num_heads, d.num_kv_heads, d.head_dim,
                                     d.causal, d.window, d.kv_seq_len, workspace=workspace)
    torch.cuda.synchronize()
    return o.cpu(), l.cpu()


def check_decode(d, heads=None):
    o, l = run_decode(d)
    O, L = oracle.flash_attention_fwd(d.q, d.k, d.v, d.num_heads, d.num_kv_heads, d.causal,
                                      d.window, d.kv_seq_len, workers=oracle_workers(),
                                      heads=heads)
    to, tl = TOL[d.q.dtype]
    sel = slice(None) if heads is None else list(heads)
    assert_close("O", to_f64(o)[:, sel], O[:, sel], to, d.q.dtype)
    assert_close("LSE", l.double().numpy()[:, sel], L[:, sel], tl)
    return o, l


def dense(B, H, Hkv, Sq, D, n, cap, causal=True, window=0, dtype=torch.bfloat16, seed=0):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, H, Sq, D, generator=g).to(dtype)
    kv = W.make_dense(B, Hkv, Hkv, 1, D, dtype=dtype, kv_seq_len=n, capacity=cap, seed=seed + 1)
    return W.Dense(q, kv.k, kv.v, H, Hkv, D, causal, window, n)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=str)
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("H,Hkv,Sq", [(8, 2, 1), (4, 4, 1), (32, 8, 4), (8, 1, 3), (16, 1, 2)],
                         ids=str)
def test_decode_small(dtype, D, H, Hkv, Sq):
    # 777 of 1000 slots: 24 full 32-key tiles and a ragged one
    check_decode(dense(2, H, Hkv, Sq, D, 777, 1000, seed=500 + D + H + Sq, dtype=dtype))


@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 1), (True, 100),
                                           (False, 333), (True, 5000)])
def test_decode_masks(causal, window):
    check_decode(dense(3, 8, 2, 4, 128, 2049, 2100, causal, window, seed=510 + window))


@pytest.mark.parametrize("n", [0, 1, 2, 31, 32, 33])
def test_decode_short_caches(n):
    # n = 0 and n < seqlen_q (causal): rows that see no key -> O = 0, LSE = -inf
    o, l = check_decode(dense(2, 8, 2, 4, 128, n, 64, causal=True, seed=520 + n))
    if n == 0:
        assert torch.all(o == 0) and torch.all(l == -math.inf)


def test_decode_matches_dense_forward():
    # same inputs through the tiled forward kernel and the split-KV path
    d = dense(4, 32, 8, 1, 128, 5000, 6000, seed=530)
    o, l = run_decode(d)
    dd = d.to(DEV)
    o2, l2 = vg.flash_attention_fwd(dd.q, dd.k, dd.v, 32, 8, 128, True, 0, 5000)
    torch.cuda.synchronize()
    assert (o.float() - o2.cpu().float()).abs().max() <= 1e-2
    assert (l - l2.cpu()).abs().max() <= 1e-3


def test_decode_workspace_sized_for_capacity_serves_every_length():
    cap = 4096
    ws = torch.empty(vg.decode_workspace_floats(2, 2, 128, cap), dtype=torch.float32,
                     device=DEV)
    for n in (4096, 300, 1, 2500):
        d = dense(2, 8, 2, 1, 128, n, cap, seed=540 + n)
        o, l = run_decode(d, workspace=ws)
        O, L = oracle.flash_attention_fwd(d.q, d.k, d.v, 8, 2, True, 0, n)
        assert_close("O", to_f64(o), O, TOL[torch.bfloat16][0], torch.bfloat16)
        assert_close("LSE", l.double().numpy(), L, TOL[torch.bfloat16][1])


def test_decode_rejects_small_workspace():
    d = dense(2, 8, 2, 1, 128, 1000, 1000, seed=550).to(DEV)
    ws = torch.empty(16, dtype=torch.float32, device=DEV)
    with pytest.raises(ValueError, match="workspace_floats"):
        vg.flash_attention_decode(d.q, d.k, d.v, 8, 2, 128, True, 0, 1000, workspace=ws)


def test_decode_is_deterministic():
    d = dense(2, 16, 2, 2, 128, 3000, 3000, seed=560)
    a = run_decode(d)
    b = run_decode(d)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_decode_workload_full_size():
    """The decode workload at full size (B=16, H=32, Hkv=8, D=128, one query,
    8192 cached keys in a 16384-slot buffer), every head against the oracle."""
    d = W.workload("dense_bf16_decode")
    check_decode(d)


@pytest.mark.parametrize("seqlen_q", [1, 8])
def test_decode_f16_probability_beyond_f16_range(seqlen_q):
    """The decode tile loop under the same large-probability row as the forward:
    one key just under 2^16 times the reference after a first tile of zeros."""
    d = f16_large_probability_case(num_heads=4, seqlen_q=seqlen_q, seed=116)
    o, _ = check_decode(d)
    assert torch.isfinite(o).all()
