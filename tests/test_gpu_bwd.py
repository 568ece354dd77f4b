"""GPU parity of the backward entry points against the f64 oracle.

Each case compares dq, dk, dv element by element with the oracle's gradient
of the exact forward.  The backward is fed either the oracle's own O (stored in
the input dtype) and LSE, which isolates the backward kernels, or the GPU
forward's results (the chained use).
"""

import numpy as np
import pytest
import torch

import oracle
import variable_length_gqa_amd as vg
from variable_length_gqa_amd import workloads as W
from tests.helpers import oracle_workers, to_f64

pytestmark = pytest.mark.gpu
DEV = "cuda"

# Tolerance: max |err| <= BWD_TOL[dtype] * max|ref| per gradient tensor (and
# an absolute floor for tensors that are ~0).  Derivation: the kernels round P
# and dS to the input dtype before the P^T dO, dS^T Q and dS K products
# (relative 2^-9 for bf16, 2^-11 for f16) and take delta from O stored in
# the input dtype; each gradient element sums up to L such terms with random
# signs, so its error is ~ 2^-9 * sqrt(L) * typical term, against a value of
# ~ sqrt(L) * typical term: a few 1e-3 of max|ref| for bf16, four times less
# for f16.  The largest errors measured on these cases are 5.3e-3 (bf16) and
# 5.5e-4 (f16) of max|ref|; the bounds leave a factor 3-4.
BWD_TOL = {torch.bfloat16: 1.5e-2, torch.float16: 2e-3}


def _close(name, got, ref, rel):
    got = to_f64(got)
    assert not np.isnan(got).any(), f"{name}: NaN"
    scale = max(float(np.abs(ref).max()), 1e-6)
    err = float(np.abs(got - ref).max())
    print(f"{name}: max|err| = {err:.3e} = {err / scale:.2e} of max|ref| {scale:.3e}")
    assert err <= rel * scale, f"{name}: {err:.3e} > {rel:.1e} * {scale:.3e}"


def _check_varlen(x, dtype, seed, chained=False):
    dO = W.make_dout(x.q, seed)
    G = x.num_heads
    dq_r, dk_r, dv_r = oracle.varlen_attention_bwd(
        dO, x.q, x.k, x.v, x.cu_q, x.cu_k, G, x.num_kv_heads, x.causal,
        workers=oracle_workers())
    xd = x.to(DEV)
    if chained:
        out, lse = vg.varlen_attention_fwd(xd.q, xd.k, xd.v, xd.cu_q, xd.cu_k, x.batch_size,
                                           G, x.num_kv_heads, x.max_seqlen_q, x.max_seqlen_k,
                                           x.head_dim, x.causal)
    else:
        O, L = oracle.varlen_attention_fwd(x.q, x.k, x.v, x.cu_q, x.cu_k, G, x.num_kv_heads,
                                           x.causal, workers=oracle_workers())
        out = torch.from_numpy(O).to(dtype).to(DEV)
        lse = torch.from_numpy(L).float().to(DEV)
    dq, dk, dv = vg.varlen_attention_bwd(dO.to(DEV), xd.q, xd.k, xd.v, out, lse, xd.cu_q,
                                         xd.cu_k, x.batch_size, G, x.num_kv_heads,
                                         x.max_seqlen_q, x.max_seqlen_k, x.head_dim, x.causal)
    torch.cuda.synchronize()
    rel = BWD_TOL[dtype]
    _close("dq", dq, dq_r, rel)
    _close("dk", dk, dk_r, rel)
    _close("dv", dv, dv_r, rel)
    return dq, dk, dv


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("H,Hkv", [(8, 2), (4, 4)])
def test_varlen_bwd_bf16(D, causal, H, Hkv):
    x = W.make_varlen([1, 37, 128, 129, 300, 0, 65], num_heads=H, num_kv_heads=Hkv,
                      head_dim=D, dtype=torch.bfloat16, causal=causal, seed=200 + D + H)
    _check_varlen(x, torch.bfloat16, 300 + D)


def test_varlen_bwd_f16():
    x = W.make_varlen([200, 77, 256], num_heads=8, num_kv_heads=4, head_dim=128,
                      dtype=torch.float16, causal=True, seed=210)
    _check_varlen(x, torch.float16, 310)


def test_varlen_bwd_unequal_q_k_lengths():
    # bottom-right causal alignment; rows before the keys start see nothing
    x = W.make_varlen([50, 300, 7], [120, 200, 40], num_heads=4, num_kv_heads=2, head_dim=128,
                      dtype=torch.bfloat16, causal=True, seed=211)
    _check_varlen(x, torch.bfloat16, 311)


def test_varlen_bwd_chained_after_gpu_forward():
    x = W.make_varlen([513, 64, 1000], num_heads=8, num_kv_heads=2, head_dim=128,
                      dtype=torch.bfloat16, causal=True, seed=212)
    _check_varlen(x, torch.bfloat16, 312, chained=True)


def test_varlen_bwd_is_deterministic():
    x = W.make_varlen([300, 129], num_heads=8, num_kv_heads=2, head_dim=128,
                      dtype=torch.bfloat16, causal=True, seed=213)
    a = _check_varlen(x, torch.bfloat16, 313, chained=True)
    b = _check_varlen(x, torch.bfloat16, 313, chained=True)
    for s, t in zip(a, b):
        assert torch.equal(s, t)


def _check_dense(B, H, Hkv, Sq, Sk, D, causal, window, seed, dtype=torch.bfloat16):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, H, Sq, D, generator=g).to(dtype)
    k = torch.randn(B, Hkv, Sk, D, generator=g).to(dtype)
    v = torch.randn(B, Hkv, Sk, D, generator=g).to(dtype)
    dO = W.make_dout(q, seed + 1)
    dq_r, dk_r, dv_r = oracle.flash_attention_bwd(dO, q, k, v, H, Hkv, causal, window,
                                                  workers=oracle_workers())
    O, L = oracle.flash_attention_fwd(q, k, v, H, Hkv, causal, window, workers=oracle_workers())
    out = torch.from_numpy(O).to(dtype).to(DEV)
    lse = torch.from_numpy(L).float().to(DEV)
    dq, dk, dv = vg.flash_attention_bwd(dO.to(DEV), q.to(DEV), k.to(DEV), v.to(DEV), out, lse,
                                        H, Hkv, D, causal, window)
    torch.cuda.synchronize()
    rel = BWD_TOL[dtype]
    _close("dq", dq, dq_r, rel)
    _close("dk", dk, dk_r, rel)
    _close("dv", dv, dv_r, rel)


@pytest.mark.parametrize("causal,window", [(True, 0), (True, 50), (False, 0), (False, 64)])
def test_dense_bwd(causal, window):
    _check_dense(2, 8, 2, 300, 300, 128, causal, window, 220 + window)


def test_dense_bwd_more_keys_than_queries():
    _check_dense(1, 4, 4, 200, 333, 128, True, 0, 230)


def test_dense_bwd_rows_without_keys():
    # 300 queries, 100 keys, causal: the first 200 rows see no key (dq = 0)
    _check_dense(1, 4, 2, 300, 100, 64, True, 0, 231)


def test_dense_bwd_f16_d64():
    _check_dense(2, 4, 2, 257, 257, 64, True, 0, 232, dtype=torch.float16)


def test_long_context_bwd_one_kv_group():
    """The long-context packed workload at full size ([8192, 4096, 2048, 2048],
    H=64, Hkv=8, D=128, causal), GPU forward then backward; dq of the 8 query
    heads of kv head 0 and that kv head's dk, dv against the oracle (whose dk /
    dv of kv head 0 need exactly those 8 query heads)."""
    x = W.workload("varlen_bf16_long")
    dO = W.make_dout(x.q, 400)
    heads = list(range(8))
    dq_r, dk_r, dv_r = oracle.varlen_attention_bwd(dO, x.q, x.k, x.v, x.cu_q, x.cu_k, 64, 8,
                                                   True, workers=oracle_workers(), heads=heads)
    xd = x.to(DEV)
    out, lse = vg.varlen_attention_fwd(xd.q, xd.k, xd.v, xd.cu_q, xd.cu_k, 4, 64, 8, 8192, 8192,
                                       128, True)
    dq, dk, dv = vg.varlen_attention_bwd(dO.to(DEV), xd.q, xd.k, xd.v, out, lse, xd.cu_q,
                                         xd.cu_k, 4, 64, 8, 8192, 8192, 128, True)
    torch.cuda.synchronize()
    rel = BWD_TOL[torch.bfloat16]
    _close("dq", dq[:, :8], dq_r[:, :8], rel)
    _close("dk", dk[:, 0], dk_r[:, 0], rel)
    _close("dv", dv[:, 0], dv_r[:, 0], rel)
