"""GPU parity at the five workloads' full sizes, in the launch configuration the
benchmark times: every output element against the f64 oracle (run across the
host's cores), plus properties that hold at any size (no NaN anywhere, causal
row 0 equal to V[0] bit for bit, LSE at least the diagonal score)."""

import json
import os

import numpy as np
import pytest
import torch

import oracle
import variable_length_gqa_amd as vg
from variable_length_gqa_amd import workloads as W

from .helpers import FP8_LSE_TOL, FP8_REL_TOL, TOL, assert_close, e4m3_decode_torch, \
    oracle_workers, to_f64

pytestmark = pytest.mark.gpu
DEV = "cuda"
GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _run_varlen(x):
    xd = x.to(DEV)
    o, l = vg.varlen_attention_fwd(xd.q, xd.k, xd.v, xd.cu_q, xd.cu_k, x.batch_size,
                                   x.num_heads, x.num_kv_heads, x.max_seqlen_q, x.max_seqlen_k,
                                   x.head_dim, x.causal)
    torch.cuda.synchronize()
    return o.cpu(), l.cpu()


def _varlen_properties(x, o, l):
    G = x.num_heads // x.num_kv_heads
    assert not torch.isnan(o).any() and torch.isfinite(l).all()
    # causal row 0 of every (sequence, head) is exactly V[0]
    for b in range(x.batch_size):
        s = int(x.cu_q[b])
        vr = x.v[s].repeat_interleave(G, dim=0)
        assert torch.equal(o[s], vr), b
    # LSE >= the diagonal score (that key is always visible)
    diag = (x.q.float() * x.k.float().repeat_interleave(G, dim=1)).sum(-1) / x.head_dim ** 0.5
    assert (l >= diag - 1e-3).all()


def test_varlen_f32_mha_full():
    x = W.workload("varlen_f32_mha")
    assert x.cu_q.tolist() == [0, 512, 812, 940]
    o, l = _run_varlen(x)
    O, L = oracle.varlen_attention_fwd(x.q, x.k, x.v, x.cu_q, x.cu_k, 4, 4, False)
    assert_close("O", to_f64(o), O, TOL[torch.float32][0])
    assert_close("LSE", l.double().numpy(), L, TOL[torch.float32][1])


def test_varlen_bf16_gqa_full():
    x = W.workload("varlen_bf16_gqa")
    assert len(x.lengths_q) == 16 and all(128 <= n <= 2048 for n in x.lengths_q)
    o, l = _run_varlen(x)
    O, L = oracle.varlen_attention_fwd(x.q, x.k, x.v, x.cu_q, x.cu_k, 32, 8, True,
                                       workers=oracle_workers())
    assert_close("O", to_f64(o), O, TOL[torch.bfloat16][0], torch.bfloat16)
    assert_close("LSE", l.double().numpy(), L, TOL[torch.bfloat16][1])
    _varlen_properties(x, o, l)


def test_varlen_bf16_long_full():
    x = W.workload("varlen_bf16_long")
    o, l = _run_varlen(x)
    _varlen_properties(x, o, l)
    O, L = oracle.varlen_attention_fwd(x.q, x.k, x.v, x.cu_q, x.cu_k, 64, 8, True,
                                       workers=oracle_workers())
    assert_close("O", to_f64(o), O, TOL[torch.bfloat16][0], torch.bfloat16)
    assert_close("LSE", l.double().numpy(), L, TOL[torch.bfloat16][1])


def test_dense_bf16_window_full():
    d = W.workload("dense_bf16_window")
    assert torch.isnan(d.k[:, :, 8192:]).all() and torch.isnan(d.v[:, :, 8192:]).all()
    dd = d.to(DEV)
    o, l = vg.flash_attention_fwd(dd.q, dd.k, dd.v, 32, 8, 128, True, 4096, 8192)
    torch.cuda.synchronize()
    o, l = o.cpu(), l.cpu()
    # the NaN tail of the K/V buffers was never read
    assert not torch.isnan(o).any() and torch.isfinite(l).all()
    for b in range(4):
        for h in range(32):
            assert torch.equal(o[b, h, 0], d.v[b, h // 4, 0])
    O, L = oracle.flash_attention_fwd(d.q, d.k, d.v, 32, 8, True, window=4096, kv_seq_len=8192,
                                      workers=oracle_workers())
    assert_close("O", to_f64(o), O, TOL[torch.bfloat16][0], torch.bfloat16)
    assert_close("LSE", l.double().numpy(), L, TOL[torch.bfloat16][1])


def test_dense_fp8_full():
    d = W.workload("dense_fp8")
    g = json.load(open(os.path.join(GOLD, "fp8_o_scale.json")))
    s = d.scales
    for k in ("q_scale", "k_scale", "v_scale"):
        assert s[k] == g[k], "the seeded fp8 inputs differ from the ones o_scale was made for"
    o_scale = g["o_scale"]
    dd = d.to(DEV)
    out, lse = vg.flash_attention_fwd_fp8(dd.q, dd.k, dd.v, 32, 8, 128, True, s["q_scale"],
                                          s["k_scale"], s["v_scale"], o_scale)
    torch.cuda.synchronize()
    out, lse = out.cpu(), lse.cpu()
    assert torch.isfinite(lse).all()
    assert not ((out == 0x7F) | (out == 0xFF)).any()       # no NaN codes
    o8, L, O = oracle.flash_attention_fwd_fp8(d.q, d.k, d.v, 32, 8, True, s["q_scale"],
                                              s["k_scale"], s["v_scale"], o_scale,
                                              workers=oracle_workers())
    assert abs(float(np.abs(O).max()) - g["amax_O"]) <= 1e-9 * g["amax_O"]
    assert_close("O(fp8)", e4m3_decode_torch(out) * o_scale, O, FP8_REL_TOL * g["amax_O"])
    assert_close("LSE", lse.double().numpy(), L, FP8_LSE_TOL)
    assert (out.numpy() == o8).mean() > 0.9
