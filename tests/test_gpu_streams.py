"""The library keeps no state between calls: forward and backward calls issued
on two streams at once (each backward with its own workspace) give bit for bit
the results of the same calls run one after the other."""

import pytest
import torch

import variable_length_gqa_amd as vg
from variable_length_gqa_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _problem(seed, lengths):
    x = W.make_varlen(lengths, num_heads=8, num_kv_heads=2, head_dim=128,
                      dtype=torch.bfloat16, causal=True, seed=seed).to(DEV)
    dO = W.make_dout(x.q, seed + 1).to(DEV)
    T, Tk = x.q.shape[0], x.k.shape[0]
    bufs = dict(out=torch.empty_like(x.q),
                lse=torch.empty(T, 8, dtype=torch.float32, device=DEV),
                dq=torch.empty_like(x.q), dk=torch.empty_like(x.k), dv=torch.empty_like(x.v),
                ws=torch.empty(vg.attention.bwd_workspace_floats(T, Tk, 8, 2, 128),
                               dtype=torch.float32, device=DEV))
    return x, dO, bufs


def _step(x, dO, b):
    L = max(x.lengths_q)
    vg.varlen_attention_fwd(x.q, x.k, x.v, x.cu_q, x.cu_k, x.batch_size, 8, 2, L, L, 128, True,
                            out=b["out"], lse=b["lse"])
    vg.varlen_attention_bwd(dO, x.q, x.k, x.v, b["out"], b["lse"], x.cu_q, x.cu_k,
                            x.batch_size, 8, 2, L, L, 128, True, dq=b["dq"], dk=b["dk"],
                            dv=b["dv"], workspace=b["ws"])


def test_concurrent_calls_on_two_streams_match_sequential():
    pa = _problem(900, [2048, 700, 33])
    pb = _problem(910, [1500, 1500, 129, 1])
    # sequential reference
    _step(*pa)
    _step(*pb)
    torch.cuda.synchronize()
    want = [{k: v.clone() for k, v in p[2].items() if k != "ws"} for p in (pa, pb)]
    for p in (pa, pb):
        for k, v in p[2].items():
            if k != "ws":
                v.fill_(float("nan"))
    # the same calls, one problem per stream, issued interleaved
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    sa.wait_stream(torch.cuda.current_stream())
    sb.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        with torch.cuda.stream(sa):
            _step(*pa)
        with torch.cuda.stream(sb):
            _step(*pb)
    torch.cuda.synchronize()
    for p, w in zip((pa, pb), want):
        for k, v in w.items():
            assert torch.equal(p[2][k], v), k
