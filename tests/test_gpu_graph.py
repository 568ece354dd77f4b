"""The entry points under HIP graph capture: the library enqueues on the
caller's stream and never synchronises, so a forward + backward step (and a
decode step, and an FP8 forward, whose scratch block for the bf16 copy of V is
taken and given back in stream order) captured once replays with the results
of the eager calls.  Each graph is replayed several times with eager work and
synchronisation in between, and every replay is compared bit for bit."""

import pytest
import torch

import variable_length_gqa_amd as vg
from variable_length_gqa_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _replay_and_compare(graph, outs, eager, other_work):
    for _ in range(3):
        for t in outs:
            t.fill_(float("nan")) if t.is_floating_point() else t.zero_()
        other_work()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, want in zip(outs, eager):
            assert torch.equal(got, want)


def test_forward_backward_step_replays_in_a_graph():
    x = W.make_varlen([300, 129, 64], num_heads=8, num_kv_heads=2, head_dim=128,
                      dtype=torch.bfloat16, causal=True, seed=800).to(DEV)
    dO = W.make_dout(x.q, 801).to(DEV)
    T, H = x.q.shape[0], 8
    out, lse = torch.empty_like(x.q), torch.empty(T, H, dtype=torch.float32, device=DEV)
    dq, dk, dv = torch.empty_like(x.q), torch.empty_like(x.k), torch.empty_like(x.v)
    ws = torch.empty(vg.attention.bwd_workspace_floats(T, x.k.shape[0], H, 2, 128),
                     dtype=torch.float32, device=DEV)

    def step():
        vg.varlen_attention_fwd(x.q, x.k, x.v, x.cu_q, x.cu_k, 3, H, 2, 300, 300, 128, True,
                                out=out, lse=lse)
        vg.varlen_attention_bwd(dO, x.q, x.k, x.v, out, lse, x.cu_q, x.cu_k, 3, H, 2, 300, 300,
                                128, True, dq=dq, dk=dk, dv=dv, workspace=ws)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    eager = [t.clone() for t in (out, lse, dq, dk, dv)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    other = torch.randn(1 << 20, device=DEV)
    _replay_and_compare(g, [out, lse, dq, dk, dv], eager, lambda: other.mul_(1.0001))


def test_decode_step_replays_in_a_graph():
    g0 = torch.Generator().manual_seed(802)
    q = torch.randn(2, 16, 1, 128, generator=g0).to(torch.bfloat16).to(DEV)
    kv = W.make_dense(2, 4, 4, 1, 128, dtype=torch.bfloat16, kv_seq_len=3000, capacity=4096,
                      seed=803).to(DEV)
    out = torch.empty_like(q)
    lse = torch.empty(2, 16, 1, dtype=torch.float32, device=DEV)
    ws = torch.empty(vg.decode_workspace_floats(2, 4, 128, 4096), dtype=torch.float32,
                     device=DEV)

    def step():
        vg.flash_attention_decode(q, kv.k, kv.v, 16, 4, 128, True, 0, 3000, out=out, lse=lse,
                                  workspace=ws)

    step()
    torch.cuda.synchronize()
    eager = [out.clone(), lse.clone()]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    other = torch.randn(1 << 20, device=DEV)
    _replay_and_compare(g, [out, lse], eager, lambda: other.mul_(1.0001))


def test_fp8_forward_replays_in_a_graph():
    d = W.make_dense_fp8(2, 8, 2, 700, 128, causal=True, seed=803).to(DEV)
    s = d.scales
    out = torch.empty(d.q.shape, dtype=torch.uint8, device=DEV)
    lse = torch.empty(d.q.shape[:3], dtype=torch.float32, device=DEV)

    def step():
        vg.flash_attention_fwd_fp8(d.q, d.k, d.v, 8, 2, 128, True, s["q_scale"], s["k_scale"],
                                   s["v_scale"], 0.05, out=out, lse=lse)

    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        step()
    torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    eager = [out.clone(), lse.clone()]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    other = torch.randn(1 << 20, device=DEV)
    _replay_and_compare(g, [out, lse], eager, lambda: other.mul_(1.0001))
