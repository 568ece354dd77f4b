"""Calls on several streams and many calls on one stream: forward and backward
calls issued on two streams at once (each backward with its own workspace)
give bit for bit the results of the same calls run one after the other.  The
forward keeps one claim counter per stream for handing out the last items of
a launch at run time; repeated launches on one stream (each continuing that
counter) give bit for bit the same results."""

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


def test_repeated_forward_launches_on_one_stream_are_identical():
    # large enough that a fifth of every XCD's slots is claimed at run time
    x = W.make_varlen([2048, 1024, 700, 300, 33], num_heads=32, num_kv_heads=8, head_dim=128,
                      dtype=torch.bfloat16, causal=True, seed=920).to(DEV)
    L = max(x.lengths_q)
    out = torch.empty_like(x.q)
    lse = torch.empty(x.q.shape[0], 32, dtype=torch.float32, device=DEV)

    def run():
        out.fill_(float("nan"))
        vg.varlen_attention_fwd(x.q, x.k, x.v, x.cu_q, x.cu_k, x.batch_size, 32, 8, L, L, 128,
                                True, out=out, lse=lse)
        return out.clone(), lse.clone()

    o0, l0 = run()
    side = torch.cuda.Stream()
    for i in range(40):
        if i % 7 == 3:  # now and then a launch on another stream
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                o, l = run()
            torch.cuda.current_stream().wait_stream(side)
        else:
            o, l = run()
        assert torch.equal(o, o0) and torch.equal(l, l0), i


def _fp8_problem(seed, batch, seqlen):
    d = W.make_dense_fp8(batch, 8, 2, seqlen, 128, causal=True, seed=seed).to(DEV)
    s = d.scales
    out = torch.empty(d.q.shape, dtype=torch.uint8, device=DEV)
    lse = torch.empty(d.q.shape[:3], dtype=torch.float32, device=DEV)
    return d, s, out, lse


def _fp8_step(d, s, out, lse):
    vg.flash_attention_fwd_fp8(d.q, d.k, d.v, 8, 2, 128, True, s["q_scale"], s["k_scale"],
                               s["v_scale"], 0.05, out=out, lse=lse)


def test_fp8_forward_on_two_streams_matches_sequential():
    """The FP8 forward widens V into a scratch block taken in stream order from
    the library's pool: calls on two streams at once, of different sizes, each
    repeated, get blocks of their own and the results of sequential calls."""
    pa = _fp8_problem(920, 2, 1500)
    pb = _fp8_problem(930, 3, 700)
    _fp8_step(*pa)
    _fp8_step(*pb)
    torch.cuda.synchronize()
    want = [(p[2].clone(), p[3].clone()) for p in (pa, pb)]
    for p in (pa, pb):
        p[2].zero_()
        p[3].fill_(float("nan"))
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    sa.wait_stream(torch.cuda.current_stream())
    sb.wait_stream(torch.cuda.current_stream())
    for _ in range(4):
        with torch.cuda.stream(sa):
            _fp8_step(*pa)
        with torch.cuda.stream(sb):
            _fp8_step(*pb)
    torch.cuda.synchronize()
    for p, (o, l) in zip((pa, pb), want):
        assert torch.equal(p[2], o) and torch.equal(p[3], l)


def test_stream_handle_reused_after_destroy_continues_the_counter():
    """The runtime gives a destroyed stream's handle to the next stream it
    creates, which then continues that stream's claim counter.  Forwards left
    pending on a stream that is destroyed at once, then forwards on new
    streams (most likely on the same handle): every result equals the
    reference bit for bit."""
    import ctypes
    import os

    hip = ctypes.CDLL(os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so"))
    x = W.make_varlen([2048, 1024, 700, 300, 33], num_heads=32, num_kv_heads=8, head_dim=128,
                      dtype=torch.bfloat16, causal=True, seed=940).to(DEV)
    L = max(x.lengths_q)
    T = x.q.shape[0]

    def launch(stream_handle, out, lse):
        rc = vg._lib.load().varlen_attention_fwd(
            x.q.data_ptr(), x.k.data_ptr(), x.v.data_ptr(), x.cu_q.data_ptr(), x.cu_k.data_ptr(),
            T, x.k.shape[0], x.batch_size, 32, 8, L, L, 128, 1, vg._lib.VLGQA_BF16,
            out.data_ptr(), lse.data_ptr(), stream_handle)
        assert rc == vg._lib.VLGQA_OK, vg._lib.load().vlgqa_last_error()

    ref_o, ref_l = torch.empty_like(x.q), torch.empty(T, 32, dtype=torch.float32, device=DEV)
    vg.varlen_attention_fwd(x.q, x.k, x.v, x.cu_q, x.cu_k, x.batch_size, 32, 8, L, L, 128, True,
                            out=ref_o, lse=ref_l)
    torch.cuda.synchronize()
    results, handles = [], []
    for _ in range(3):
        s = ctypes.c_void_p()
        assert hip.hipStreamCreate(ctypes.byref(s)) == 0
        handles.append(s.value)
        for _ in range(4):
            o = torch.full_like(x.q, float("nan"))
            l = torch.full((T, 32), float("nan"), device=DEV)
            torch.cuda.synchronize()  # the fills are on torch's stream
            launch(s.value, o, l)
            results.append((o, l))
        assert hip.hipStreamDestroy(s) == 0  # with the launches still pending
    torch.cuda.synchronize()
    for i, (o, l) in enumerate(results):
        assert torch.equal(o, ref_o) and torch.equal(l, ref_l), (i, handles)
