"""The allocation-free decode entry point (library-owned static scratch)
through the C ABI, against flash_attention_decode with a caller workspace and
against the f64 oracle: two calls in a row, the second smaller, then a call too
large for the scratch, rejected before any launch."""

import ctypes

import pytest
import torch

import oracle
import variable_length_gqa_amd as vg
from variable_length_gqa_amd import _lib
from variable_length_gqa_amd import workloads as W

from .helpers import TOL, assert_close, oracle_workers, to_f64

pytestmark = pytest.mark.gpu
DEV = "cuda"
CODE = {torch.bfloat16: _lib.VLGQA_BF16, torch.float16: _lib.VLGQA_F16}


def dense(B, H, Hkv, Sq, D, n, cap, causal, window, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, H, Sq, D, generator=g).to(dtype)
    kv = W.make_dense(B, Hkv, Hkv, 1, D, dtype=dtype, kv_seq_len=n, capacity=cap, seed=seed + 1)
    return W.Dense(q, kv.k, kv.v, H, Hkv, D, causal, window, n)


def noalloc(lib, dd, d, out, lse):
    B, H, Sq, D = dd.q.shape
    return lib.flash_attention_decode_noalloc(
        dd.q.data_ptr(), dd.k.data_ptr(), dd.v.data_ptr(), B, H, d.num_kv_heads, Sq,
        dd.k.shape[2], D, int(d.causal), d.window, -1 if d.kv_seq_len is None else d.kv_seq_len,
        CODE[d.q.dtype], out.data_ptr(), lse.data_ptr(),
        torch.cuda.current_stream().cuda_stream)


def check_against_workspace_and_oracle(lib, d):
    dd = d.to(DEV)
    B, H, Sq, D = d.q.shape
    out = torch.full_like(dd.q, float("nan"))
    lse = torch.full((B, H, Sq), float("nan"), dtype=torch.float32, device=DEV)
    assert noalloc(lib, dd, d, out, lse) == _lib.VLGQA_OK, lib.vlgqa_last_error()
    ref_o, ref_l = vg.flash_attention_decode(dd.q, dd.k, dd.v, H, d.num_kv_heads, D, d.causal,
                                             d.window, d.kv_seq_len)
    torch.cuda.synchronize()
    # the same kernels on the same inputs: the same bits
    assert torch.equal(out.view(torch.int16), ref_o.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), ref_l.view(torch.int32))
    O, L = oracle.flash_attention_fwd(d.q, d.k, d.v, H, d.num_kv_heads, d.causal, d.window,
                                      d.kv_seq_len, workers=oracle_workers())
    to, tl = TOL[d.q.dtype]
    assert_close("O", to_f64(out.cpu()), O, to, d.q.dtype)
    assert_close("LSE", lse.cpu().double().numpy(), L, tl)


def test_noalloc_decode_two_calls_second_smaller():
    lib = _lib.load()
    # the decode workload's shape: 16 sequences, 8192 cached keys of 16384
    # slots (NaN tail), H = 32, Hkv = 8, one query each
    check_against_workspace_and_oracle(lib, dense(16, 32, 8, 1, 128, 8192, 16384, True, 0,
                                                  torch.bfloat16, 900))
    # then a smaller one on the same scratch: f16, D = 64, 4 queries, a window
    check_against_workspace_and_oracle(lib, dense(2, 8, 2, 4, 64, 777, 1000, True, 100,
                                                  torch.float16, 901))


def test_noalloc_decode_rejects_a_problem_beyond_the_scratch():
    lib = _lib.load()
    A = 0x10000  # never dereferenced: the size check comes first
    rc = lib.flash_attention_decode_noalloc(A, A, A, 2048, 64, 8, 1, 8192, 128, 1, 0, 8192,
                                            _lib.VLGQA_BF16, A, A, None)
    assert rc == _lib.VLGQA_EINVAL
    assert lib.vlgqa_last_error().decode().startswith("batch:")
