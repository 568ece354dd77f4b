"""GPU parity: the HIP kernels (through the C ABI) against the f64 oracle,
element by element, on seeded inputs that span several 128-row query tiles and
64-key tiles with ragged tails, plus the edge cases of the method."""

import math

import numpy as np
import pytest
import torch

import oracle
import variable_length_gqa_amd as vg
from variable_length_gqa_amd import workloads as W

from .helpers import FP8_LSE_TOL, FP8_REL_TOL, TOL, assert_close, e4m3_decode_torch, \
    f16_large_probability_case, nan_like, to_f64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run_varlen(x, out=None, lse=None, max_q=None, max_k=None):
    xd = x.to(DEV)
    o, l = vg.varlen_attention_fwd(xd.q, xd.k, xd.v, xd.cu_q, xd.cu_k, x.batch_size,
                                   x.num_heads, x.num_kv_heads,
                                   x.max_seqlen_q if max_q is None else max_q,
                                   x.max_seqlen_k if max_k is None else max_k, x.head_dim,
                                   x.causal, out=out, lse=lse)
    torch.cuda.synchronize()
    return o.cpu(), l.cpu()


def check_varlen(x):
    o, l = run_varlen(x)
    O, L = oracle.varlen_attention_fwd(x.q, x.k, x.v, x.cu_q, x.cu_k, x.num_heads,
                                       x.num_kv_heads, x.causal)
    to, tl = TOL[x.q.dtype]
    assert_close("O", to_f64(o), O, to, x.q.dtype)
    assert_close("LSE", l.double().numpy(), L, tl)
    return o, l


def run_dense(d):
    dd = d.to(DEV)
    o, l = vg.flash_attention_fwd(dd.q, dd.k, dd.v, d.num_heads, d.num_kv_heads, d.head_dim,
                                  d.causal, d.window, d.kv_seq_len)
    torch.cuda.synchronize()
    return o.cpu(), l.cpu()


def check_dense(d):
    o, l = run_dense(d)
    O, L = oracle.flash_attention_fwd(d.q, d.k, d.v, d.num_heads, d.num_kv_heads, d.causal,
                                      d.window, d.kv_seq_len)
    to, tl = TOL[d.q.dtype]
    assert_close("O", to_f64(o), O, to, d.q.dtype)
    assert_close("LSE", l.double().numpy(), L, tl)
    return o, l


DTYPES = [torch.bfloat16, torch.float16, torch.float32]
LENGTHS = [[129, 300, 0, 64, 513], [128, 127, 1, 256]]


# --------------------------------------------------------------------------
# packed varlen
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", DTYPES, ids=str)
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("heads", [(4, 4), (8, 2), (8, 1)], ids=str)
@pytest.mark.parametrize("li", [0, 1])
def test_varlen_small(dtype, D, causal, heads, li):
    H, Hkv = heads
    x = W.make_varlen(LENGTHS[li], num_heads=H, num_kv_heads=Hkv, head_dim=D, dtype=dtype,
                      causal=causal, seed=100 + li)
    check_varlen(x)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=str)
@pytest.mark.parametrize("causal", [False, True])
def test_varlen_unequal_q_and_k_lengths(dtype, causal):
    # queries are the newest Lq of Lk positions (bottom-right causal alignment);
    # Lq > Lk leaves the first Lq - Lk rows without keys (O = 0, LSE = -inf)
    x = W.make_varlen([5, 100, 200, 70, 1], [70, 100, 400, 3, 0], num_heads=4, num_kv_heads=2,
                      head_dim=128, dtype=dtype, causal=causal, seed=110)
    o, l = check_varlen(x)
    if causal:
        s = int(x.cu_q[3])
        assert torch.isneginf(l[s:s + 67]).all() and (o[s:s + 67] == 0).all()
    assert (o[-1] == 0).all() and torch.isneginf(l[-1]).all()   # sequence with no keys


def test_varlen_only_valid_rows_written():
    """Rows past cu_seqlens_q[-1] (padding of the buffer) are never written; every
    valid row is written exactly once (no NaN left behind)."""
    x = W.make_varlen([200, 0, 77], num_heads=4, num_kv_heads=2, head_dim=128,
                      dtype=torch.bfloat16, causal=True, seed=111)
    pad = 50
    q = torch.cat([x.q, torch.randn(pad, 4, 128).to(torch.bfloat16)])
    xp = W.Varlen(q, x.k, x.v, x.cu_q, x.cu_k, x.lengths_q, x.lengths_k, 4, 2, 128, True)
    out = nan_like(q).to(DEV)
    lse = torch.full((q.shape[0], 4), math.nan, device=DEV)
    o, l = run_varlen(xp, out=out, lse=lse)
    T = sum(x.lengths_q)
    assert not torch.isnan(o[:T]).any() and not torch.isnan(l[:T]).any()
    assert torch.isnan(o[T:]).all() and torch.isnan(l[T:]).all()
    O, L = oracle.varlen_attention_fwd(x.q, x.k, x.v, x.cu_q, x.cu_k, 4, 2, True)
    assert_close("O", to_f64(o[:T]), O, 1e-2, torch.bfloat16)
    assert_close("LSE", l[:T].double().numpy(), L, 1e-3)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=str)
def test_varlen_rows_beyond_max_seqlen_are_nan(dtype):
    """A sequence longer than max_seqlen_q (300 > 200, which the host's
    total_q <= batch_size * max_seqlen_q test cannot see) gets its rows past the
    launch's reach (256 = two 128-row tiles) written as NaN, never left stale;
    the rows within reach and the other sequence are still exact."""
    x = W.make_varlen([300, 10], num_heads=4, num_kv_heads=2, head_dim=128, dtype=dtype,
                      causal=True, seed=160)
    out = torch.zeros((310, 4, 128), dtype=dtype, device=DEV)
    lse = torch.zeros((310, 4), dtype=torch.float32, device=DEV)
    o, l = run_varlen(x, out=out, lse=lse, max_q=200)
    assert torch.isnan(o[256:300].float()).all() and torch.isnan(l[256:300]).all()
    O, L = oracle.varlen_attention_fwd(x.q, x.k, x.v, x.cu_q, x.cu_k, 4, 2, True)
    keep = np.r_[0:256, 300:310]
    to, tl = TOL[dtype]
    assert_close("O", to_f64(o)[keep], O[keep], to, dtype)
    assert_close("LSE", l.double().numpy()[keep], L[keep], tl)


def test_two_heads_per_workgroup_rows_beyond_max_seqlen_are_nan():
    """max_seqlen_q >= 4096 with an even group: the 16-bit kernel takes two
    heads of 64 rows per workgroup.  Every row within the launch's reach (65
    tiles of 64 rows = 4160) matches the oracle in both heads of each pair, and
    the rows of the 4200-token sequence past it are NaN in every head."""
    x = W.make_varlen([4200, 10], num_heads=4, num_kv_heads=2, head_dim=128,
                      dtype=torch.bfloat16, causal=True, seed=161)
    out = torch.zeros((4210, 4, 128), dtype=torch.bfloat16, device=DEV)
    lse = torch.zeros((4210, 4), dtype=torch.float32, device=DEV)
    o, l = run_varlen(x, out=out, lse=lse, max_q=4100)
    assert torch.isnan(o[4160:4200].float()).all() and torch.isnan(l[4160:4200]).all()
    O, L = oracle.varlen_attention_fwd(x.q, x.k, x.v, x.cu_q, x.cu_k, 4, 2, True)
    keep = np.r_[0:4160, 4200:4210]
    to, tl = TOL[torch.bfloat16]
    assert_close("O", to_f64(o)[keep], O[keep], to, torch.bfloat16)
    assert_close("LSE", l.double().numpy()[keep], L[keep], tl)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=str)
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_varlen_two_heads_per_workgroup(dtype, D, causal):
    """max_seqlen_q >= 4096 with an even group: the 16-bit kernel's two-head
    form (64 rows of two query heads per workgroup).  Ragged lengths with an
    empty sequence, one of exactly 4096 rows and unequal q / k lengths (rows
    without keys under the causal bound), every element against the oracle."""
    x = W.make_varlen([4133, 0, 700, 4096], [4133, 9, 1500, 4000], num_heads=4, num_kv_heads=2,
                      head_dim=D, dtype=dtype, causal=causal, seed=162)
    check_varlen(x)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=str)
def test_dense_window_two_heads_per_workgroup(dtype):
    """The dense layout with a capacity stride and a sliding window on the
    two-head form: 4100 query rows, 4150 of 4200 key slots, window 1000."""
    d = W.make_dense(2, 4, 2, 4100, 64, dtype=dtype, causal=True, window=1000, kv_seq_len=4150,
                     capacity=4200, seed=163)
    check_dense(d)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32], ids=str)
def test_causal_first_row_is_v0_bit_exact(dtype):
    x = W.make_varlen([300, 1, 129], num_heads=8, num_kv_heads=2, head_dim=128, dtype=dtype,
                      causal=True, seed=112)
    o, _ = run_varlen(x)
    for b in range(3):
        s = int(x.cu_q[b])
        for h in range(8):
            assert torch.equal(o[s, h], x.v[s, h // 4]), (b, h)


@pytest.mark.parametrize("seqlen_q", [1, 8, 130])
def test_f16_probability_beyond_f16_range(seqlen_q):
    """A later tile raises a row's score to just under 2^16 times the running
    reference: the probability must not be rounded to f16 unchecked (it would
    become inf and O NaN)."""
    d = f16_large_probability_case(num_heads=4, seqlen_q=seqlen_q, seed=115)
    o, _ = check_dense(d)
    assert torch.isfinite(o).all()


def test_deterministic():
    x = W.make_varlen([700, 33], num_heads=8, num_kv_heads=2, head_dim=128,
                      dtype=torch.bfloat16, causal=True, seed=113)
    a = run_varlen(x)
    b = run_varlen(x)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_varlen_all_empty_sequences():
    x = W.make_varlen([0, 0], num_heads=4, num_kv_heads=4, head_dim=64, dtype=torch.bfloat16,
                      seed=114)
    o, l = run_varlen(x, max_q=0, max_k=0)
    assert o.shape == (0, 4, 64) and l.shape == (0, 4)


# --------------------------------------------------------------------------
# dense: window, capacity buffer, GQA
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", DTYPES, ids=str)
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("window", [0, 1, 37, 128, 300, 10000])
def test_dense_window_capacity(dtype, D, window):
    d = W.make_dense(2, 8, 2, 333, D, dtype=dtype, causal=True, window=window, kv_seq_len=333,
                     capacity=512, seed=120 + window)
    o, l = check_dense(d)
    assert not torch.isnan(o).any()


@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 64), (False, 50)])
def test_dense_shorter_queries_than_keys(causal, window):
    # decode-like: 200 new queries against 333 cached keys of a 400-slot buffer
    g = torch.Generator().manual_seed(121)
    q = torch.randn(2, 4, 200, 128, generator=g).to(torch.bfloat16)
    kv = W.make_dense(2, 4, 4, 333, 128, dtype=torch.bfloat16, kv_seq_len=333, capacity=400,
                      seed=122)
    d = W.Dense(q, kv.k, kv.v, 4, 4, 128, causal, window, 333)
    check_dense(d)


def test_dense_kv_seq_len_none_uses_capacity():
    d = W.make_dense(1, 4, 1, 260, 128, dtype=torch.bfloat16, causal=True, seed=123)
    assert d.kv_seq_len is None
    check_dense(d)


# --------------------------------------------------------------------------
# FP8 (E4M3)
# --------------------------------------------------------------------------

def check_fp8(d, o_scale=None):
    s = d.scales
    if o_scale is None:
        _, _, O = oracle.flash_attention_fwd_fp8(d.q, d.k, d.v, d.num_heads, d.num_kv_heads,
                                                 d.causal, s["q_scale"], s["k_scale"],
                                                 s["v_scale"], 1.0)
        o_scale = float(np.abs(O).max()) / 448.0
    o8, L, O = oracle.flash_attention_fwd_fp8(d.q, d.k, d.v, d.num_heads, d.num_kv_heads,
                                              d.causal, s["q_scale"], s["k_scale"],
                                              s["v_scale"], o_scale)
    dd = d.to(DEV)
    out, lse = vg.flash_attention_fwd_fp8(dd.q, dd.k, dd.v, d.num_heads, d.num_kv_heads,
                                          d.head_dim, d.causal, s["q_scale"], s["k_scale"],
                                          s["v_scale"], o_scale)
    torch.cuda.synchronize()
    got = e4m3_decode_torch(out.cpu()) * o_scale
    amax = float(np.abs(O).max())
    assert_close("O(fp8)", got, O, FP8_REL_TOL * amax)
    assert_close("LSE", lse.cpu().double().numpy(), L, FP8_LSE_TOL)
    # P is rounded to bf16 and V is exact, so O is within a few bf16 roundings
    # of the oracle and most codes agree exactly with the oracle's own
    # rounding of O / o_scale; the mean error is a small fraction of a code
    # spacing (rounding P to E4M3 instead gives ~60% agreement)
    err = np.abs(got - O)
    assert err.mean() <= 1e-2 * amax, err.mean() / amax
    agree = float((out.cpu().numpy() == o8).mean())
    assert agree > 0.9, agree
    return out


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_small(D, causal):
    d = W.make_dense_fp8(2, 8, 2, 300, D, causal=causal, seed=130 + D)
    check_fp8(d)


def test_fp8_row0_reproduces_v_codes():
    d = W.make_dense_fp8(1, 4, 1, 200, 128, causal=True, seed=131)
    s = d.scales
    dd = d.to(DEV)
    out, _ = vg.flash_attention_fwd_fp8(dd.q, dd.k, dd.v, 4, 1, 128, True, s["q_scale"],
                                        s["k_scale"], s["v_scale"], s["v_scale"])
    torch.cuda.synchronize()
    for h in range(4):
        assert torch.equal(out[0, h, 0].cpu(), d.v[0, 0, 0])


def _fp8_case(B, H, Hkv, Sq, Sk, D, causal, seed):
    """E4M3 q [B,H,Sq,D] and k, v [B,Hkv,Sk,D] from seeded N(0,1) draws, per-tensor
    scales amax/448."""
    g = torch.Generator().manual_seed(seed)
    q8, qs = W.quantize_e4m3(torch.randn(B, H, Sq, D, generator=g))
    k8, ks = W.quantize_e4m3(torch.randn(B, Hkv, Sk, D, generator=g))
    v8, vs = W.quantize_e4m3(torch.randn(B, Hkv, Sk, D, generator=g))
    return W.Dense(q8, k8, v8, H, Hkv, D, causal, 0, None, f"fp8 {Sq} q x {Sk} k",
                   {"q_scale": qs, "k_scale": ks, "v_scale": vs})


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Sq,Sk,D", [(200, 333, 128), (333, 200, 128), (300, 517, 64),
                                     (1, 300, 128)], ids=str)
def test_fp8_unequal_query_and_key_lengths(Sq, Sk, D, causal):
    # causal with Sq > Sk: the first Sq - Sk rows see no key (O = 0, LSE = -inf)
    d = _fp8_case(2, 8, 2, Sq, Sk, D, causal, 140 + Sq + D)
    out = check_fp8(d)
    if causal and Sq > Sk:
        assert (out[:, :, :Sq - Sk].cpu() == 0).all()


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_output_saturates(causal):
    """o_scale a quarter of amax|O|/448: the outputs beyond the E4M3 range must
    be stored as the saturated +-448 codes (0x7E / 0xFE, the oracle's), never
    as a NaN code; every output is within 6e-2 of the representable range of
    the oracle's value clipped to that range."""
    d = _fp8_case(2, 8, 2, 300, 300, 128, causal, 150)
    s = d.scales
    _, _, O1 = oracle.flash_attention_fwd_fp8(d.q, d.k, d.v, 8, 2, causal, s["q_scale"],
                                              s["k_scale"], s["v_scale"], 1.0)
    o_scale = float(np.abs(O1).max()) / 448.0 / 4.0
    o8, L, O = oracle.flash_attention_fwd_fp8(d.q, d.k, d.v, 8, 2, causal, s["q_scale"],
                                              s["k_scale"], s["v_scale"], o_scale)
    dd = d.to(DEV)
    out, lse = vg.flash_attention_fwd_fp8(dd.q, dd.k, dd.v, 8, 2, 128, causal, s["q_scale"],
                                          s["k_scale"], s["v_scale"], o_scale)
    torch.cuda.synchronize()
    codes = out.cpu().numpy()
    assert not ((codes & 0x7F) == 0x7F).any(), "NaN code in the output"
    x = O / o_scale
    sure = np.abs(x) >= 480.0           # saturated whatever the computation's rounding
    assert int(sure.sum()) > 100, int(sure.sum())
    np.testing.assert_array_equal(codes[sure], o8[sure])
    assert set(np.unique(o8[sure]).tolist()) <= {0x7E, 0xFE}
    top = 448.0 * o_scale
    got = e4m3_decode_torch(out.cpu()) * o_scale
    err = np.abs(got - np.clip(O, -top, top))
    print(f"saturated {int(sure.sum())} of {x.size}; max err {err.max() / top:.3e} of 448 o_scale")
    assert err.max() <= FP8_REL_TOL * top, err.max() / top
    assert float((codes == o8).mean()) > 0.9
    assert_close("LSE", lse.cpu().double().numpy(), L, FP8_LSE_TOL)
