"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these compares the oracle with itself: each check is a printed value,
a closed form, an invariant stated by the pages, a special case, or an
independent brute force.  They run on the CPU (not marked gpu).
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import brute, e4m3, online
from variable_length_gqa_amd import workloads as W
from variable_length_gqa_amd.flops import visible_key_span, visible_pairs

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _tiny(lengths_q, lengths_k=None, H=4, Hkv=2, D=4, seed=7):
    return W.make_varlen(lengths_q, lengths_k, num_heads=H, num_kv_heads=Hkv, head_dim=D,
                         dtype=torch.float32, seed=seed)


def _nested(x):
    return x.double().tolist()


# --------------------------------------------------------------------------
# cu_seqlens: the worked example printed on the varlen page
# --------------------------------------------------------------------------

def test_cu_seqlens_worked_example():
    g = json.load(open(os.path.join(GOLD, "cu_seqlens_example.json")))
    cu = oracle.cu_seqlens_from_lengths(g["lengths"])
    assert cu.dtype == np.int32
    assert cu.tolist() == g["cu_seqlens"]


def test_cu_seqlens_edge_cases():
    assert oracle.cu_seqlens_from_lengths([]).tolist() == [0]
    assert oracle.cu_seqlens_from_lengths([0, 3, 0]).tolist() == [0, 0, 3, 3]
    with pytest.raises(ValueError):
        oracle.cu_seqlens_from_lengths([1, -1])


# --------------------------------------------------------------------------
# brute force on tiny ragged inputs, every mask mode
# --------------------------------------------------------------------------

MODES = [(False, 0), (True, 0), (True, 1), (True, 2), (True, 3), (False, 2)]


@pytest.mark.parametrize("causal,window", MODES)
@pytest.mark.parametrize("lens_q,lens_k", [([3, 1, 0, 5], None), ([2, 4, 1], [5, 4, 3])])
def test_numpy_oracle_equals_brute_force(causal, window, lens_q, lens_k):
    x = _tiny(lens_q, lens_k)
    O, L = oracle.varlen_attention_fwd(x.q, x.k, x.v, x.cu_q, x.cu_k, 4, 2, causal, window)
    Ob, Lb = brute.varlen(_nested(x.q), _nested(x.k), _nested(x.v), x.lengths_q, x.lengths_k,
                          4, 2, causal, window)
    Ob, Lb = np.array(Ob), np.array(Lb)
    assert O.shape == Ob.shape == (sum(lens_q), 4, 4)
    np.testing.assert_allclose(O, Ob, rtol=0, atol=1e-12)
    fin = np.isfinite(Lb)
    assert (np.isfinite(L) == fin).all()
    np.testing.assert_allclose(L[fin], Lb[fin], rtol=0, atol=1e-12)


def test_online_tiled_recurrence_equals_definition():
    """realizar IMP-111b pattern: the tiled online recurrence verified by the
    materialised computation, here with masks and several tile sizes."""
    rng = np.random.default_rng(3)
    for (Lq, Lk) in [(7, 7), (5, 9), (13, 13)]:
        qh, kh, vh = rng.standard_normal((Lq, 8)), rng.standard_normal((Lk, 8)), \
            rng.standard_normal((Lk, 8))
        for causal, window in MODES:
            O, L = oracle.attention._attend_head(qh, kh, vh, causal, window, 1 / math.sqrt(8))
            for tile in (1, 3, 4, 16):
                To, TL = online.tiled_head(qh, kh, vh, causal, window, tile)
                np.testing.assert_allclose(To, O, rtol=0, atol=1e-12)
                assert (np.isfinite(TL) == np.isfinite(L)).all()
                f = np.isfinite(L)
                np.testing.assert_allclose(TL[f], L[f], rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# invariants the pages state
# --------------------------------------------------------------------------

def test_varlen_equals_each_sequence_alone():
    """Packing changes nothing: every sequence gives what it gives on its own."""
    x = W.make_varlen([17, 5, 33], num_heads=4, num_kv_heads=2, head_dim=16,
                      dtype=torch.float32, seed=11)
    for causal in (False, True):
        O, L = oracle.varlen_attention_fwd(x.q, x.k, x.v, x.cu_q, x.cu_k, 4, 2, causal)
        for b, n in enumerate(x.lengths_q):
            s = int(x.cu_q[b])
            qd = x.q[s:s + n].permute(1, 0, 2)[None]
            kd = x.k[s:s + n].permute(1, 0, 2)[None]
            vd = x.v[s:s + n].permute(1, 0, 2)[None]
            Od, Ld = oracle.flash_attention_fwd(qd, kd, vd, 4, 2, causal)
            np.testing.assert_allclose(O[s:s + n], Od[0].transpose(1, 0, 2), atol=1e-13, rtol=0)
            np.testing.assert_allclose(L[s:s + n], Ld[0].T, atol=1e-13, rtol=0)


def test_permuting_sequences_permutes_rows():
    x = W.make_varlen([9, 4, 12], num_heads=2, num_kv_heads=1, head_dim=8,
                      dtype=torch.float32, seed=12)
    O, L = oracle.varlen_attention_fwd(x.q, x.k, x.v, x.cu_q, x.cu_k, 2, 1, True)
    order = [2, 0, 1]
    segs = [slice(int(x.cu_q[b]), int(x.cu_q[b + 1])) for b in range(3)]
    qp = torch.cat([x.q[segs[b]] for b in order])
    kp = torch.cat([x.k[segs[b]] for b in order])
    vp = torch.cat([x.v[segs[b]] for b in order])
    cu = oracle.cu_seqlens_from_lengths([x.lengths_q[b] for b in order])
    Op, Lp = oracle.varlen_attention_fwd(qp, kp, vp, cu, cu, 2, 1, True)
    np.testing.assert_array_equal(Op, np.concatenate([O[segs[b]] for b in order]))
    np.testing.assert_array_equal(Lp, np.concatenate([L[segs[b]] for b in order]))


@pytest.mark.parametrize("H,Hkv", [(4, 2), (8, 2), (6, 1)])
def test_gqa_equals_mha_with_replicated_kv(H, Hkv):
    """boostr flash.rs "GQA support": no repeat_kv needed, i.e. the grouped
    result equals MHA on K/V heads replicated as kv_head = q_head / (H/Hkv)."""
    x = W.make_varlen([6, 11], num_heads=H, num_kv_heads=Hkv, head_dim=8,
                      dtype=torch.float32, seed=13)
    G = H // Hkv
    kr = x.k.repeat_interleave(G, dim=1)
    vr = x.v.repeat_interleave(G, dim=1)
    for causal in (False, True):
        O, L = oracle.varlen_attention_fwd(x.q, x.k, x.v, x.cu_q, x.cu_k, H, Hkv, causal)
        Om, Lm = oracle.varlen_attention_fwd(x.q, kr, vr, x.cu_q, x.cu_k, H, H, causal)
        np.testing.assert_array_equal(O, Om)
        np.testing.assert_array_equal(L, Lm)


def test_gqa_head_map_is_grouped_not_strided():
    """kv_head = q_head // G: heads 0..G-1 share kv head 0.  Planting a strided
    map (q_head % Hkv) must give a different answer, so the pin has teeth."""
    x = W.make_varlen([8], num_heads=4, num_kv_heads=2, head_dim=8, dtype=torch.float32,
                      seed=14)
    O, _ = oracle.varlen_attention_fwd(x.q, x.k, x.v, x.cu_q, x.cu_k, 4, 2, False)
    for h in range(4):
        ref, _ = oracle.varlen_attention_fwd(x.q[:, h:h + 1], x.k[:, h // 2:h // 2 + 1],
                                             x.v[:, h // 2:h // 2 + 1], x.cu_q, x.cu_k, 1, 1,
                                             False)
        np.testing.assert_array_equal(O[:, h], ref[:, 0])
    strided, _ = oracle.varlen_attention_fwd(x.q[:, 1:2], x.k[:, 1:2], x.v[:, 1:2], x.cu_q,
                                             x.cu_k, 1, 1, False)
    assert np.abs(O[:, 1] - strided[:, 0]).max() > 1e-3


def test_kv_seq_len_equals_narrowed_copy():
    """boostr flash.rs "kv_seq_len": a capacity buffer read to n positions equals
    the contiguous narrowed copy; the NaN tail must never be read."""
    d = W.make_dense(2, 4, 2, 10, 8, dtype=torch.float32, causal=True, kv_seq_len=10,
                     capacity=16, seed=15)
    assert torch.isnan(d.k[:, :, 10:]).all()
    for causal, window in [(True, 0), (True, 3), (False, 0)]:
        O, L = oracle.flash_attention_fwd(d.q, d.k, d.v, 4, 2, causal, window, kv_seq_len=10)
        On, Ln = oracle.flash_attention_fwd(d.q, d.k[:, :, :10].contiguous(),
                                            d.v[:, :, :10].contiguous(), 4, 2, causal, window)
        assert np.isfinite(O).all()
        np.testing.assert_array_equal(O, On)
        np.testing.assert_array_equal(L, Ln)


# --------------------------------------------------------------------------
# closed forms and special cases
# --------------------------------------------------------------------------

def test_lse_is_logsumexp_of_scaled_scores():
    x = _tiny([6, 9], H=2, Hkv=1, D=8, seed=16)
    O, L = oracle.varlen_attention_fwd(x.q, x.k, x.v, x.cu_q, x.cu_k, 2, 1, True)
    q, k = x.q.double().numpy(), x.k.double().numpy()
    for b in range(2):
        s0 = int(x.cu_q[b])
        for h in range(2):
            for i in range(x.lengths_q[b]):
                sc = [float(q[s0 + i, h] @ k[s0 + j, 0]) / math.sqrt(8) for j in range(i + 1)]
                mx = max(sc)
                ref = mx + math.log(math.fsum(math.exp(s - mx) for s in sc))
                assert abs(L[s0 + i, h] - ref) < 1e-12


def test_causal_first_row_is_v0():
    x = W.make_varlen([7, 3, 12], num_heads=4, num_kv_heads=2, head_dim=16,
                      dtype=torch.float32, seed=17)
    O, L = oracle.varlen_attention_fwd(x.q, x.k, x.v, x.cu_q, x.cu_k, 4, 2, True)
    for b in range(3):
        s = int(x.cu_q[b])
        for h in range(4):
            np.testing.assert_array_equal(O[s, h], x.v[s, h // 2].double().numpy())
            s00 = float(x.q[s, h].double() @ x.k[s, h // 2].double()) / 4.0
            assert abs(L[s, h] - s00) < 1e-13


def test_window_one_and_window_covering_everything():
    d = W.make_dense(1, 2, 1, 9, 8, dtype=torch.float32, causal=True, seed=18)
    O1, L1 = oracle.flash_attention_fwd(d.q, d.k, d.v, 2, 1, True, window=1)
    for h in range(2):
        np.testing.assert_array_equal(O1[0, h], d.v[0, 0].double().numpy())
        sii = (d.q[0, h].double() * d.k[0, 0].double()).sum(-1).numpy() / math.sqrt(8)
        np.testing.assert_allclose(L1[0, h], sii, atol=1e-13, rtol=0)
    Oc, Lc = oracle.flash_attention_fwd(d.q, d.k, d.v, 2, 1, True)
    for Wn in (9, 10, 100):
        Ow, Lw = oracle.flash_attention_fwd(d.q, d.k, d.v, 2, 1, True, window=Wn)
        np.testing.assert_array_equal(Ow, Oc)
        np.testing.assert_array_equal(Lw, Lc)


@pytest.mark.parametrize("causal,window", [(True, 0), (True, 4), (False, 0)])
def test_zero_queries_give_mean_and_log_count(causal, window):
    d = W.make_dense(1, 2, 2, 11, 8, dtype=torch.float32, seed=19)
    q0 = torch.zeros_like(d.q)
    O, L = oracle.flash_attention_fwd(q0, d.k, d.v, 2, 2, causal, window)
    v = d.v.double().numpy()
    for i in range(11):
        lo = max(0, i - window + 1) if window else 0
        hi = i if (causal or window) else 10
        cnt = hi - lo + 1
        np.testing.assert_allclose(O[0, :, i], v[0, :, lo:hi + 1].mean(axis=1), atol=1e-14)
        np.testing.assert_allclose(L[0, :, i], math.log(cnt), atol=1e-14)


def test_output_is_a_convex_combination():
    x = W.make_varlen([40, 25], num_heads=2, num_kv_heads=2, head_dim=8,
                      dtype=torch.float32, seed=20)
    O, _ = oracle.varlen_attention_fwd(x.q, x.k, x.v, x.cu_q, x.cu_k, 2, 2, True)
    v = x.v.double().numpy()
    for b in range(2):
        s = int(x.cu_q[b])
        for i in range(x.lengths_q[b]):
            vis = v[s:s + i + 1]
            assert (O[s + i] >= vis.min(axis=0) - 1e-12).all()
            assert (O[s + i] <= vis.max(axis=0) + 1e-12).all()


def test_empty_rows_and_sequences():
    # zero-length sequences are legal; a row with no visible key gives 0 / -inf
    x = _tiny([0, 3, 0], [2, 0, 4], H=2, Hkv=1, D=4, seed=21)
    O, L = oracle.varlen_attention_fwd(x.q, x.k, x.v, x.cu_q, x.cu_k, 2, 1, True)
    assert O.shape == (3, 2, 4)
    np.testing.assert_array_equal(O, 0.0)                 # sequence 1 has no keys
    assert np.isneginf(L).all()
    # Lq > Lk with causal: rows i < Lq - Lk see nothing (bottom-right alignment)
    y = _tiny([5], [3], H=1, Hkv=1, D=4, seed=22)
    O, L = oracle.varlen_attention_fwd(y.q, y.k, y.v, y.cu_q, y.cu_k, 1, 1, True)
    assert np.isneginf(L[:2]).all() and np.isfinite(L[2:]).all()
    np.testing.assert_array_equal(O[:2], 0.0)
    np.testing.assert_array_equal(O[2, 0], y.v[0, 0].double().numpy())


def test_sampled_rows_match_full():
    x = W.make_varlen([30, 17], num_heads=4, num_kv_heads=1, head_dim=8,
                      dtype=torch.float32, seed=23)
    O, L = oracle.varlen_attention_fwd(x.q, x.k, x.v, x.cu_q, x.cu_k, 4, 1, True)
    samples = [(0, 3, 29), (1, 0, 0), (1, 2, 16), (0, 1, 5)]
    Os, Ls = oracle.varlen_rows(x.q, x.k, x.v, x.cu_q, x.cu_k, 4, 1, True, samples)
    for n, (b, h, i) in enumerate(samples):
        t = int(x.cu_q[b]) + i
        np.testing.assert_allclose(Os[n], O[t, h], atol=1e-13, rtol=0)
        assert abs(Ls[n] - L[t, h]) < 1e-13


@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 3)])
def test_dense_rows_equal_brute_force(causal, window):
    """dense_rows on a GQA group of 3 (a strided head map would differ), with
    a K/V capacity of 12 attended to kv_seq_len = 9 (the tail is NaN, so any
    read of it poisons the row) and Sq = 7 != 9 (swapped extents would move the
    causal diagonal): every sampled row equals the pure-Python brute force."""
    g = torch.Generator().manual_seed(31)
    B, H, Hkv, Sq, cap, n, D = 2, 6, 2, 7, 12, 9, 4
    q = torch.randn(B, H, Sq, D, generator=g, dtype=torch.float64)
    k = torch.randn(B, Hkv, cap, D, generator=g, dtype=torch.float64)
    v = torch.randn(B, Hkv, cap, D, generator=g, dtype=torch.float64)
    k[:, :, n:] = math.nan
    v[:, :, n:] = math.nan
    samples = [(0, 0, 0), (0, 1, 6), (0, 2, 3), (1, 3, 1), (1, 4, 5), (1, 5, 6), (0, 5, 2)]
    Os, Ls = oracle.dense_rows(q, k, v, H, Hkv, causal, samples, window=window, kv_seq_len=n)
    assert Os.shape == (len(samples), D) and Ls.shape == (len(samples),)
    for r, (b, h, i) in enumerate(samples):
        kvh = h // (H // Hkv)
        keys = k[b, kvh, :n].tolist()
        vals = v[b, kvh, :n].tolist()
        ob, lb = brute.attention_one_row(q[b, h, i].tolist(), keys, vals,
                                         brute.visible_keys(i, Sq, n, causal, window),
                                         1 / math.sqrt(D))
        np.testing.assert_allclose(Os[r], ob, rtol=0, atol=1e-12)
        assert abs(Ls[r] - lb) < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_rows_equal_brute_force_and_saturate(causal):
    """fp8_rows against the brute force on inputs decoded by torch's own float8
    type (not the oracle codec): Sq = 5 queries on Sk = 8 keys, a GQA group of
    2; o_scale is a third of amax|O|/448, so some codes saturate.  The codes are
    torch's round-to-nearest-even cast where |O/o_scale| <= 448 and the
    saturated +-448 (0x7E / 0xFE) beyond."""
    g = torch.Generator().manual_seed(32)
    B, H, Hkv, Sq, Sk, D = 2, 4, 2, 5, 8, 8
    q8, qs = W.quantize_e4m3(torch.randn(B, H, Sq, D, generator=g))
    k8, ks = W.quantize_e4m3(torch.randn(B, Hkv, Sk, D, generator=g))
    v8, vs = W.quantize_e4m3(torch.randn(B, Hkv, Sk, D, generator=g))
    dec = lambda c, s: (c.view(torch.float8_e4m3fn).to(torch.float64) * s)
    qf, kf, vf = dec(q8, qs), dec(k8, ks), dec(v8, vs)
    samples = [(b, h, i) for b in range(B) for h in range(H) for i in range(Sq)]
    ref = []
    for (b, h, i) in samples:
        kvh = h // (H // Hkv)
        ob, lb = brute.attention_one_row(qf[b, h, i].tolist(), kf[b, kvh].tolist(),
                                         vf[b, kvh].tolist(),
                                         brute.visible_keys(i, Sq, Sk, causal, 0),
                                         1 / math.sqrt(D))
        ref.append((ob, lb))
    Ob = np.array([o for o, _ in ref])
    Lb = np.array([l for _, l in ref])
    o_scale = float(np.abs(Ob).max()) / 448.0 / 3.0
    codes, O, L = oracle.fp8_rows(q8, k8, v8, H, Hkv, causal, samples, qs, ks, vs, o_scale)
    np.testing.assert_allclose(O, Ob, rtol=0, atol=1e-12)
    fin = np.isfinite(Lb)
    assert (np.isfinite(L) == fin).all()
    np.testing.assert_allclose(L[fin], Lb[fin], rtol=0, atol=1e-12)
    x = Ob / o_scale
    big = np.abs(x) > 448.0
    assert big.any() and (~big).any()
    want = torch.from_numpy(np.where(big, 0.0, x)).to(torch.float8_e4m3fn).view(torch.uint8)
    want = np.where(big, np.where(x > 0, 0x7E, 0xFE), want.numpy())
    np.testing.assert_array_equal(codes, want)


def test_worker_pool_gives_same_result():
    x = W.make_varlen([20, 31, 9], num_heads=4, num_kv_heads=2, head_dim=8,
                      dtype=torch.float32, seed=24)
    a = oracle.varlen_attention_fwd(x.q, x.k, x.v, x.cu_q, x.cu_k, 4, 2, True, workers=1)
    b = oracle.varlen_attention_fwd(x.q, x.k, x.v, x.cu_q, x.cu_k, 4, 2, True, workers=3)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


# --------------------------------------------------------------------------
# E4M3 codec
# --------------------------------------------------------------------------

def test_e4m3_decode_hand_values():
    g = json.load(open(os.path.join(GOLD, "e4m3_codes.json")))
    for code, val in g["codes"].items():
        got = e4m3.decode_code(int(code, 16))
        assert got == val and math.copysign(1, got) == math.copysign(1, val), code
    for code in g["nan_codes"]:
        assert math.isnan(e4m3.decode_code(int(code, 16)))


def test_e4m3_decode_closed_form_all_codes():
    vals = e4m3.decode(np.arange(256, dtype=np.uint8))
    for c in range(256):
        e, m, s = (c >> 3) & 15, c & 7, -1.0 if c & 0x80 else 1.0
        if e == 15 and m == 7:
            assert math.isnan(vals[c])
        elif e == 0:
            assert vals[c] == s * (m / 8) * 2.0 ** -6
        else:
            assert vals[c] == s * (1 + m / 8) * 2.0 ** (e - 7)
    fin = vals[np.isfinite(vals)]
    assert fin.max() == 448.0 and fin.min() == -448.0


def test_e4m3_encode_cases_roundtrip_and_saturation():
    g = json.load(open(os.path.join(GOLD, "e4m3_codes.json")))
    for case in g["encode_cases"]:
        assert e4m3.encode_value(case["x"]) == int(case["code"], 16), case
    codes = np.arange(256, dtype=np.uint8)
    vals = e4m3.decode(codes)
    fin = np.isfinite(vals)
    back = e4m3.encode(vals[fin])
    # +0 and -0 both round-trip to their own code
    assert (back == codes[fin]).all()
    assert e4m3.encode(np.array([np.nan]))[0] == 0x7F
    assert (e4m3.encode(np.array([449.0, 1e30, -500.0])) == [0x7E, 0x7E, 0xFE]).all()


def test_e4m3_vector_encode_equals_scalar_encode():
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(20000) * 50, rng.standard_normal(2000) * 1e-3,
                        (np.arange(-900, 900) / 2.0)])
    vec = e4m3.encode(x)
    sca = np.array([e4m3.encode_value(v) for v in x], dtype=np.uint8)
    np.testing.assert_array_equal(vec, sca)


def test_e4m3_agrees_with_torch_on_range():
    rng = np.random.default_rng(6)
    x = np.concatenate([rng.uniform(-448, 448, 50000), rng.standard_normal(50000),
                        rng.standard_normal(5000) * 1e-3])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(e4m3.encode(x), ref)
    dec = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    dec = dec.to(torch.float64).numpy()
    ours = e4m3.decode(np.arange(256, dtype=np.uint8))
    f = np.isfinite(ours)
    np.testing.assert_array_equal(ours[f], dec[f])


# --------------------------------------------------------------------------
# FP8 entry point: scale conventions through special cases
# --------------------------------------------------------------------------

def test_fp8_causal_row0_reproduces_v_codes():
    """Row 0 of a causal head is v_0 exactly; with o_scale = v_scale the output
    codes of row 0 equal the input V codes (dequant multiplies, output quant
    divides)."""
    d = W.make_dense_fp8(2, 4, 2, 16, 32, causal=True, seed=25)
    s = d.scales
    o8, L, O = oracle.flash_attention_fwd_fp8(d.q, d.k, d.v, 4, 2, True, s["q_scale"],
                                              s["k_scale"], s["v_scale"], s["v_scale"])
    v8 = d.v.numpy()
    for b in range(2):
        for h in range(4):
            np.testing.assert_array_equal(o8[b, h, 0], v8[b, h // 2, 0])
            qv = e4m3.decode(d.q[b, h, 0].numpy()) * s["q_scale"]
            kv = e4m3.decode(d.k[b, h // 2, 0].numpy()) * s["k_scale"]
            assert abs(L[b, h, 0] - float(qv @ kv) / math.sqrt(32)) < 1e-12


def test_fp8_equals_dense_on_dequantised_inputs():
    d = W.make_dense_fp8(1, 2, 1, 24, 16, causal=True, seed=26)
    s = d.scales
    o8, L, O = oracle.flash_attention_fwd_fp8(d.q, d.k, d.v, 2, 1, True, s["q_scale"],
                                              s["k_scale"], s["v_scale"], 0.01)
    # dequantise by the closed-form decoder written out in the test
    def deq(t, sc):
        c = t.numpy().astype(np.int64)
        e, m, sg = (c >> 3) & 15, c & 7, np.where(c & 0x80, -1.0, 1.0)
        val = np.where(e == 0, m / 8 * 2.0 ** -6, (1 + m / 8) * 2.0 ** (e - 7))
        return sg * val * sc
    Od, Ld = oracle.flash_attention_fwd(deq(d.q, s["q_scale"]), deq(d.k, s["k_scale"]),
                                        deq(d.v, s["v_scale"]), 2, 1, True)
    np.testing.assert_allclose(O, Od, atol=1e-13, rtol=0)
    np.testing.assert_allclose(L, Ld, atol=1e-13, rtol=0)
    # o8 decodes to within half an E4M3 step of O / o_scale
    dec = e4m3.decode(o8) * 0.01
    assert np.all(np.abs(dec - O) <= np.maximum(np.abs(O) * 2.0 ** -4, 2.0 ** -10 * 0.01) + 1e-15)


def test_fp8_rejects_bad_scales():
    d = W.make_dense_fp8(1, 1, 1, 4, 8, seed=27)
    for bad in (0.0, -1.0, float("nan"), float("inf")):
        with pytest.raises(ValueError):
            oracle.flash_attention_fwd_fp8(d.q, d.k, d.v, 1, 1, True, 1.0, 1.0, 1.0, bad)


# --------------------------------------------------------------------------
# FLOP counter (package host logic) against closed forms and the oracle's mask
# --------------------------------------------------------------------------

def test_visible_pairs_closed_forms():
    for n in (1, 2, 7, 128, 1000):
        assert visible_pairs(n, n, False) == n * n
        assert visible_pairs(n, n, True) == n * (n + 1) // 2
        for w in (1, 3, 64):
            if w <= n:
                assert visible_pairs(n, n, True, w) == w * (w + 1) // 2 + (n - w) * w
    assert visible_pairs(8192, 8192, True, 4096) == 4096 * 4097 // 2 + 4096 * 4096
    assert visible_pairs(0, 5, True) == 0 and visible_pairs(5, 0, True) == 0


def test_visible_pairs_equals_mask_count():
    for (Lq, Lk) in [(5, 9), (9, 5), (13, 13), (1, 7)]:
        for causal, window in MODES:
            m = oracle.allowed_keys(np.arange(Lq), Lq, Lk, causal, window)
            assert visible_pairs(Lq, Lk, causal, window) == int(m.sum())


def test_visible_key_span_equals_mask_columns():
    # keys seen by at least one row: the K/V rows a decode pass has to read
    for (Lq, Lk) in [(1, 9), (4, 9), (9, 5), (13, 13), (1, 1), (3, 0), (0, 3)]:
        for causal, window in MODES + [(True, 1), (False, 2)]:
            m = oracle.allowed_keys(np.arange(Lq), Lq, Lk, causal, window)
            assert visible_key_span(Lq, Lk, causal, window) == int(m.any(axis=0).sum())
