"""Pins of the CPU oracle's FP8 backward (flash_attention_bwd_fp8).

Reading: the inputs are E4M3 codes times per-tensor scales; the row term of
the softmax Jacobian comes from the stored forward output (o8 * o_scale); the
gradients are encoded as E4M3(g / g_scale).  The pins tie it to other, already
pinned functions on inputs dequantised by torch's own float8 type (not the
oracle's codec):
  * the row term from an exact output equals the Jacobian's own row term;
  * the result equals the exact gradient (pinned by finite differences) plus
    the closed-form effect of the stored output's rounding, whose pieces are
    the forward oracle with V := K and the backward oracle's dv with a
    substituted dout (the row term enters linearly);
  * the codes are torch's E4M3 cast of g / g_scale;
  * only the dequantised output matters (an exact power-of-two rescaling of
    o8 and o_scale changes nothing), and a one-key row whose stored output is
    its value row has dq = 0.
CPU only.
"""

import math

import numpy as np
import pytest
import torch

import oracle


def _q8(x):
    """Per-tensor E4M3 codes (uint8) and scale amax/448, by torch's cast."""
    amax = float(np.abs(x).max())
    s = amax / 448.0 if amax > 0 else 1.0
    codes = torch.from_numpy(x / s).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, s


def _deq(codes, s):
    return torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy() * s


def _case(B=2, H=4, Hkv=2, Sq=5, Sk=7, D=8, causal=True, seed=31):
    g = torch.Generator().manual_seed(seed)
    r = lambda *s: torch.randn(*s, generator=g, dtype=torch.float64).numpy()
    q8, qs = _q8(r(B, H, Sq, D))
    k8, ks = _q8(r(B, Hkv, Sk, D))
    v8, vs = _q8(r(B, Hkv, Sk, D))
    do8, dos = _q8(r(B, H, Sq, D))
    q, k, v, do = _deq(q8, qs), _deq(k8, ks), _deq(v8, vs), _deq(do8, dos)
    O, _ = oracle.flash_attention_fwd(q, k, v, H, Hkv, causal)
    o8, os_ = _q8(O)
    return dict(q8=q8, k8=k8, v8=v8, do8=do8, o8=o8, qs=qs, ks=ks, vs=vs, dos=dos, os=os_,
                q=q, k=k, v=v, do=do, O=O, H=H, Hkv=Hkv, causal=causal)


def _run(c, dq_s=1.0, dk_s=1.0, dv_s=1.0, o8=None, os_=None):
    return oracle.flash_attention_bwd_fp8(
        c["do8"], c["q8"], c["k8"], c["v8"], c["o8"] if o8 is None else o8, c["H"], c["Hkv"],
        c["causal"], c["qs"], c["ks"], c["vs"], c["dos"], c["os"] if os_ is None else os_,
        dq_s, dk_s, dv_s)


def test_row_term_from_exact_output_equals_jacobian_row_term():
    g = torch.Generator().manual_seed(5)
    r = lambda *s: torch.randn(*s, generator=g, dtype=torch.float64).numpy()
    q, K, V, dO = r(6, 8), r(9, 8), r(9, 8), r(6, 8)
    rows = np.arange(6)
    O, _ = oracle.attend_rows(q, K, V, rows, 6, 9, True, 0, 1 / math.sqrt(8))
    a = oracle.attend_rows_bwd(q, K, V, dO, rows, 6, 9, True, 0, 1 / math.sqrt(8))
    b = oracle.attend_rows_bwd(q, K, V, dO, rows, 6, 9, True, 0, 1 / math.sqrt(8), Orows=O)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, atol=1e-13)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("H,Hkv", [(4, 2), (3, 3)])
def test_equals_exact_gradient_plus_stored_output_correction(causal, H, Hkv):
    c = _case(H=H, Hkv=Hkv, causal=causal, seed=32 + H)
    _, _, _, dq, dk, dv = _run(c)
    q, k, v, do, O = c["q"], c["k"], c["v"], c["do"], c["O"]
    scale = 1 / math.sqrt(q.shape[-1])
    eq, ek, ev = oracle.flash_attention_bwd(do, q, k, v, H, Hkv, causal)
    # the row term moves by e_i = <dO_i, O'_i - O_i>; dS_ij moves by -P_ij e_i
    e = (do * (_deq(c["o8"], c["os"]) - O)).sum(axis=-1, keepdims=True)
    Pk, _ = oracle.flash_attention_fwd(q, k, k, H, Hkv, causal)    # sum_j P_ij k_j
    _, _, Pq = oracle.flash_attention_bwd(e * q, q, k, v, H, Hkv, causal)  # sum_i P_ij e_i q_i
    np.testing.assert_allclose(dv, ev, atol=1e-12)
    np.testing.assert_allclose(dq, eq - scale * e * Pk, atol=1e-12)
    np.testing.assert_allclose(dk, ek - scale * Pq, atol=1e-12)
    assert np.abs(e).max() > 1e-4   # the stored output's rounding does matter here


def test_codes_are_e4m3_of_gradient_over_scale():
    c = _case(seed=40)
    _, _, _, dq, dk, dv = _run(c)
    sc = [float(np.abs(t).max()) / 448 for t in (dq, dk, dv)]
    dq8, dk8, dv8, *_ = _run(c, *sc)
    for codes, g, s in zip((dq8, dk8, dv8), (dq, dk, dv), sc):
        want = torch.from_numpy(g / s).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        np.testing.assert_array_equal(codes, want)
        # and the decoded codes are within half an E4M3 ulp of the gradient
        err = np.abs(_deq(codes, s) - g)
        assert err.max() <= 16 * s + 1e-15   # half ulp at the top binade [256, 448]


def test_only_the_dequantised_output_matters():
    c = _case(seed=41)
    a = _run(c)
    # halve every stored output value exactly (codes of normal numbers: exponent
    # field - 1) and double its scale
    o8 = c["o8"].copy()
    e = (o8 >> 3) & 0xF
    ok = e >= 2
    o8[ok] = o8[ok] - (1 << 3)
    if (~ok).any():
        pytest.skip("subnormal output codes in this draw")
    b = _run(c, o8=o8, os_=2 * c["os"])
    for x, y in zip(a[3:], b[3:]):
        np.testing.assert_allclose(x, y, atol=1e-13)


def test_one_key_row_with_its_value_as_output_has_zero_dq():
    c = _case(Sq=7, Sk=7, causal=True, seed=42)
    # row 0 of every head sees key 0 only: store O_0 = v_0 exactly
    o8 = c["o8"].copy()
    G = c["H"] // c["Hkv"]
    for h in range(c["H"]):
        o8[:, h, 0] = c["v8"][:, h // G, 0]
    _, _, _, dq, _, _ = _run(c, o8=o8, os_=c["vs"])
    np.testing.assert_allclose(dq[:, :, 0], 0.0, atol=1e-14)
    assert np.abs(dq[:, :, 1:]).max() > 1e-3


def test_rejects_bad_scales():
    c = _case(seed=43)
    for bad in (0.0, -1.0, float("nan"), float("inf")):
        with pytest.raises(ValueError):
            _run(c, dq_s=bad)
