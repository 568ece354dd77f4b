"""GPU parity of the FP8 (E4M3) backward against the f64 oracle.

Inputs: E4M3 codes of seeded N(0,1) q, k, v and dout with per-tensor scales
amax/448; the forward output as E4M3 codes with o_scale = amax(O)/448 and the
LSE, either from the oracle (isolating the backward) or from the GPU FP8
forward (the chained use).  Gradient scales: amax of the oracle's gradient /
448.  Bound per gradient tensor: max |g8 * g_scale - g| <= 6e-2 amax|g| (the
E4M3 rounding of the result alone reaches 3.6% of amax at the top binade; P
and dS are rounded to bf16 before their products), the mean error a small
fraction of that, and most codes equal to the oracle's own rounding.
"""

import numpy as np
import pytest
import torch

import oracle
import variable_length_gqa_amd as vg
from variable_length_gqa_amd import workloads as W

from .helpers import FP8_REL_TOL, e4m3_decode_torch, oracle_workers

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _codes(x):
    return W.quantize_e4m3(x)


def make_case(B, H, Hkv, Sq, Sk, D, causal, seed, chained=False, batches=None):
    g = torch.Generator().manual_seed(seed)
    r = lambda *s: torch.randn(*s, generator=g, dtype=torch.float32)
    (q8, qs), (k8, ks), (v8, vs), (do8, dos) = (_codes(r(B, H, Sq, D)), _codes(r(B, Hkv, Sk, D)),
                                                _codes(r(B, Hkv, Sk, D)), _codes(r(B, H, Sq, D)))
    sel = slice(None) if batches is None else slice(0, batches)
    wk = oracle_workers()
    if chained:
        # o_scale from the oracle's forward, O and LSE from the GPU forward
        _, _, O = oracle.flash_attention_fwd_fp8(q8[sel], k8[sel], v8[sel], H, Hkv, causal, qs,
                                                 ks, vs, 1.0, workers=wk)
        os_ = float(np.abs(O).max()) / 448.0
        o8d, lsed = vg.flash_attention_fwd_fp8(q8.to(DEV), k8.to(DEV), v8.to(DEV), H, Hkv, D,
                                               causal, qs, ks, vs, os_)
        o8, lse = o8d.cpu(), lsed.cpu()
    else:
        _, L, O = oracle.flash_attention_fwd_fp8(q8, k8, v8, H, Hkv, causal, qs, ks, vs, 1.0,
                                                 workers=wk)
        o8, os_ = _codes(torch.from_numpy(O).float())
        lse = torch.from_numpy(L).float()
    return dict(q8=q8, k8=k8, v8=v8, do8=do8, o8=o8, lse=lse, qs=qs, ks=ks, vs=vs, dos=dos,
                os=os_, H=H, Hkv=Hkv, D=D, causal=causal, sel=sel)


def check(c, shrink=1.0):
    """GPU against the oracle; gradient scales amax/448/shrink (shrink > 1:
    the largest gradients lie beyond the E4M3 range and must come back as the
    saturated +-448 codes, exactly the oracle's)."""
    sel = c["sel"]
    _, _, _, dq, dk, dv = oracle.flash_attention_bwd_fp8(
        c["do8"][sel], c["q8"][sel], c["k8"][sel], c["v8"][sel], c["o8"][sel], c["H"], c["Hkv"],
        c["causal"], c["qs"], c["ks"], c["vs"], c["dos"], c["os"], 1.0, 1.0, 1.0,
        workers=oracle_workers())
    scales = [max(float(np.abs(t).max()), 1e-30) / 448.0 / shrink for t in (dq, dk, dv)]
    codes = oracle.flash_attention_bwd_fp8(
        c["do8"][sel], c["q8"][sel], c["k8"][sel], c["v8"][sel], c["o8"][sel], c["H"], c["Hkv"],
        c["causal"], c["qs"], c["ks"], c["vs"], c["dos"], c["os"], *scales,
        workers=oracle_workers())[:3]
    d = {k: c[k].to(DEV) for k in ("do8", "q8", "k8", "v8", "o8", "lse")}
    got = vg.flash_attention_bwd_fp8(d["do8"], d["q8"], d["k8"], d["v8"], d["o8"], d["lse"],
                                     c["H"], c["Hkv"], c["D"], c["causal"], c["qs"], c["ks"],
                                     c["vs"], c["dos"], c["os"], *scales)
    torch.cuda.synchronize()
    for name, g8, ref, s, want in zip(("dq", "dk", "dv"), got, (dq, dk, dv), scales, codes):
        g8 = g8.cpu()[sel]
        val = e4m3_decode_torch(g8) * s
        amax = float(np.abs(ref).max())
        err = np.abs(val - ref)
        agree = float((g8.numpy() == want).mean())
        print(f"{name}: max err {err.max() / amax:.3e}, mean {err.mean() / amax:.2e} of amax; "
              f"codes agreeing {agree:.3f}")
        assert not np.isnan(val).any(), name
        if shrink > 1.0:
            # beyond the range (with a margin for the computation's rounding):
            # exactly the oracle's saturated codes; the rest as below
            sure = np.abs(ref / s) >= 480.0
            assert int(sure.sum()) > 0, name
            np.testing.assert_array_equal(g8.numpy()[sure], want[sure])
            assert set(np.unique(want[sure]).tolist()) <= {0x7E, 0xFE}
            err = np.where(sure, 0.0, err)
        assert err.max() <= FP8_REL_TOL * amax, (name, err.max() / amax)
        assert err.mean() <= 1e-2 * amax, (name, err.mean() / amax)
        # with shrink > 1 the codes are finer than the computation's rounding
        # relative to amax, so fewer of the unsaturated ones can agree
        assert agree > (0.8 if shrink == 1.0 else 0.5), (name, agree)
    return got


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("H,Hkv", [(8, 2), (4, 4), (6, 2)], ids=str)
def test_fp8_bwd_small(D, causal, H, Hkv):
    # (6, 2): an odd group, whose dk / dv go through the partial sums unsplit
    check(make_case(2, H, Hkv, 300, 300, D, causal, 600 + D + H))


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_bwd_gradients_saturate(causal):
    check(make_case(2, 8, 2, 300, 300, 128, causal, 620 + causal), shrink=4.0)


def test_fp8_bwd_more_keys_than_queries():
    check(make_case(1, 4, 2, 200, 333, 128, True, 610))


def test_fp8_bwd_chained_after_gpu_forward():
    check(make_case(2, 8, 2, 513, 513, 128, True, 611, chained=True))


def test_fp8_bwd_is_deterministic():
    c = make_case(1, 8, 2, 257, 257, 128, True, 612)
    a = check(c)
    b = check(c)
    for s, t in zip(a, b):
        assert torch.equal(s, t)


def test_fp8_bwd_rejects_small_workspace():
    c = make_case(1, 4, 2, 64, 64, 64, True, 613)
    d = {k: c[k].to(DEV) for k in ("do8", "q8", "k8", "v8", "o8", "lse")}
    ws = torch.empty(100, dtype=torch.float32, device=DEV)
    with pytest.raises(ValueError):
        vg.flash_attention_bwd_fp8(d["do8"], d["q8"], d["k8"], d["v8"], d["o8"], d["lse"], 4, 2,
                                   64, True, c["qs"], c["ks"], c["vs"], c["dos"], c["os"], 1.0,
                                   1.0, 1.0, workspace=ws)


def test_fp8_bwd_workload_shape_first_batch():
    """The FP8 workload's shape (B=8, S=4096, H=32, Hkv=8, D=128, causal),
    GPU forward then backward over all of it; batch 0 against the oracle."""
    check(make_case(8, 32, 8, 4096, 4096, 128, True, 614, chained=True, batches=1))
