"""Comparison helpers shared by the GPU parity tests (no attention arithmetic)."""

from __future__ import annotations

import math
import os

import numpy as np
import torch

# tolerances against the f64 oracle (max absolute error)
#   f32 storage: O and LSE 1e-4; bf16: O 1e-2, LSE 1e-3 (the stated bounds).
#   The O bound limits the computation; a 16-bit O is also allowed the final
#   rounding to its storage dtype, half an ulp at |O| (see assert_close), which
#   alone reaches 7.8e-3 at |O| in [2, 4) and 1.6e-2 at [4, 8) in bf16 -- even
#   the exact O stored in bf16 would fail a flat 1e-2 there.  Per binade
#   [2^e, 2^(e+1)) of |O| the allowance is therefore tol + 2^(e-8) (bf16) and
#   tol + 2^(e-11) (f16).
#   f16: O 3e-3 for the computation alone -- derived: P is rounded to f16
#   (relative error <= 2^-11) before P.V, so O moves by at most
#   2^-11 * max|v| <= 2.9e-3 for |v| <= 6 (every f16 case draws N(0,1) values);
#   the f32 products and sums add ~1e-6.  Scores are exact products summed in
#   f32, so LSE errors stay near 1e-5 (bound 1e-3).
#   E4M3: |o8 * o_scale - O| <= 6e-2 * amax|O| and LSE 1e-3.
TOL = {
    torch.float32: (1e-4, 1e-4),
    torch.bfloat16: (1e-2, 1e-3),
    torch.float16: (3e-3, 1e-3),
}
FP8_REL_TOL = 6e-2
FP8_LSE_TOL = 1e-3


def oracle_workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def to_f64(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype in (torch.bfloat16, torch.float16):
        t = t.float()
    return t.double().numpy()


MANT_BITS = {torch.bfloat16: 7, torch.float16: 10}


def half_ulp(x: np.ndarray, dtype) -> np.ndarray:
    """Half the spacing of ``dtype`` (bf16 / f16) at |x|: the largest error of
    rounding x to that dtype (normal range)."""
    _, e = np.frexp(np.abs(x))               # |x| = m 2^e, m in [0.5, 1)
    return np.where(x == 0, 0.0, np.ldexp(1.0, e - 2 - MANT_BITS[dtype]))  # 0 is stored exactly


def assert_close(name, got, ref, tol, dtype=None):
    """Max-abs comparison.  Shapes must match, the result must hold no NaN and
    its -inf entries must coincide with the reference's.  With a 16-bit
    ``dtype`` (the storage of ``got``) each finite element may differ by ``tol``
    plus half an ulp of that dtype at the reference value (the rounding of the
    result to storage).  Returns the raw max |err| over the finite entries."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert not np.isnan(got).any(), f"{name}: NaN in the result"
    ninf_ref, ninf_got = np.isneginf(ref), np.isneginf(got)
    assert (ninf_ref == ninf_got).all(), f"{name}: -inf pattern differs " \
        f"({int(ninf_ref.sum())} expected, {int(ninf_got.sum())} got)"
    f = ~ninf_ref
    if not f.any():
        return 0.0
    r0 = np.where(f, ref, 0.0)
    err = np.where(f, np.abs(got - r0), 0.0)
    raw = float(err.max())
    allow = np.full(ref.shape, float(tol))
    if dtype in MANT_BITS:
        allow = allow + half_ulp(r0, dtype)
    excess = err - allow
    worst = int(np.argmax(excess))
    at = np.unravel_index(worst, got.shape)
    assert excess.flat[worst] <= 0.0, \
        f"{name}: |err| {err.flat[worst]:.3e} > allowed {allow.flat[worst]:.3e} at {at} " \
        f"(ref {ref.flat[worst]:.6g}, got {got.flat[worst]:.6g}; raw max |err| {raw:.3e}, " \
        f"tol {tol:.1e}{' + half an ulp' if dtype in MANT_BITS else ''})"
    return raw


def e4m3_decode_torch(codes: torch.Tensor) -> np.ndarray:
    """E4M3 codes -> float64 via torch's own float8 type (not the oracle codec)."""
    return codes.detach().cpu().view(torch.float8_e4m3fn).to(torch.float64).numpy()


def sample_rows(rng, lengths, heads, n):
    """n random (sequence, head, row) triples plus each sequence's first/last rows."""
    out = []
    for b, L in enumerate(lengths):
        if L == 0:
            continue
        for h in (0, heads - 1):
            out += [(b, h, 0), (b, h, L - 1), (b, h, min(L - 1, 127)), (b, h, min(L - 1, 128))]
    nz = [b for b, L in enumerate(lengths) if L > 0]
    for _ in range(n):
        b = int(rng.choice(nz))
        out.append((b, int(rng.integers(heads)), int(rng.integers(lengths[b]))))
    return sorted(set(out))


def nan_like(t: torch.Tensor) -> torch.Tensor:
    if t.dtype == torch.uint8:
        return torch.full_like(t, 0x7F)
    return torch.full_like(t, math.nan)


def f16_large_probability_case(num_heads=4, seqlen_q=8, seed=0):
    """Dense f16 input whose second 32-key tile holds one key scoring 15.99976
    (log2 units, after the 1/sqrt(128) scale) above the first tile's maximum:
    exp2 of it is 65525, which rounds past the largest finite f16 (65504), while
    the row's running sum of probabilities stays below 2^16.  Keys 0-31 score 0,
    key 32 scores 124.5 + 1989/2048 (exact in f32), keys 33-63 score -128.  One KV
    head, non-causal, 64 keys."""
    g = torch.Generator().manual_seed(seed)
    D = 128
    q = torch.zeros(1, num_heads, seqlen_q, D)
    q[..., 0] = 1.0
    q[..., 1] = 1.0
    k = torch.zeros(1, 1, 64, D)
    k[0, 0, 32, 0] = 124.5
    k[0, 0, 32, 1] = 1989 / 2048  # exact in f16
    k[0, 0, 33:, :2] = -64.0
    v = torch.randn(1, 1, 64, D, generator=g)
    assert float(k[0, 0, 32, :2].half().float().sum()) == 124.5 + 1989 / 2048
    from variable_length_gqa_amd.workloads import Dense
    return Dense(q.half(), k.half(), v.half(), num_heads, 1, D, False, 0, None,
                 "f16-large-probability")
