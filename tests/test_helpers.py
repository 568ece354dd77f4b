"""CPU checks of the comparison helpers used by the GPU parity tests."""

import numpy as np
import torch

from tests.helpers import assert_close, half_ulp


def test_half_ulp_bounds_the_rounding_to_16_bit():
    rng = np.random.default_rng(3)
    x = rng.normal(0, 3, 100000) * np.exp2(rng.integers(-8, 8, 100000))
    x = x.astype(np.float32).astype(np.float64)  # torch rounds f64 via f32: avoid double rounding
    for dt in (torch.bfloat16, torch.float16):
        r = torch.from_numpy(x).to(dt).double().numpy()
        h = half_ulp(x, dt)
        lo, hi = (2.0 ** -14, 65000) if dt == torch.float16 else (1e-30, 1e30)
        ok = (np.abs(x) >= lo) & (np.abs(x) < hi)          # normal range
        assert np.all(np.abs(r - x)[ok] <= h[ok])
        # and it is tight: some roundings use most of it
        assert np.max((np.abs(r - x) / h)[ok]) > 0.99


def test_assert_close_allows_storage_rounding_only():
    ref = np.array([2.3542632164274417, 0.5, -3.9])
    got = torch.tensor(ref).to(torch.bfloat16).double().numpy()
    assert_close("x", got, ref, 0.0, torch.bfloat16)      # exact rounding passes at tol 0
    bad = got.copy()
    bad[0] += 0.0157                                      # one bf16 step too far
    try:
        assert_close("x", bad, ref, 1e-3, torch.bfloat16)
    except AssertionError:
        pass
    else:
        raise AssertionError("a wrong code passed")


def test_assert_close_checks_shape_and_infinities_on_every_path():
    ref = np.array([[0.5, -np.inf], [1.0, 2.0]])
    got = ref.copy()
    for dt in (None, torch.bfloat16, torch.float16):
        assert assert_close("x", got, ref, 1e-3, dt) == 0.0
        for bad in (got[:1], got.reshape(4)):                  # broadcastable or reshaped
            try:
                assert_close("x", bad, ref, 1e-3, dt)
            except AssertionError:
                pass
            else:
                raise AssertionError(f"a shape mismatch passed ({dt})")
        fin = got.copy()
        fin[0, 1] = -1e30                                      # finite where -inf is expected
        try:
            assert_close("x", fin, ref, 1e-3, dt)
        except AssertionError:
            pass
        else:
            raise AssertionError(f"a finite value in place of -inf passed ({dt})")


def test_assert_close_returns_the_raw_error():
    ref = np.array([0.25, 3.0])
    got = np.array([0.25, 3.0 + 0.01])
    assert abs(assert_close("x", got, ref, 1e-2, torch.bfloat16) - 0.01) < 1e-15
    assert abs(assert_close("x", got, ref, 2e-2) - 0.01) < 1e-15


def test_zero_is_allowed_no_rounding():
    # a reference of exactly 0 is stored exactly: only tol is allowed there
    try:
        assert_close("x", np.array([1.5e-3]), np.array([0.0]), 1e-3, torch.bfloat16)
    except AssertionError:
        pass
    else:
        raise AssertionError("half an ulp was allowed at 0")
