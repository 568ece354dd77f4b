"""OCP FP8 E4M3 ("e4m3fn") decode and round-to-nearest-even saturating encode.

TEST INFRASTRUCTURE ONLY: never imported by the product path.

The pages only say "FP8" with per-tensor scales (boostr flash.rs,
``flash_attention_fwd_fp8``).  Reading taken: the OCP E4M3 format, the one
CDNA4 matrix cores consume natively:
  bits  s eeee mmm, exponent bias 7,
  e = 0       : subnormal, value (-1)^s * 2^-6 * m/8
  1 <= e <= 15: normal,    value (-1)^s * 2^(e-7) * (1 + m/8)
  e = 15, m=7 : NaN (0x7F / 0xFF); there is no infinity; largest finite 448.
Encoding rounds to nearest, ties to an even mantissa, and saturates anything
of magnitude beyond 448 to +-448 (NaN stays NaN).

Written from the format definition with exact float64 arithmetic (scaling by
powers of two is exact), not from any library's conversion routine.
"""

from __future__ import annotations

import math

import numpy as np

MAX_FINITE = 448.0
NAN_CODE = 0x7F


def decode_code(code: int) -> float:
    """Value of one 8-bit code, from the bit fields."""
    code = int(code) & 0xFF
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 15 and m == 7:
        return math.nan
    if e == 0:
        return s * math.ldexp(m / 8.0, -6)
    return s * math.ldexp(1.0 + m / 8.0, e - 7)


_TABLE = np.array([decode_code(c) for c in range(256)], dtype=np.float64)


def decode(codes) -> np.ndarray:
    """Decode an array of uint8 codes to float64."""
    codes = np.asarray(codes)
    if codes.dtype != np.uint8:
        codes = codes.view(np.uint8) if codes.dtype.itemsize == 1 else codes.astype(np.uint8)
    return _TABLE[codes]


def _round_half_even(x: float) -> int:
    fl = math.floor(x)
    frac = x - fl
    if frac > 0.5:
        return fl + 1
    if frac < 0.5:
        return fl
    return fl if fl % 2 == 0 else fl + 1


def encode_value(x: float) -> int:
    """Code of the E4M3 value nearest to x (ties to even), saturating at 448."""
    x = float(x)
    if math.isnan(x):
        return NAN_CODE
    sign = 0x80 if (x < 0 or (x == 0 and math.copysign(1.0, x) < 0)) else 0
    a = abs(x)
    if a >= MAX_FINITE:
        return sign | 0x7E
    if a < math.ldexp(1.0, -6):
        # subnormal spacing 2^-9; n = 8 lands exactly on the smallest normal
        n = _round_half_even(math.ldexp(a, 9))
        return sign | n
    _, ex = math.frexp(a)          # a = f * 2^ex with f in [0.5, 1)
    e = ex - 1                     # a in [2^e, 2^(e+1))
    n = _round_half_even(math.ldexp(a, 3 - e))   # in [8, 16]
    if n == 16:
        e += 1
        n = 8
    if e + 7 > 15 or (e + 7 == 15 and n - 8 == 7):
        return sign | 0x7E        # rounding carried past 448: saturate
    return sign | ((e + 7) << 3) | (n - 8)


def encode(x) -> np.ndarray:
    """Encode an array of float64 to uint8 E4M3 codes.

    The same steps as ``encode_value`` applied elementwise (np.rint rounds
    half to even); pinned against ``encode_value`` in the tests.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    neg = np.signbit(x)
    with np.errstate(invalid="ignore"):
        f, ex = np.frexp(a)
        e = ex.astype(np.int64) - 1
        n = np.rint(np.ldexp(a, (3 - e).astype(np.int64))).astype(np.int64)
        carry = n == 16
        e = np.where(carry, e + 1, e)
        n = np.where(carry, 8, n)
        normal = ((e + 7) << 3) | (n - 8)
        sub = np.rint(np.ldexp(a, 9)).astype(np.int64)
        code = np.where(a < 2.0 ** -6, sub, normal)
        sat = (a >= MAX_FINITE) | (e + 7 > 15) | ((e + 7 == 15) & (n - 8 == 7))
        code = np.where(sat & ~(a < 2.0 ** -6), 0x7E, code)
    code = np.where(np.isnan(x), NAN_CODE, code | np.where(neg, 0x80, 0))
    return code.astype(np.uint8)
