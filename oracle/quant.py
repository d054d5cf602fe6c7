"""FP8 (OCP E4M3) shared block with per-row power-of-two scales, in fp64.

This is the pages' quantized-shared-block headroom ("Quality (Gemma 4 31B)"
page, "Verdict": trained sharing on 4-bit shared blocks) taken in this
part's own 8-bit format.  A stored W0 row w (bf16 values) becomes codes
c_j and one scale q = 2^e such that w_j ~= value(c_j) * q:

* e is the smallest integer with max_j |w_j| <= 448 * 2^e (448 is the largest
  finite E4M3 value); an all-zero row takes e = 0.  With |w| = f * 2^E,
  f in [1, 2): e = E - 8 if f <= 1.75 else E - 7.
* c_j is w_j / q (exact: q is a power of two) rounded to the nearest E4M3
  value, ties to the even mantissa; |w_j / q| <= 448 never overflows.

E4M3 (OCP): sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent field
0 encodes subnormals m * 2^-9; exponent 15 with mantissa 7 is NaN (no
infinities), so the largest finite magnitude is 1.75 * 2^8 = 448.

The forward of a quantized bundle is the factored forward with W0 replaced
by value(c) * q (oracle.forward.factored); nothing else changes.
"""
import math

import numpy as np


def e4m3_value(code):
    """Value of one E4M3 code (0..255); NaN for the two NaN codes."""
    code = int(code)
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 15 and man == 7:
        return math.nan
    if exp == 0:
        return sign * man * 2.0 ** -9
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


E4M3 = np.array([e4m3_value(c) for c in range(256)], np.float64)
_POS_CODES = np.array([c for c in range(128) if not math.isnan(E4M3[c])])   # 0 .. 126
_POS_VALUES = E4M3[_POS_CODES]                                             # ascending


def encode(v):
    """Nearest E4M3 code of each |v| <= 448 (ties to the even mantissa)."""
    v = np.asarray(v, np.float64)
    if np.any(np.abs(v) > 448.0):
        raise ValueError("value outside the E4M3 range")
    a = np.abs(v)
    hi = np.searchsorted(_POS_VALUES, a, side="left")      # first value >= a
    hi = np.clip(hi, 0, len(_POS_VALUES) - 1)
    lo = np.clip(hi - 1, 0, len(_POS_VALUES) - 1)
    dlo = a - _POS_VALUES[lo]
    dhi = _POS_VALUES[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (_POS_CODES[hi] % 2 == 0) & (hi != lo))
    codes = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo])
    codes = np.where(a == _POS_VALUES[hi], _POS_CODES[hi], codes)
    return (codes | np.where(np.signbit(v) & (codes != 0), 0x80, 0)).astype(np.uint8)


def row_exponent(absmax):
    """Smallest e with absmax <= 448 * 2^e (0 for an all-zero row)."""
    if absmax == 0.0:
        return 0
    f, E = math.frexp(absmax)        # absmax = f * 2^E, f in [0.5, 1)
    f, E = 2.0 * f, E - 1            # f in [1, 2)
    return E - 8 if f <= 1.75 else E - 7


def quantize_rows(W0):
    """(codes [N, K] uint8, q [N] float64) of a bf16-valued W0."""
    W0 = np.asarray(W0, np.float64)
    q = np.array([2.0 ** row_exponent(float(np.max(np.abs(r)))) if r.size else 1.0 for r in W0])
    codes = encode(W0 / q[:, None])
    return codes, q


def dequantize(codes, q):
    """value(c) * q, the W0 the quantized bundle stands for."""
    return E4M3[np.asarray(codes)] * np.asarray(q, np.float64)[:, None]
