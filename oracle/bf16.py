"""bfloat16 rounding for the oracle's stored decomposition outputs.

The pages store the decomposed arrays in the model dtype, bfloat16 ("Add a new
model architecture" page, "Decompose HF weights: the uniform case", step 6).
fp64 values are first rounded to fp32 (numpy, IEEE round-to-nearest-even),
then to bfloat16 by rounding the fp32 significand to 8 bits, ties to even.

This version works on the value, not the bit pattern: it splits x = m * 2**e
with frexp and rounds m * 2**8 to the nearest integer with numpy's rint (which
rounds halves to even).  The library rounds on bit patterns; the two are
independent implementations of the same rounding.
"""
import numpy as np


def round_bf16(a):
    """Nearest-even bfloat16 value of each element, returned as float64."""
    a32 = np.asarray(a, dtype=np.float64).astype(np.float32).astype(np.float64)
    out = np.array(a32, dtype=np.float64, copy=True)
    finite = np.isfinite(a32) & (a32 != 0.0)
    m, e = np.frexp(a32[finite])            # a = m * 2**e, 0.5 <= |m| < 1
    # bf16 keeps 8 significant bits (1 implicit + 7 stored): m in [0.5, 1)
    # carries its 8 bits as round(m * 2**8) * 2**-8.  Subnormals of fp32 (e <
    # -125) keep fewer bits: their spacing is 2**-133 for bf16.
    spacing_exp = np.maximum(e - 8, -133)
    q = np.rint(a32[finite] * np.ldexp(1.0, -spacing_exp))
    out[finite] = np.ldexp(q, spacing_exp)
    # values that round up past the bf16 maximum become infinity
    big = np.abs(out) > 3.3895313892515355e38
    out[big] = np.copysign(np.inf, out[big])
    return out


def bits_bf16(a):
    """Bit patterns (uint16) of round_bf16(a); used only by the pins."""
    v = round_bf16(a).astype(np.float32)
    return (v.view(np.uint32) >> 16).astype(np.uint16)
