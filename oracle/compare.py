"""Parity tolerance between a GPU output and the fp64 oracle.

bf16 inputs with fp32 accumulation: per call, the largest absolute difference
must stay within 1e-2 of the largest reference magnitude, and every token row
t must satisfy ||y[t] - y_ref[t]||_2 <= 5e-3 * ||y_ref[t]||_2.  A reference row
that is exactly zero must be matched exactly.
"""
import numpy as np

MAX_ABS_FRAC = 1e-2
ROW_REL_L2 = 5e-3


def compare(y, y_ref, max_abs_frac=MAX_ABS_FRAC, row_rel=ROW_REL_L2):
    y = np.asarray(y, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    if y.shape != y_ref.shape:
        return {"ok": False, "reason": f"shape {y.shape} vs {y_ref.shape}"}
    if y.size == 0:
        return {"ok": True, "max_abs": 0.0, "ref_max": 0.0, "worst_row_rel": 0.0}
    if not np.all(np.isfinite(y)):
        return {"ok": False, "reason": "non-finite output"}
    d = y - y_ref
    max_abs = float(np.abs(d).max())
    ref_max = float(np.abs(y_ref).max())
    y2 = y_ref.reshape(y_ref.shape[0], -1) if y_ref.ndim > 1 else y_ref[None, :]
    d2 = d.reshape(y2.shape)
    rn = np.linalg.norm(y2, axis=1)
    dn = np.linalg.norm(d2, axis=1)
    zero = rn == 0
    rel = np.where(zero, np.where(dn == 0, 0.0, np.inf), dn / np.where(zero, 1.0, rn))
    worst = float(rel.max())
    ok = (max_abs <= max_abs_frac * ref_max or max_abs == 0.0) and worst <= row_rel
    return {"ok": bool(ok), "max_abs": max_abs, "ref_max": ref_max,
            "worst_row_rel": worst, "max_abs_frac": max_abs / ref_max if ref_max else 0.0}
