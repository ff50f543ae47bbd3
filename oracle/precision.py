"""Precision standard for comparing a result against the fp64 reference.

TEST INFRASTRUCTURE ONLY (used by the tests, the smoke check and the benchmark).

The SparseFlashAttention page, section 4 ("precision requirements"), defines
for sampled output points
    relative error  e = |actual - golden| / (|golden| + 1e-7)
    MERE = mean(e),  MARE = max(e)
and passes a result when MERE < Thr and MARE < 10 * Thr, with Thr per dtype
(float16 2^-10, bfloat16 2^-7, float32 2^-13, HiFloat32 2^-11,
float8 E4M3 2^-3, float8 E5M2 2^-2).

Reading used here (the page does not say which points are "sampled"):
  * golden is the unrounded fp64 reference;
  * MERE is taken literally over every compared element;
  * MARE is taken over the elements with |golden| >= tau, tau = 2^-10 * RMS(golden);
    an element below tau must instead satisfy |actual - golden| <= 10 * Thr * tau.
    (An output can sit arbitrarily close to zero, where even the exactly rounded
    fp64 value has an unbounded relative error, so a literal max over every
    element cannot be met by any finite-precision result.)
  * The literal MARE over all elements is always reported beside it.
"""
from __future__ import annotations

import math

import numpy as np

THRESHOLDS = {
    "fp16": 2.0 ** -10,
    "bf16": 2.0 ** -7,
    "fp32": 2.0 ** -13,
    "hif32": 2.0 ** -11,
    "fp8_e4m3": 2.0 ** -3,
    "fp8_e5m2": 2.0 ** -2,
}
GUARD = 1e-7
TAU_FACTOR = 2.0 ** -10


def relative_errors(actual, golden) -> np.ndarray:
    a = np.asarray(actual, dtype=np.float64).ravel()
    g = np.asarray(golden, dtype=np.float64).ravel()
    return np.abs(a - g) / (np.abs(g) + GUARD)


def mere_mare(actual, golden):
    """The page's two metrics, literally, over every element."""
    e = relative_errors(actual, golden)
    if e.size == 0:
        return 0.0, 0.0
    return float(e.mean()), float(e.max())


def gate(actual, golden, dtype: str) -> dict:
    """Applies the precision standard (reading above); returns a report with 'pass'."""
    thr = THRESHOLDS[dtype]
    a = np.asarray(actual, dtype=np.float64).ravel()
    g = np.asarray(golden, dtype=np.float64).ravel()
    if a.shape != g.shape:
        raise ValueError(f"shape mismatch {a.shape} vs {g.shape}")
    if not np.all(np.isfinite(a)):
        return {"pass": False, "reason": "non-finite output", "threshold": thr}
    n = a.size
    if n == 0:
        return {"pass": True, "n": 0, "threshold": thr, "mere": 0.0, "mare_literal": 0.0,
                "mare_tau": 0.0, "small_abs_max": 0.0, "tau": 0.0}
    e = np.abs(a - g) / (np.abs(g) + GUARD)
    mere = float(e.mean())
    rms = math.sqrt(float(np.mean(g * g)))
    tau = TAU_FACTOR * rms
    big = np.abs(g) >= tau
    mare_tau = float(e[big].max()) if big.any() else 0.0
    small_abs = float(np.abs(a - g)[~big].max()) if (~big).any() else 0.0
    ok = (mere < thr) and (mare_tau < 10 * thr) and (small_abs <= 10 * thr * tau)
    return {
        "pass": bool(ok),
        "n": int(n),
        "threshold": thr,
        "mere": mere,
        "mere_over_thr": mere / thr,
        "mare_tau": mare_tau,
        "mare_literal": float(e.max()),
        "literal_over_10thr": int((e >= 10 * thr).sum()),
        "tau": tau,
        "small_abs_max": small_abs,
        "small_abs_limit": 10 * thr * tau,
        "max_abs": float(np.abs(a - g).max()),
    }
