"""Round-to-nearest-even from fp64 to a storage format, in one step (no double rounding).

Test infrastructure only (see the package docstring).

The pages store every tensor in bf16, fp16 or fp32 and say nothing about rounding; the reading
used throughout is IEEE 754 round-to-nearest-ties-to-even, applied once per stored value, with
gradual underflow and overflow to infinity.
"""

from __future__ import annotations

import numpy as np

# name -> (significand bits including the hidden bit, minimum normal exponent, maximum exponent)
DTYPE_FORMATS = {
    "f32": (24, -126, 127),
    "bf16": (8, -126, 127),
    "f16": (11, -14, 15),
}


def rho(v, dtype: str) -> np.ndarray:
    """Round fp64 values to ``dtype`` ('f32', 'bf16', 'f16'; 'f64' is the identity).

    For |v| with leading-bit exponent E (clamped below at the format's minimum normal exponent),
    the representable neighbours are the multiples of q = 2**(E - p + 1); v/q is rounded to the
    nearest integer with ties to even (numpy.rint) and scaled back. Results above the largest
    finite value become +-inf. Returns fp64 arrays holding exactly representable values.
    """
    v = np.asarray(v, dtype=np.float64)
    if dtype == "f64":
        return v.copy()
    p, emin, emax = DTYPE_FORMATS[dtype]
    with np.errstate(invalid="ignore", over="ignore"):
        _, e = np.frexp(v)  # v = m * 2**e with 0.5 <= |m| < 1, so the leading bit is 2**(e-1)
        lead = np.maximum(e.astype(np.int64) - 1, emin)
        qexp = lead - (p - 1)
        out = np.ldexp(np.rint(np.ldexp(v, -qexp)), qexp)
        maxfinite = np.ldexp(2.0 - 2.0 ** (1 - p), emax)
        big = np.abs(out) > maxfinite
        out = np.where(big & np.isfinite(v), np.copysign(np.inf, v), out)
    return out
