"""Rounding of real values to bfloat16 under three rules (TEST INFRASTRUCTURE ONLY).

Only tests/, the smoke check and the benchmark's CPU-baseline leg may use this
module; the library never does.

"MoonMath AI open-sources a HIP attention kernel for AMD MI300X that beats
AITER v3" (benchmark paragraph, and the numerics paragraph before it) measures
its bf16 attention output under three rounding rules for the final conversion:

* RTNE: round to the nearest bf16 value, a tie going to the one whose last
  significand bit is 0;
* RTNA: round to the nearest bf16 value, a tie going to the one of larger
  magnitude (away from zero);
* RTZ: truncate toward zero (the bf16 value of largest magnitude not above
  |x|, with x's sign).

The function below applies a rule to float64 values directly from these
definitions: it scales |x| by the bf16 spacing of its binade (8 significant
bits; below 2^-126 the spacing stays 2^-133, the subnormal range) and rounds the
quotient to an integer.  Values beyond the largest finite bf16, (2 - 2^-7) *
2^127, go to infinity under the two nearest rules when they are at least half
a spacing above it, and to the largest finite value under RTZ.  Zeros and
infinities keep their sign; NaN stays NaN.
"""
from __future__ import annotations

import numpy as np

MODES = ("rtne", "rtna", "rtz")
BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def spacing(a: np.ndarray) -> np.ndarray:
    """bf16 spacing (one unit in the last place) at magnitude a > 0."""
    _, e2 = np.frexp(a)                      # a = f * 2^e2, f in [0.5, 1)
    e = np.maximum(e2.astype(np.int64) - 1, -126)
    return np.ldexp(1.0, (e - 7).astype(np.int32))


def round_bf16(x, mode: str) -> np.ndarray:
    """Round float64 values to bf16 under `mode` ('rtne', 'rtna' or 'rtz');
    returns float64 values that bf16 represents exactly."""
    if mode not in MODES:
        raise ValueError(f"unknown rounding mode {mode!r}")
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, dtype=np.float64, copy=True)
    fin = np.isfinite(x) & (x != 0)
    a = np.abs(x[fin])
    u = spacing(a)
    q = a / u                                # exact: u is a power of two
    n = np.floor(q)
    frac = q - n                             # exact: n < 2^9
    if mode == "rtz":
        r = n
    elif mode == "rtna":
        r = n + (frac >= 0.5)
    else:
        odd = np.mod(n, 2) == 1
        r = n + ((frac > 0.5) | ((frac == 0.5) & odd))
    mag = r * u
    if mode == "rtz":
        mag = np.minimum(mag, BF16_MAX)
    else:
        mag = np.where(mag > BF16_MAX, np.inf, mag)
    out[fin] = np.copysign(mag, x[fin])
    return out


def bf16_bits(values) -> np.ndarray:
    """uint16 bit patterns of values that bf16 represents exactly (as returned
    by round_bf16); NaN maps to the quiet NaN with the value's sign."""
    v = np.asarray(values, dtype=np.float64)
    f = v.astype(np.float32)
    if not np.array_equal(f.astype(np.float64), v, equal_nan=True):
        raise ValueError("value not representable in float32")
    bits = f.view(np.uint32)
    if np.any((bits & 0xFFFF)[~np.isnan(v)] != 0):
        raise ValueError("value not representable in bf16")
    out = (bits >> 16).astype(np.uint16)
    nan = np.isnan(v)
    out[nan] = ((bits[nan] >> 16) & 0x8000 | 0x7FC0).astype(np.uint16)
    return out
