"""Parity tolerance for bf16 outputs against the fp64 oracle.

|O - O_ref| <= 2 * ulp_bf16(|O_ref|) + 1e-3 elementwise, and
|LSE - LSE_ref| <= 1e-3, where ulp_bf16(x) = 2^(max(floor(log2 x), -126) - 7)
for x > 0 and 2^-133 at 0 (bf16 keeps 8 significant bits).
"""
from __future__ import annotations

import numpy as np

O_ABS = 1e-3
LSE_ABS = 1e-3


def ulp_bf16(x: np.ndarray) -> np.ndarray:
    x = np.abs(np.asarray(x, dtype=np.float64))
    out = np.full(x.shape, 2.0 ** -133)
    nz = x > 0
    e = np.floor(np.log2(x[nz]))
    # guard log2 rounding at exact powers of two
    e = np.where(2.0 ** e > x[nz], e - 1, e)
    e = np.where(2.0 ** (e + 1) <= x[nz], e + 1, e)
    out[nz] = 2.0 ** (np.maximum(e, -126) - 7)
    return out


def o_tolerance(o_ref: np.ndarray) -> np.ndarray:
    return 2.0 * ulp_bf16(o_ref) + O_ABS


def check_o(o, o_ref, what=""):
    """Assert elementwise O parity; returns (max_err, max err/tol)."""
    o = np.asarray(o, dtype=np.float64)
    o_ref = np.asarray(o_ref, dtype=np.float64)
    assert o.shape == o_ref.shape, (o.shape, o_ref.shape)
    assert np.all(np.isfinite(o)), f"{what}: non-finite output"
    err = np.abs(o - o_ref)
    tol = o_tolerance(o_ref)
    ratio = err / tol
    worst = np.unravel_index(np.argmax(ratio), ratio.shape)
    assert ratio.max() <= 1.0, (
        f"{what}: O mismatch at {worst}: got {o[worst]!r} ref {o_ref[worst]!r} "
        f"err {err[worst]:.3g} tol {tol[worst]:.3g}")
    return float(err.max()), float(ratio.max())


def check_lse(lse, lse_ref, what=""):
    lse = np.asarray(lse, dtype=np.float64)
    lse_ref = np.asarray(lse_ref, dtype=np.float64)
    assert lse.shape == lse_ref.shape
    ninf = lse_ref == -np.inf
    assert np.all(lse[ninf] == -np.inf), f"{what}: empty rows must give LSE=-inf"
    err = np.abs(lse[~ninf] - lse_ref[~ninf])
    if err.size:
        i = int(np.argmax(err))
        assert err.max() <= LSE_ABS, f"{what}: LSE err {err[i]:.3g} at flat {i}"
        return float(err.max())
    return 0.0
