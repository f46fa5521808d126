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


# ---------------------------------------------------------------------------
# Large V.  The bound above assumes |V| of order one.  The kernels round the
# probabilities that multiply V to fp16 (unit roundoff u = 2^-11; bf16,
# u = 2^-8, on the fallback for V beyond the fp16 range) and divide by the sum
# of the same rounded values.  With p~_j = p_j (1 + e_j) the computed output is,
# to first order in u,
#     O~ - O = sum_j pi_j e_j (v_j - O),      pi_j = p_j / l,
# so |O~ - O| <= sum_j max(u pi_j, 2^-25 / l) |v_j - O|, where 2^-25 (half
# the fp16 subnormal spacing, probabilities taken against the row max) bounds
# the error of a probability that falls among the fp16 subnormals.  When a row
# nearly cancels (|O| << sum_j pi_j |v_j|) this exceeds 1e-3 as soon as |V| is
# large, whatever the kernel does, so large-V inputs are checked against
#     |O - O_ref| <= 2 ulp_bf16(|O_ref|) + 1e-3 + (1 + 2^-4) * spread,
#     spread = sum_j max(u pi_j, 2^-25 / l) |v_j - O_ref|
# (the factor 1 + 2^-4 covers the second-order terms and the fp32
# accumulation).  LSE does not depend on V; it keeps its bound where the
# probabilities are fp16 (l moves by at most 2^-11 relative).  On the bf16
# fallback l sums bf16-rounded probabilities: l~/l - 1 = sum_j pi_j e_j with
# |e_j| <= 2^-8, so LSE is checked against 1e-3 + 2^-8 there
# (check_lse_bf16_fallback).

P_UNIT_F16 = 2.0 ** -11
P_UNIT_BF16 = 2.0 ** -8
P_SUB_F16 = 2.0 ** -25


def pv_spread_rows(q, k, v, scale, n_visible=None, unit=P_UNIT_F16, bias=None):
    """spread for query rows q [n, d] against keys k, values v [Sk, d]
    (float64), row i limited to keys 0..n_visible[i]-1; bias [n, Sk] (an
    ALiBi bias) is added to the scaled scores, so pi are the probabilities of
    the biased scores.  Returns [n, d]."""
    import oracle.attention as att
    n, d = q.shape[0], v.shape[1]
    if k.shape[0] == 0:
        return np.zeros((n, d))
    s = att.scores(q, k, scale)
    if bias is not None:
        s = s + bias
    if n_visible is not None:
        j = np.arange(k.shape[0])
        s = np.where(j[None, :] >= np.asarray(n_visible)[:, None], -np.inf, s)
    p, m, l = att.row_softmax(s)          # p = pi (normalised), l against the row max
    o = p @ v
    lsafe = np.where(l > 0, l, 1.0)
    w = np.maximum(unit * p, np.where(p > 0, P_SUB_F16 / lsafe[:, None], 0.0))
    spread = np.zeros((n, d))
    for c in range(d):
        spread[:, c] = (w * np.abs(v[None, :, c] - o[:, c:c + 1])).sum(axis=1)
    return spread


def pv_spread_prefill(p, unit=P_UNIT_F16, alibi_slopes=None):
    """spread [B, Hq, Sq, d] for a generator prefill problem (bf16 bits),
    with the ALiBi bias of query head h when alibi_slopes [Hq] is given."""
    import oracle.attention as att
    qv = att._logical(p.q, p.layout)
    kv = att._logical(p.k, p.layout)
    vv = att._logical(p.v, p.layout)
    sc = att.scale_as_f32(p.scale)
    nvis = np.array([att.visible_keys(i, p.Sq, p.Sk, p.causal) for i in range(p.Sq)])
    out = np.zeros((p.B, p.Hq, p.Sq, p.q.shape[-1]))
    for b in range(p.B):
        for h in range(p.Hq):
            g = att.kv_head_of(h, p.Hq, p.Hkv)
            bias = None
            if alibi_slopes is not None:
                bias = att.alibi_bias(np.arange(p.Sq), p.Sq, p.Sk, alibi_slopes[h])
            out[b, h] = pv_spread_rows(att.bf16_to_f64(qv[b, h]), att.bf16_to_f64(kv[b, g]),
                                       att.bf16_to_f64(vv[b, g]), sc, nvis, unit, bias)
    return out


def check_lse_bf16_fallback(lse, lse_ref, what=""):
    """LSE of a problem that ran with bf16 probabilities (V beyond the fp16
    range): |LSE - LSE_ref| <= 1e-3 + 2^-8, -inf rows exact."""
    lse = np.asarray(lse, dtype=np.float64)
    lse_ref = np.asarray(lse_ref, dtype=np.float64)
    assert lse.shape == lse_ref.shape
    ninf = lse_ref == -np.inf
    assert np.all(lse[ninf] == -np.inf), f"{what}: empty rows must give LSE=-inf"
    err = np.abs(lse[~ninf] - lse_ref[~ninf])
    if err.size:
        i = int(np.argmax(err))
        assert err.max() <= LSE_ABS + P_UNIT_BF16, f"{what}: LSE err {err[i]:.3g} at flat {i}"
        return float(err.max())
    return 0.0


def check_o_large_v(o, o_ref, spread, what=""):
    """Assert O parity under the large-V bound; returns (max_err, max err/tol,
    max err/tol under the plain bound) -- the last is for reporting only."""
    o = np.asarray(o, dtype=np.float64)
    o_ref = np.asarray(o_ref, dtype=np.float64)
    assert o.shape == o_ref.shape == spread.shape, (o.shape, o_ref.shape, spread.shape)
    assert np.all(np.isfinite(o)), f"{what}: non-finite output"
    err = np.abs(o - o_ref)
    tol = o_tolerance(o_ref) + (1.0 + 2.0 ** -4) * spread
    ratio = err / tol
    worst = np.unravel_index(np.argmax(ratio), ratio.shape)
    assert ratio.max() <= 1.0, (
        f"{what}: O mismatch at {worst}: got {o[worst]!r} ref {o_ref[worst]!r} "
        f"err {err[worst]:.3g} tol {tol[worst]:.3g}")
    return float(err.max()), float(ratio.max()), float((err / o_tolerance(o_ref)).max())
