"""FP8 (E4M3) inputs for the attention forward, in float64 (TEST
INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline use it; the library never does).

The pages name FP8 inputs only in passing: one says the Blackwell-specific
FP8 handling has to fall back to FP16 when the kernel moves to ROCm ("Engineering
the FlashAttention-4 kernel port to ROCm", section on the HIP migration), another
lists low-precision FP8 as a way to cut HBM traffic where the hardware has it
("IO-aware tiling strategy in FlashAttention-4", monitoring paragraph).  They fix
neither the format nor a scaling rule.  Readings taken:

* the format is the OCP 8-bit E4M3 ("FN" variant) that gfx950 computes with:
  1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0
  holds the subnormals m/8 * 2^-6; exponent field 15 is an ordinary binade
  except that mantissa 7 there is NaN; there is no infinity (largest finite
  value 448);
* each of Q, K and V carries one float32 descale factor for the whole tensor,
  so the attention is computed on the real values descale_q*q, descale_k*k,
  descale_v*v: exactly the forward of ``oracle.attention`` on those values
  (same scale, GQA mapping, causal alignment, empty-row rule), O and LSE
  defined as there.
"""
from __future__ import annotations

import numpy as np

from .attention import (_logical, _run, attend_rows, kv_head_of, scale_as_f32,
                        visible_keys)

E4M3_BIAS = 7


def e4m3_to_f64(b: np.ndarray) -> np.ndarray:
    """Decode OCP E4M3 (FN) bytes to float64, exactly (every E4M3 value is a
    float64)."""
    b = np.asarray(b, dtype=np.uint8).astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - E4M3_BIAS)
    sub = (m / 8.0) * 2.0 ** (1 - E4M3_BIAS)
    val = sign * np.where(e == 0, sub, normal)
    return np.where((e == 0xF) & (m == 7), np.nan, val)


def attention_fp8(q8, k8, v8, descale_q, descale_k, descale_v, B, Hq, Hkv, Sq, Sk, scale,
                  causal, layout, rows=None, chunk=256, workers=None):
    """The forward on E4M3 inputs (uint8 arrays in `layout`, BSHD or BHSD)
    with per-tensor float32 descales.  Returns (o [B, Hq, Sq, D], lse
    [B, Hq, Sq]) in float64, logical head-major order.  rows, if given, is a
    list of (b, h, i) query rows: only those are computed (the rest stay
    NaN)."""
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    dq, dk, dv = (float(np.float32(x)) for x in (descale_q, descale_k, descale_v))
    qv, kv, vv = _logical(q8, layout), _logical(k8, layout), _logical(v8, layout)
    d = q8.shape[-1]
    sc = scale_as_f32(scale)
    o = np.full((B, Hq, Sq, d), np.nan)
    lse = np.full((B, Hq, Sq), np.nan)
    nvis = np.array([visible_keys(i, Sq, Sk, causal) for i in range(Sq)], np.int64)

    def job(b, h, idx):
        g = kv_head_of(h, Hq, Hkv)
        kmax = int(nvis[idx].max()) if causal else Sk
        qq = dq * e4m3_to_f64(qv[b, h, idx])
        kk = dk * e4m3_to_f64(kv[b, g, :kmax])
        vv_ = dv * e4m3_to_f64(vv[b, g, :kmax])
        oo, ll = attend_rows(qq, kk, vv_, sc, np.minimum(nvis[idx], kmax))
        o[b, h, idx] = oo
        lse[b, h, idx] = ll

    if rows is None:
        jobs = [(b, h, np.arange(i0, min(Sq, i0 + chunk)))
                for b in range(B) for h in range(Hq) for i0 in range(0, Sq, chunk)]
    else:
        by = {}
        for b, h, i in rows:
            by.setdefault((b, h), []).append(i)
        jobs = [(b, h, np.array(sorted(set(ii)), np.int64)) for (b, h), ii in by.items()]
    _run(job, jobs, workers)
    return o, lse
