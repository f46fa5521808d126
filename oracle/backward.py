"""Gradient of exact attention in float64: the backward oracle (TEST
INFRASTRUCTURE ONLY).

Only tests/, the smoke check and the benchmark's CPU-baseline leg may use this
module; the library never does.

What it computes, and where the pages fix it:

* The backward pass keeps only the per-row softmax statistics of the forward
  and recomputes the score and probability tiles from them instead of storing
  P ("IO-aware tiling strategy in FlashAttention-4", the paragraph on the
  backward pass; "Reverse engineering Flash Attention 4's proprietary fused
  attention kernel", point 2, recompute of S/P from max_log and row_sum).
  That is how the GPU path works.  What it must produce is fixed by the
  forward's definition alone: the gradient of L = sum(dO * O) with respect to
  Q, K and V, where O = softmax(scale * Q K^T, masked) V is the forward of
  ``oracle.attention`` (same GQA head mapping, same bottom-right causal
  alignment, same empty-row rule).
* This module writes that gradient out by the chain rule on the materialised
  matrices of one (batch, query head):
      P  = row softmax of S = scale * Q K^T (masked entries -inf, P = 0 there)
      dV = P^T dO
      dP = dO V^T
      dS = P * (dP - rowsum(P * dP))        (Jacobian of the row softmax)
      dQ = scale * dS K,   dK = scale * dS^T Q
  and a K/V head's gradients are the sums over the query heads that read it.
  The row sum rowsum(P * dP) equals dO_i . O_i in exact arithmetic; the
  oracle uses the former (the Jacobian as defined), the GPU the latter.
* A row with no visible key has O = 0 whatever Q, K, V are: its dQ is zero
  and it adds nothing to dK or dV.

Inputs are bf16 bit patterns (uint16, upcast exactly) or float64 arrays (used
by the finite-difference pins); the scale is rounded to float32 first, as the
library receives it.  Everything else is float64.  Row chunks only split the
sums over query rows of dK and dV.
"""
from __future__ import annotations

import numpy as np

from .attention import (BHSD, BSHD, _logical, _run, alibi_bias, bf16_to_f64,  # noqa: F401
                        kv_head_of, row_softmax, scale_as_f32, scores, visible_keys)


def as_f64(x: np.ndarray) -> np.ndarray:
    """bf16 bits (uint16) upcast exactly; float arrays taken as float64."""
    if x.dtype == np.uint16:
        return bf16_to_f64(x)
    return np.asarray(x, dtype=np.float64)


def probabilities(q, k, scale, n_visible=None, bias=None):
    """P [n, Sk] of query rows q [n, d] against keys k [Sk, d], with row i
    limited to keys 0..n_visible[i]-1 (all-masked rows give P = 0) and bias
    [n, Sk] (ALiBi), if given, added to the scaled scores."""
    s = scores(q, k, scale)
    if bias is not None:
        s = s + bias
    if n_visible is not None:
        j = np.arange(k.shape[0])
        s = np.where(j[None, :] >= np.asarray(n_visible)[:, None], -np.inf, s)
    p, _, _ = row_softmax(s)
    return p


def grad_rows(q, k, v, do, scale, n_visible=None, bias=None):
    """Gradient of sum(do * O) for O = attention of query rows q [n, d]
    against k, v [Sk, d] (float64).  A bias (constant in Q, K, V) enters only
    P.  Returns (dq [n, d], dk [Sk, d], dv [Sk, d])."""
    p = probabilities(q, k, scale, n_visible, bias)
    dv = p.T @ do
    dp = do @ v.T
    ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    return dq, dk, dv


def grad_magnitudes(q, k, v, do, scale, n_visible=None, bias=None):
    """Sums of absolute terms behind each gradient entry, the scale of its
    rounding error when the products are formed from bf16-rounded operands
    (P, dS) and the row term from a rounded O.  With
    Dabs_i = sum_c |dO_ic O_ic| and A = P * (|dP| + Dabs):
        mdv = P^T |dO|,  mdq = scale * A |K|,  mdk = scale * A^T |Q|.
    Returns (mdq [n, d], mdk [Sk, d], mdv [Sk, d])."""
    p = probabilities(q, k, scale, n_visible, bias)
    o = p @ v
    dabs = np.abs(do * o).sum(axis=1, keepdims=True)
    a = p * (np.abs(do @ v.T) + dabs)
    return scale * (a @ np.abs(k)), scale * (a.T @ np.abs(q)), p.T @ np.abs(do)


def attention_backward(q_in, k_in, v_in, do_in, B, Hq, Hkv, Sq, Sk, scale, causal, layout,
                       chunk=512, workers=None, magnitudes=False, alibi_slopes=None):
    """Full backward oracle.  q_in/do_in: [B,Sq,Hq,D] (BSHD) or [B,Hq,Sq,D]
    (BHSD); k_in/v_in likewise with Hkv heads and Sk rows.  Returns
    (dq [B,Hq,Sq,D], dk [B,Hkv,Sk,D], dv [B,Hkv,Sk,D]) float64 in logical
    head-major order, followed by the three magnitude arrays of
    ``grad_magnitudes`` (same shapes) when magnitudes=True.  alibi_slopes
    [Hq]: the forward had the ALiBi bias of ``oracle.attention.alibi_bias``."""
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    qv, kv, vv, dov = (_logical(x, layout) for x in (q_in, k_in, v_in, do_in))
    d = q_in.shape[-1]
    sc = scale_as_f32(scale)
    dq = np.zeros((B, Hq, Sq, d))
    dk = np.zeros((B, Hkv, Sk, d))
    dv = np.zeros((B, Hkv, Sk, d))
    if magnitudes:
        mq, mk, mv = np.zeros_like(dq), np.zeros_like(dk), np.zeros_like(dv)
    nvis = np.array([visible_keys(i, Sq, Sk, causal) for i in range(Sq)], np.int64)

    def job(b, g):
        kk = as_f64(kv[b, g])
        vv_ = as_f64(vv[b, g])
        for h in range(Hq):
            if kv_head_of(h, Hq, Hkv) != g:
                continue
            for i0 in range(0, Sq, chunk):
                i1 = min(Sq, i0 + chunk)
                bias = None
                if alibi_slopes is not None:
                    bias = alibi_bias(np.arange(i0, i1), Sq, Sk, alibi_slopes[h])
                args = (as_f64(qv[b, h, i0:i1]), kk, vv_, as_f64(dov[b, h, i0:i1]), sc,
                        nvis[i0:i1], bias)
                gq, gk, gv = grad_rows(*args)
                dq[b, h, i0:i1] = gq
                dk[b, g] += gk
                dv[b, g] += gv
                if magnitudes:
                    aq, ak, av = grad_magnitudes(*args)
                    mq[b, h, i0:i1] = aq
                    mk[b, g] += ak
                    mv[b, g] += av

    _run(job, [(b, g) for b in range(B) for g in range(Hkv)], workers)
    if magnitudes:
        return dq, dk, dv, mq, mk, mv
    return dq, dk, dv


def attention_backward_varlen(q_in, k_in, v_in, do_in, cu_q, cu_k, Hkv, scale, causal,
                              workers=None, magnitudes=False):
    """Backward oracle for packed sequences (the forward of
    ``oracle.attention.attention_varlen``): each sequence's gradients are
    those of its own problem.  q_in/do_in [total_q, Hq, D], k_in/v_in
    [total_k, Hkv, D] (bf16 bits or float64).  Returns (dq, dk, dv) in the
    packed layouts, then the three magnitude arrays when magnitudes=True."""
    total_q, Hq, d = q_in.shape
    total_k = k_in.shape[0]
    outs = [np.zeros((total_q, Hq, d)), np.zeros((total_k, Hkv, d)), np.zeros((total_k, Hkv, d))]
    if magnitudes:
        outs += [np.zeros_like(outs[0]), np.zeros_like(outs[1]), np.zeros_like(outs[2])]
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        if q1 == q0 or k1 == k0:
            continue   # no row sees a key: every gradient of the sequence is 0
        r = attention_backward(q_in[q0:q1][None], k_in[k0:k1][None], v_in[k0:k1][None],
                               do_in[q0:q1][None], 1, Hq, Hkv, q1 - q0, k1 - k0, scale, causal,
                               BSHD, workers=workers, magnitudes=magnitudes)
        for i, x in enumerate(r):
            rows = slice(q0, q1) if i % 3 == 0 else slice(k0, k1)
            outs[i][rows] = x[0].transpose(1, 0, 2)
    return tuple(outs)


def flops_backward(B, Hq, Sq, Sk, d, causal):
    """Algorithmic FLOP of the backward: the five products (S recomputed,
    dP, dV, dQ, dK) of 2*Sq*Sk*d each per head, 10*B*Hq*Sq*Sk*d, halved when
    causal."""
    f = 10.0 * B * Hq * Sq * Sk * d
    return f / 2 if causal else f


__all__ = ["as_f64", "probabilities", "grad_rows", "grad_magnitudes", "attention_backward",
           "attention_backward_varlen", "flops_backward"]
