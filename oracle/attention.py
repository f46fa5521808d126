"""Materialised fp64 attention: the oracle (TEST INFRASTRUCTURE ONLY).

Only tests/, the smoke check and the benchmark's CPU-baseline leg may use this
module; the library never does.

What it computes, and where the pages define it:

* Attention is the fused operation softmax(Q K^T / sqrt(d)) V ("MoonMath AI
  open-sources a HIP attention kernel for AMD MI300X that beats AITER v3",
  definition paragraph), here with a caller-given scale (the default
  1/sqrt(d) is the one in "IO-aware tiling strategy in FlashAttention-4",
  checklist item 2).  The plain, materialised form builds the full score matrix
  S = scale*Q*K^T, takes a row softmax and multiplies by V ("IO-aware tiling
  strategy in FlashAttention-4", body, second paragraph).
* Several query heads share one K/V head (MQA/GQA: "Engineering the
  FlashAttention-4 kernel port to ROCm", section on vendor-agnostic multi-query
  inference).  Reading taken: contiguous groups, kv = h // (Hq / Hkv).
* Causal masking keeps the lower triangle ("Reverse engineering Flash Attention
  4's proprietary fused attention kernel", point 1, the upper_triangular mask).
  Reading taken when Sq != Sk: bottom-right alignment, key j is visible from
  query i iff j <= i + (Sk - Sq).  A row with no visible key returns O = 0 and
  LSE = -inf.
* ALiBi (optional): a per-query-head linear bias -slope * |i + Sk - Sq - j|
  added to the scaled scores before the softmax (see ``alibi_bias``).
* LSE is the natural log of the softmax denominator over visible keys,
  m + ln(l), the statistics the pages say are kept ("Reverse engineering ...",
  point 2; "IO-aware tiling ...", backward-pass paragraph).
* Packed sequences (variable-length batches): each sequence is its own
  problem of the definition above, with its own lengths.
* Paged decode: K/V of sequence b live in 16-token pages listed by an int32
  block table ("Engineering the FlashAttention-4 kernel port to ROCm",
  multi-query section, paged KV cache); the oracle gathers them into a dense
  [len_b, Hkv, d] tensor and applies the same definition with one query row.

Inputs are the bf16 bit patterns the GPU sees, upcast exactly to float64; the
scale is rounded to float32 first, as the library receives it.  Everything else
is float64.  Rows are independent, so computing them in chunks changes nothing.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
from threadpoolctl import threadpool_limits

BSHD = 0
BHSD = 1
PAGE = 16


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact upcast of bf16 bit patterns (uint16) to float64."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def scale_as_f32(scale: float) -> float:
    """The library takes the scale as a float32; the oracle uses that value."""
    return float(np.float32(scale))


def kv_head_of(h: int, Hq: int, Hkv: int) -> int:
    """Query head h reads K/V head h // (Hq/Hkv) (contiguous GQA groups)."""
    return h // (Hq // Hkv)


def visible_keys(i: int, Sq: int, Sk: int, causal: bool) -> int:
    """Number of keys (a prefix 0..n-1) that query row i attends to."""
    if not causal:
        return Sk
    return max(0, min(Sk, i + (Sk - Sq) + 1))


def scores(q: np.ndarray, k: np.ndarray, scale: float) -> np.ndarray:
    """S = scale * Q K^T for q [n, d], k [Sk, d] -> [n, Sk]."""
    return scale * (q @ k.T)


def row_softmax(s: np.ndarray):
    """Row softmax of s (entries -inf are masked).  Returns (P, m, l) with
    m the row max and l = sum_j exp(s_ij - m); an all-masked row has P = 0,
    m = -inf, l = 0."""
    m = s.max(axis=1)
    empty = m == -np.inf
    m_safe = np.where(empty, 0.0, m)
    e = np.exp(s - m_safe[:, None])
    l = e.sum(axis=1)
    p = e / np.where(empty, 1.0, l)[:, None]
    return p, m, l


def alibi_bias(rows, Sq, Sk, slope):
    """ALiBi bias of query rows `rows` against keys 0..Sk-1: -slope * |i + Sk
    - Sq - j| (linear in the distance from the row's own position; the query
    positions are aligned to the end of the keys, as the causal mask is).
    The IO-aware tiling page asks that ALiBi positional biases be supported
    ("IO-aware tiling strategy in FlashAttention-4", integration paragraph);
    the bias itself is not defined there."""
    i = np.asarray(rows, np.float64)[:, None]
    j = np.arange(Sk, dtype=np.float64)[None, :]
    return -float(slope) * np.abs(i + (Sk - Sq) - j)


def attend_rows(q, k, v, scale, n_visible=None, bias=None):
    """Materialised attention for query rows q [n, d] against k, v [Sk, d]
    (float64).  n_visible[i] limits row i to keys 0..n_visible[i]-1; bias
    [n, Sk], if given, is added to the scaled scores.  Returns (o [n, d],
    lse [n])."""
    if k.shape[0] == 0:  # no key at all: every row is empty
        return np.zeros((q.shape[0], v.shape[1])), np.full(q.shape[0], -np.inf)
    s = scores(q, k, scale)
    if bias is not None:
        s = s + bias
    if n_visible is not None:
        j = np.arange(k.shape[0])
        s = np.where(j[None, :] >= np.asarray(n_visible)[:, None], -np.inf, s)
    p, m, l = row_softmax(s)
    o = p @ v
    with np.errstate(divide="ignore"):
        lse = np.where(m == -np.inf, -np.inf, m + np.log(np.where(l > 0, l, 1.0)))
    return o, lse


def _logical(x, layout):
    """View a [B,S,H,D] (BSHD) or [B,H,S,D] (BHSD) array as [B,H,S,D]."""
    return x.transpose(0, 2, 1, 3) if layout == BSHD else x


def _workers():
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def attention(q_bits, k_bits, v_bits, B, Hq, Hkv, Sq, Sk, scale, causal, layout,
              chunk=256, workers=None, alibi_slopes=None):
    """Full prefill oracle.  Returns (o [B, Hq, Sq, D] float64 in logical
    head-major order, lse [B, Hq, Sq] float64).  alibi_slopes [Hq] (float32
    values, used as float64), if given, adds ``alibi_bias`` with query head
    h's slope to the scaled scores."""
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    qv = _logical(q_bits, layout)
    kv = _logical(k_bits, layout)
    vv = _logical(v_bits, layout)
    d = q_bits.shape[-1]
    sc = scale_as_f32(scale)
    o = np.zeros((B, Hq, Sq, d), np.float64)
    lse = np.zeros((B, Hq, Sq), np.float64)
    nvis = np.array([visible_keys(i, Sq, Sk, causal) for i in range(Sq)], np.int64)

    def job(b, h, i0):
        g = kv_head_of(h, Hq, Hkv)
        i1 = min(Sq, i0 + chunk)
        kmax = int(nvis[i0:i1].max()) if causal else Sk
        qq = bf16_to_f64(qv[b, h, i0:i1])
        kk = bf16_to_f64(kv[b, g, :kmax])
        vv_ = bf16_to_f64(vv[b, g, :kmax])
        bias = None
        if alibi_slopes is not None:
            bias = alibi_bias(np.arange(i0, i1), Sq, Sk, alibi_slopes[h])[:, :kmax]
        oo, ll = attend_rows(qq, kk, vv_, sc, np.minimum(nvis[i0:i1], kmax), bias)
        o[b, h, i0:i1] = oo
        lse[b, h, i0:i1] = ll

    jobs = [(b, h, i0) for b in range(B) for h in range(Hq) for i0 in range(0, Sq, chunk)]
    _run(job, jobs, workers)
    return o, lse


def attention_sampled(q_bits, k_bits, v_bits, B, Hq, Hkv, Sq, Sk, scale, causal,
                      layout, samples, workers=None):
    """Oracle outputs for selected query rows only.  samples: list of
    (b, h, i).  Returns (o [n, D], lse [n]) in the order given."""
    qv = _logical(q_bits, layout)
    kv = _logical(k_bits, layout)
    vv = _logical(v_bits, layout)
    sc = scale_as_f32(scale)
    d = q_bits.shape[-1]
    o = np.zeros((len(samples), d), np.float64)
    lse = np.zeros(len(samples), np.float64)
    # group rows by (b, h) so each K/V head is upcast once per group
    groups = {}
    for n, (b, h, i) in enumerate(samples):
        groups.setdefault((b, h), []).append((n, i))

    def job(b, h):
        g = kv_head_of(h, Hq, Hkv)
        items = groups[(b, h)]
        rows = np.array([i for _, i in items])
        nv = np.array([visible_keys(int(i), Sq, Sk, causal) for i in rows])
        kmax = int(nv.max())
        qq = bf16_to_f64(qv[b, h, rows])
        kk = bf16_to_f64(kv[b, g, :kmax])
        vv_ = bf16_to_f64(vv[b, g, :kmax])
        oo, ll = attend_rows(qq, kk, vv_, sc, nv)
        for r, (n, _) in enumerate(items):
            o[n] = oo[r]
            lse[n] = ll[r]

    _run(job, list(groups.keys()), workers)
    return o, lse


def attention_varlen(q_bits, k_bits, v_bits, cu_q, cu_k, Hkv, scale, causal, workers=None):
    """Oracle for packed sequences of different lengths: sequence b is query
    rows cu_q[b]..cu_q[b+1]-1 of q [total_q, Hq, D] against key rows
    cu_k[b]..cu_k[b+1]-1 of k, v [total_k, Hkv, D], each sequence being one
    problem of the definition above with its own lengths (causal alignment
    per sequence).  Variable-length batching is what the MoonMath page lists
    among its kernel's limits ("MoonMath AI open-sources a HIP attention
    kernel for AMD MI300X that beats AITER v3", limitations paragraph).
    Returns (o [total_q, Hq, D], lse [Hq, total_q]) float64."""
    total_q, Hq, d = q_bits.shape
    sc = scale_as_f32(scale)
    o = np.zeros((total_q, Hq, d), np.float64)
    lse = np.full((Hq, total_q), -np.inf)

    def job(b):
        q0, q1 = int(cu_q[b]), int(cu_q[b + 1])
        k0, k1 = int(cu_k[b]), int(cu_k[b + 1])
        sq, sk = q1 - q0, k1 - k0
        if sq == 0:
            return
        nv = np.array([visible_keys(i, sq, sk, causal) for i in range(sq)], np.int64)
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            oo, ll = attend_rows(bf16_to_f64(q_bits[q0:q1, h]), bf16_to_f64(k_bits[k0:k1, g]),
                                 bf16_to_f64(v_bits[k0:k1, g]), sc, nv)
            o[q0:q1, h] = oo
            lse[h, q0:q1] = ll

    _run(job, list(range(len(cu_q) - 1)), workers)
    return o, lse


def gather_pages(pool_bits, block_table, seq_len, b, g):
    """Dense [len, D] view of KV head g of sequence b from a paged pool
    [num_pages, 16, Hkv, D]: token t lives in page block_table[b, t // 16],
    slot t % 16."""
    t = np.arange(int(seq_len))
    pages = block_table[b, t // PAGE]
    return pool_bits[pages, t % PAGE, g]


def decode_paged(q_bits, k_pool, v_pool, block_table, seq_lens, Hkv, scale,
                 workers=None):
    """Paged decode oracle: one query row per (b, h) against all seq_lens[b]
    cached tokens.  Returns (o [B, Hq, D], lse [B, Hq]) float64."""
    B, Hq, d = q_bits.shape
    sc = scale_as_f32(scale)
    o = np.zeros((B, Hq, d), np.float64)
    lse = np.zeros((B, Hq), np.float64)

    def job(b):
        n = int(seq_lens[b])
        for g in range(Hkv):
            kk = bf16_to_f64(gather_pages(k_pool, block_table, n, b, g))
            vv = bf16_to_f64(gather_pages(v_pool, block_table, n, b, g))
            heads = [h for h in range(Hq) if kv_head_of(h, Hq, Hkv) == g]
            oo, ll = attend_rows(bf16_to_f64(q_bits[b, heads]), kk, vv, sc)
            o[b, heads] = oo
            lse[b, heads] = ll

    _run(job, list(range(B)), workers)
    return o, lse


def append_token(k_pool, v_pool, block_table, seq_lens, k_new, v_new):
    """KV-cache append: the current token of sequence b is token seq_lens[b]-1
    (the lengths count it), and its K and V rows k_new[b], v_new[b] ([Hkv, D]
    bf16 bits) go to slot (len-1) % 16 of page block_table[b, (len-1) // 16]
    of the paged pools ("Engineering the FlashAttention-4 kernel port to
    ROCm", multi-query section, for the paged format; "Reverse engineering
    Flash Attention 4's proprietary fused attention kernel", first point, for
    updating the shared KV cache together with the attention).  Returns
    updated copies of the pools."""
    kp = k_pool.copy()
    vp = v_pool.copy()
    for b in range(len(seq_lens)):
        t = int(seq_lens[b]) - 1
        page = block_table[b, t // PAGE]
        kp[page, t % PAGE] = k_new[b]
        vp[page, t % PAGE] = v_new[b]
    return kp, vp


def decode_paged_append(q_bits, k_new, v_new, k_pool, v_pool, block_table, seq_lens, Hkv,
                        scale, workers=None):
    """Append the current token's K/V to the cache, then the paged decode over
    every token including it.  Returns (o, lse, k_pool', v_pool')."""
    kp, vp = append_token(k_pool, v_pool, block_table, seq_lens, k_new, v_new)
    o, lse = decode_paged(q_bits, kp, vp, block_table, seq_lens, Hkv, scale, workers)
    return o, lse, kp, vp


def _run(fn, jobs, workers):
    workers = workers or _workers()
    if workers == 1 or len(jobs) == 1:
        for j in jobs:
            fn(*j) if isinstance(j, tuple) else fn(j)
        return
    # one BLAS thread per worker: the parallelism is over independent rows
    with threadpool_limits(limits=1, user_api="blas"), \
            ThreadPoolExecutor(max_workers=workers) as ex:
        futs = [ex.submit(fn, *j) if isinstance(j, tuple) else ex.submit(fn, j) for j in jobs]
        for f in futs:
            f.result()


def flops_prefill(B, Hq, Sq, Sk, d, causal):
    """Algorithmic FLOP of the forward: 4*B*Hq*Sq*Sk*d, halved when causal."""
    f = 4.0 * B * Hq * Sq * Sk * d
    return f / 2 if causal else f


__all__ = ["bf16_to_f64", "scale_as_f32", "kv_head_of", "visible_keys", "scores",
           "row_softmax", "alibi_bias", "attend_rows", "attention", "attention_sampled", "attention_varlen",
           "gather_pages", "decode_paged", "append_token", "decode_paged_append",
           "flops_prefill"]
