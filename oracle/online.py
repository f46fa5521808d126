"""Float64 model of the blockwise online softmax and of the split-KV merge
(TEST INFRASTRUCTURE ONLY; used to pin the materialised oracle, never by the
library).

"IO-aware tiling strategy in FlashAttention-4" (body, third paragraph) keeps,
per query row, a running max m and denominator l while K/V blocks stream by,
and merges a new block with m' = max(m, m_new), l' = l*exp(m - m') + l_new.
As printed, the rule only holds if l_new is the block's sum of exp(s - m'),
i.e. taken after the max update; that is the reading modelled here.  The
output accumulator is multiplied by the same per-row factor exp(m - m') and is
divided by l once, at the end.

The split-KV merge ("MoonMath AI open-sources a HIP attention kernel ...",
third-Q-tile paragraph: the Flash-Decoding style tail split of the keys)
combines normalised partial outputs O_s with their log-sum-exps LSE_s:
LSE = M + ln sum_s exp(LSE_s - M) with M = max_s LSE_s, and
O = sum_s exp(LSE_s - LSE) * O_s.  A partial over no key has LSE_s = -inf and
contributes nothing.
"""
from __future__ import annotations

import numpy as np


def online_attention_row(q, k, v, scale, edges):
    """One query row q [d] against k, v [Sk, d], processing keys in blocks
    [edges[t], edges[t+1]).  Returns (o [d], lse)."""
    d = v.shape[1]
    m = -np.inf
    l = 0.0
    acc = np.zeros(d)
    for a, b in zip(edges[:-1], edges[1:]):
        if b <= a:
            continue
        s = scale * (k[a:b] @ q)
        m_new = max(m, float(s.max()))
        if m_new == -np.inf:
            continue
        alpha = 0.0 if m == -np.inf else np.exp(m - m_new)
        p = np.exp(s - m_new)
        l = l * alpha + p.sum()          # l_new summed against the updated max
        acc = acc * alpha + p @ v[a:b]   # same per-row factor on the output
        m = m_new
    if l == 0.0:
        return np.zeros(d), -np.inf
    return acc / l, m + np.log(l)


def merge_partials(parts):
    """Merge [(o_s [d], lse_s), ...] of disjoint key sets into (o, lse)."""
    lses = np.array([p[1] for p in parts], dtype=np.float64)
    M = lses.max()
    d = parts[0][0].shape[0]
    if M == -np.inf:
        return np.zeros(d), -np.inf
    w = np.exp(lses - M)
    L = w.sum()
    lse = M + np.log(L)
    o = np.zeros(d)
    for (o_s, lse_s), w_s in zip(parts, w):
        if lse_s != -np.inf:
            o = o + (w_s / L) * o_s
    return o, lse
