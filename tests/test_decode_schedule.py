"""The decode work schedule, checked on the CPU.

decode_partial_kernel cuts the page slots (unit group x, concatenated pages of
all sequences) into equal chunks of at most 64 and at least 4 pages and walks
each chunk in segments that end at sequence boundaries; the merge kernel then
finds a (sequence, unit group)'s partial results in slots 0 .. count-1.  This
test restates that arithmetic (the same integer formulas as the kernel) and
checks what the kernel relies on for memory safety and correctness: every
(unit group, sequence, page) is visited exactly once, a segment never exceeds
the 64 table entries a wave holds, every slot index stays below the
workspace's partial count, and each (sequence, unit group) gets exactly the
slots 0 .. count-1.
"""
import numpy as np
import pytest

import exact_attention_60_amd as ea

MAX_CHUNK, MIN_CHUNK = 64, 4


def chunks(T, X, nwg):
    W = X * T
    if W == 0:
        return W, 0, 0, 0
    rounds = (W + MAX_CHUNK * nwg - 1) // (MAX_CHUNK * nwg)
    NC = max(min(nwg * rounds, W // MIN_CHUNK), 1)
    q = W // NC
    return W, NC, q, W - q * NC


def begin(c, q, rem):
    return c * q + min(c, rem)


def chunk_of(L, q, rem):
    big = rem * (q + 1)
    return L // (q + 1) if L < big else rem + (L - big) // q


def walk(lens, max_blocks, X, nwg):
    npg = [(min(max(int(l), 0), max_blocks * 16) + 15) // 16 for l in lens]
    pre = np.concatenate([[0], np.cumsum(npg)]).astype(np.int64)
    T = int(pre[-1])
    W, NC, q, rem = chunks(T, X, nwg)
    seen, cnt = {}, {}
    for j in range(nwg):
        for c in range(j, NC, nwg):
            L, Lend = begin(c, q, rem), begin(c + 1, q, rem)
            assert 0 < Lend - L <= MAX_CHUNK
            while L < Lend:
                x, r = divmod(L, T)
                b = int(np.searchsorted(pre, r, side="right") - 1)   # last b with pre[b] <= r
                assert pre[b] <= r < pre[b + 1]
                seg_end = min(Lend, x * T + pre[b] + npg[b])
                p0 = r - pre[b]
                p1 = p0 + (seg_end - L)
                assert 0 <= p0 < p1 <= npg[b] and p1 - p0 <= MAX_CHUNK
                first = chunk_of(x * T + pre[b], q, rem)
                if p0 == 0:
                    cnt[(b, x)] = chunk_of(x * T + pre[b] + npg[b] - 1, q, rem) - first + 1
                for p in range(p0, p1):
                    assert (x, b, p) not in seen
                    seen[(x, b, p)] = c - first
                L = seg_end
    return npg, seen, cnt


@pytest.mark.parametrize("B,max_blocks,X,nwg", [
    (1, 1, 1, 256), (1, 2500, 1, 256), (32, 256, 1, 256), (32, 256, 2, 768), (5, 20, 3, 7),
    (65, 40, 1, 256), (130, 12, 2, 256), (700, 3, 1, 256), (3, 1000, 16, 1)])
def test_every_page_once_and_slots_in_range(B, max_blocks, X, nwg):
    rng = np.random.default_rng(B * 7 + max_blocks)
    lens = rng.integers(-3, max_blocks * 16 + 40, size=B)   # includes out-of-contract values
    npg, seen, cnt = walk(lens, max_blocks, X, nwg)
    S = (max_blocks + 3) // 4 + 1                            # partial results per (b, head)
    assert len(seen) == X * sum(npg)
    for x in range(X):
        for b in range(B):
            if npg[b] == 0:
                continue
            slots = sorted({seen[(x, b, p)] for p in range(npg[b])})
            assert slots == list(range(cnt[(b, x)]))
            assert cnt[(b, x)] <= S


def test_workspace_holds_the_partials_the_schedule_can_need():
    for B, Hq, mb in [(1, 1, 1), (32, 32, 256), (3, 8, 1000)]:
        S = (mb + 3) // 4 + 1
        assert ea.attn_decode_workspace_bytes(B, Hq, mb) == B * Hq * (S * 129 + 1) * 4
