"""One dominant logit selects its V row, on every forward kernel and on the
paged decode (GPU).

Closed form (the softmax definition of "FlashAttention: Fast and
Memory-Efficient Exact Attention with IO-Awareness", Section 2.2): if the
score of key j exceeds every other score of its row by at least 40, the row's
weights are 1 for j and below exp(-40) for each other key, so O_i = V_j to
within exp(-40) * Sk * max|V| and LSE_i = s_ij to within exp(-40) * Sk.
Here the gap is about 60 and every V value is a bf16 that fp16 also holds
(or, for the bf16 path, a value beyond fp16's range), so those bounds are far
below half a bf16 spacing of any V value: O must equal V_j bit for bit.

Construction: per (batch, K/V head) a vector u of +-1 entries; every query
row of the heads that share that K/V head is bf16(u + 0.05 * noise); key j
is alpha * u with scale * alpha * d = 60, the other keys bf16(0.01 * noise),
so their scores are about 0.01 and key j's about 60.  Key j sits in the
middle of the sequence: the rows see tiles of small scores first, and the
running maximum then jumps by about 60, which takes the kernels' full
rescale of the accumulated output (the lazy rescale's slow path).  Only rows
that see key j are checked (causal rows before it are ordinary rows, which
the parity tests cover).  The expected LSE is s_ij computed in float64 from
the same bf16 inputs."""

import math

import numpy as np
import pytest
import torch

import attn_inputs as gen
import exact_attention_60_amd as ea
from gpu_util import bits_of, dev_bf16, dev_i32, need_gpu

pytestmark = pytest.mark.gpu

GAP = 60.0
# LSE is s_ij plus terms below 1e-20; what remains is the float32 rounding of
# a score near 60 and of the log-sum-exp arithmetic (a few ulps of 64)
LSE_TOL = 5e-5


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _bf16_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _values(rng, shape, big: bool) -> np.ndarray:
    """bf16 bits of +-(1 + m/128) * 2^e, e in [-2, 2] (fp16 holds them
    exactly) or, with big, e in [17, 19] (beyond fp16's range, so that the
    kernels take their bf16 path)."""
    m = rng.integers(0, 128, size=shape).astype(np.uint32)
    e = rng.integers(17, 20, size=shape) if big else rng.integers(-2, 3, size=shape)
    s = rng.integers(0, 2, size=shape).astype(np.uint32)
    return ((s << 15) | ((127 + e).astype(np.uint32) << 7) | m).astype(np.uint16)


def _alpha_bits(d: int, scale: float) -> np.uint16:
    return gen.f32_to_bf16_bits(np.float32([GAP / (scale * d)]))[0]


def dominant_prefill(B, Hq, Hkv, Sq, Sk, d, *, layout, causal, seed, big=False):
    """A prefill problem (logical [B, S, H, d] built, then laid out) whose
    rows of K/V head g see key js[b, g] about GAP above every other key."""
    rng = np.random.default_rng([seed, 60])
    g = Hq // Hkv
    scale = 1.0 / math.sqrt(d)
    u = np.where(rng.integers(0, 2, size=(B, Hkv, d)) == 1, 1.0, -1.0).astype(np.float32)
    qf = np.repeat(u, g, axis=1)[:, None, :, :] + 0.05 * rng.standard_normal(
        (B, Sq, Hq, d), dtype=np.float32)
    q = gen.f32_to_bf16_bits(qf)
    k = gen.f32_to_bf16_bits(0.01 * rng.standard_normal((B, Sk, Hkv, d), dtype=np.float32))
    v = _values(rng, (B, Sk, Hkv, d), big)
    # mid-sequence, away from tile edges, different per (b, g)
    js = rng.integers(Sk // 3, max(Sk // 3 + 1, (2 * Sk) // 3), size=(B, Hkv))
    a = _alpha_bits(d, scale)
    ubits = np.where(u > 0, a, a | 0x8000).astype(np.uint16)
    for b in range(B):
        for h in range(Hkv):
            k[b, js[b, h], h] = ubits[b, h]
    if layout == gen.BHSD:
        q, k, v = (np.ascontiguousarray(x.transpose(0, 2, 1, 3)) for x in (q, k, v))
    p = gen.Prefill(q, k, v, B, Hq, Hkv, Sq, Sk, layout, bool(causal), scale)
    return p, js


def _logical(x: np.ndarray, layout: int) -> np.ndarray:
    """[B, S, H, d] view of an array in `layout`."""
    return x if layout == gen.BSHD else x.transpose(0, 2, 1, 3)


def check_prefill(p, js, o, lse):
    q = _logical(p.q, p.layout)
    k = _logical(p.k, p.layout)
    v = _logical(p.v, p.layout)
    ob = bits_of(o)
    ob = ob if p.layout == gen.BSHD else ob.transpose(0, 2, 1, 3)
    lse = lse.cpu().numpy().astype(np.float64)          # [B, Hq, Sq]
    g = p.Hq // p.Hkv
    checked = 0
    for b in range(p.B):
        for h in range(p.Hq):
            j = int(js[b, h // g])
            nvis = np.arange(p.Sq) + (p.Sk - p.Sq) + 1 if p.causal else np.full(p.Sq, p.Sk)
            rows = np.nonzero(nvis > j)[0]
            if rows.size == 0:
                continue
            want = v[b, j, h // g]
            got = ob[b, rows, h]
            bad = np.nonzero((got != want[None, :]).any(axis=1))[0]
            assert bad.size == 0, (f"b{b} h{h} key {j}: row {rows[bad[0]]} of O is not V[{j}] "
                                   f"({bad.size} rows differ)")
            s = p.scale * (_bf16_f64(q[b, rows, h]) @ _bf16_f64(k[b, j, h // g]))
            assert s.min() > GAP - 5
            err = np.abs(lse[b, h, rows] - s).max()
            assert err <= LSE_TOL, f"b{b} h{h}: LSE off s_ij by {err}"
            checked += rows.size
    assert checked > 0


# B, Hq, Hkv, Sq, Sk, d, layout, causal.  Head dim 128 with Hq == Hkv runs the
# MHA kernel (64-key tiles), groups of four the GQA kernel (32-key tiles);
# d = 64 and d = 256 have kernels of their own.
SHAPES = [
    (2, 4, 4, 300, 700, 128, gen.BSHD, False),
    (1, 4, 4, 513, 513, 128, gen.BHSD, True),
    (2, 8, 2, 257, 900, 128, gen.BSHD, False),
    (1, 8, 2, 600, 600, 128, gen.BHSD, True),
    (2, 4, 2, 300, 700, 64, gen.BSHD, False),
    (1, 8, 2, 513, 513, 64, gen.BHSD, True),
    (2, 4, 2, 200, 400, 256, gen.BSHD, False),
    (1, 4, 4, 300, 300, 256, gen.BHSD, True),
]


def _sid(s):
    return "B%d_Hq%d_Hkv%d_Sq%d_Sk%d_d%d_%s_%s" % (
        s[0], s[1], s[2], s[3], s[4], s[5], "bshd" if s[6] == gen.BSHD else "bhsd",
        "causal" if s[7] else "full")


@pytest.mark.parametrize("big", [False, True], ids=["fp16_v", "bf16_v"])
@pytest.mark.parametrize("prep", [False, True], ids=["single", "prepared"])
@pytest.mark.parametrize("shape", SHAPES, ids=_sid)
def test_dominant_logit_prefill(shape, prep, big):
    B, Hq, Hkv, Sq, Sk, d, layout, causal = shape
    p, js = dominant_prefill(B, Hq, Hkv, Sq, Sk, d, layout=layout, causal=causal,
                             seed=Sq + 7 * Sk + d, big=big)
    print(f"case: {_sid(shape)} prepared={prep} big_v={big}", flush=True)
    lay = "bshd" if layout == gen.BSHD else "bhsd"
    o, lse = ea.attn_fwd(dev_bf16(p.q), dev_bf16(p.k), dev_bf16(p.v), causal=causal,
                         scale=p.scale, layout=lay, prepare_v=prep)
    torch.cuda.synchronize()
    check_prefill(p, js, o, lse)


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_dominant_logit_varlen(causal):
    """The packed-sequence forward: each sequence's own dominant key."""
    lens_q = [1, 130, 77, 300]
    lens_k = [5, 200, 77, 450]
    Hq, Hkv, d = 8, 2, 128
    parts = []
    for n, (sq, sk) in enumerate(zip(lens_q, lens_k)):
        parts.append(dominant_prefill(1, Hq, Hkv, sq, sk, d, layout=gen.BSHD, causal=causal,
                                      seed=900 + n))
    q = np.concatenate([p.q[0] for p, _ in parts])
    k = np.concatenate([p.k[0] for p, _ in parts])
    v = np.concatenate([p.v[0] for p, _ in parts])
    cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int32)
    print(f"case: varlen causal={causal} lens_q={lens_q} lens_k={lens_k}", flush=True)
    o, lse = ea.attn_fwd_varlen(dev_bf16(q), dev_bf16(k), dev_bf16(v), dev_i32(cu_q),
                                dev_i32(cu_k), max(lens_q), causal=causal, scale=parts[0][0].scale)
    torch.cuda.synchronize()
    for n, (p, js) in enumerate(parts):
        r0, r1 = int(cu_q[n]), int(cu_q[n + 1])
        check_prefill(p, js, o[None, r0:r1], lse[None, :, r0:r1])


def dominant_decode(lens, Hq, Hkv, *, seed, big=False):
    """A paged decode problem (random page table, NaN past each end) whose
    query of K/V head g in sequence b sees token ts[b, g] about GAP above
    every other token."""
    lens = np.asarray(lens, dtype=np.int32)
    B = lens.shape[0]
    max_len = int(-(-int(lens.max()) // gen.PAGE) * gen.PAGE)
    p = gen.decode_inputs(B, Hq, Hkv, max_len=max_len, seed=seed, lens=lens)
    d = gen.D
    rng = np.random.default_rng([seed, 61])
    g = Hq // Hkv
    u = np.where(rng.integers(0, 2, size=(B, Hkv, d)) == 1, 1.0, -1.0).astype(np.float32)
    p.q = gen.f32_to_bf16_bits(np.repeat(u, g, axis=1) + 0.05 * rng.standard_normal(
        (B, Hq, d), dtype=np.float32))
    small = gen.f32_to_bf16_bits(0.01 * rng.standard_normal(p.k_pool.shape, dtype=np.float32))
    vals = _values(rng, p.v_pool.shape, big)
    a = _alpha_bits(d, p.scale)
    ts = np.zeros((B, Hkv), np.int64)
    for b in range(B):
        n = int(lens[b])
        for t in range(n):
            pg = p.block_table[b, t // gen.PAGE]
            p.k_pool[pg, t % gen.PAGE] = small[pg, t % gen.PAGE]
            p.v_pool[pg, t % gen.PAGE] = vals[pg, t % gen.PAGE]
        for h in range(Hkv):
            t = int(rng.integers(n // 3, max(n // 3 + 1, (2 * n) // 3)))
            ts[b, h] = t
            pg = p.block_table[b, t // gen.PAGE]
            p.k_pool[pg, t % gen.PAGE, h] = np.where(u[b, h] > 0, a, a | 0x8000)
    return p, ts


@pytest.mark.parametrize("big", [False, True], ids=["fp16_v", "bf16_v"])
@pytest.mark.parametrize("heads", [(8, 8), (32, 8), (16, 1)], ids=["mha", "gqa4", "mqa"])
def test_dominant_logit_decode(heads, big):
    Hq, Hkv = heads
    lens = [1, 17, 300, 1000, 2500, 4096]
    p, ts = dominant_decode(lens, Hq, Hkv, seed=Hq + Hkv + 31 * big, big=big)
    print(f"case: decode Hq{Hq} Hkv{Hkv} big_v={big} lens={lens}", flush=True)
    o, lse = ea.attn_decode_paged(dev_bf16(p.q), dev_bf16(p.k_pool), dev_bf16(p.v_pool),
                                  dev_i32(p.block_table), dev_i32(p.seq_lens), scale=p.scale)
    torch.cuda.synchronize()
    ob = bits_of(o)
    lse = lse.cpu().numpy().astype(np.float64)
    g = Hq // Hkv
    for b in range(p.B):
        for h in range(Hq):
            t = int(ts[b, h // g])
            pg = p.block_table[b, t // gen.PAGE]
            want = p.v_pool[pg, t % gen.PAGE, h // g]
            assert np.array_equal(ob[b, h], want), f"b{b} h{h}: O is not V of token {t}"
            s = p.scale * (_bf16_f64(p.q[b, h]) @ _bf16_f64(p.k_pool[pg, t % gen.PAGE, h // g]))
            assert s > GAP - 5
            assert abs(lse[b, h] - s) <= LSE_TOL, f"b{b} h{h}: LSE off s_ij by {lse[b, h] - s}"
