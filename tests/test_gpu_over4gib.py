"""Tensors larger than 4 GiB (GPU): every kernel's base addresses past the
32-bit range.

The kernels address one (batch, head) sequence with 32-bit buffer offsets
from a 64-bit base; these problems put K and V (and the prepared V^T tiles,
the paged pools, dK and dV) beyond 4 GiB, so a base computed in 32 bits
anywhere would read or write the wrong rows of the last batches or pages.
Inputs are N(0, 1) bf16 drawn on the device by torch's seeded generator (the
host would take minutes to draw 10 GiB); the oracle gets the batches and
pages it checks copied back before any kernel runs, and every element of
those is compared under the usual tolerance."""

import numpy as np
import pytest
import torch

import attn_inputs as gen
import exact_attention_60_amd as ea
import oracle.attention as att
import oracle.backward as bwd
from gpu_util import bits_of, dev_i32, host_f64, need_gpu
from tolerance import check_lse, check_o, ulp_bf16

pytestmark = pytest.mark.gpu

GIB = 1 << 30


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def randn(shape, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device="cuda", dtype=torch.bfloat16)


def _shape(layout, B, H, S, d):
    return (B, S, H, d) if layout == gen.BSHD else (B, H, S, d)


def _sub(p_q, p_k, p_v, b, Hq, Hkv, Sq, Sk, layout, causal, scale):
    """Host copy of batch b as a one-batch problem."""
    return gen.Prefill(bits_of(p_q[b:b + 1]), bits_of(p_k[b:b + 1]), bits_of(p_v[b:b + 1]),
                       1, Hq, Hkv, Sq, Sk, layout, causal, scale)


# B, Hq, Hkv, Sq, Sk, d, layout, causal: K and V 5 GiB each.  MHA and a group
# of 4 at d = 128 (the two d = 128 kernels), d = 64 and d = 256.
SHAPES = [
    (40, 32, 32, 77, 16384, 128, gen.BSHD, False),
    (160, 32, 8, 65, 16384, 128, gen.BHSD, True),
    (160, 16, 8, 50, 32768, 64, gen.BSHD, True),
    (80, 8, 4, 40, 32768, 256, gen.BHSD, False),
]


def _sid(s):
    return "B%d_Hq%d_Hkv%d_Sq%d_Sk%d_d%d_%s_%s" % (
        s[0], s[1], s[2], s[3], s[4], s[5], "bshd" if s[6] == gen.BSHD else "bhsd",
        "causal" if s[7] else "full")


@pytest.mark.parametrize("prep", [False, True], ids=["single", "prepared"])
@pytest.mark.parametrize("shape", SHAPES, ids=_sid)
def test_prefill_beyond_4gib(shape, prep):
    B, Hq, Hkv, Sq, Sk, d, layout, causal = shape
    kv_bytes = B * Hkv * Sk * d * 2
    assert kv_bytes > 4 * GIB
    print(f"case: {_sid(shape)} prepared={prep}", flush=True)
    seed = 1000 + d + Hq
    q = randn(_shape(layout, B, Hq, Sq, d), seed)
    k = randn(_shape(layout, B, Hkv, Sk, d), seed + 1)
    v = randn(_shape(layout, B, Hkv, Sk, d), seed + 2)
    scale = 1.0 / d ** 0.5
    subs = {b: _sub(q, k, v, b, Hq, Hkv, Sq, Sk, layout, causal, scale) for b in (B - 1, B // 2)}
    lay = "bshd" if layout == gen.BSHD else "bhsd"
    if prep:
        assert ea.attn_prep_v_bytes(B, Hq, Hkv, Sk, d) > 4 * GIB
    o, lse = ea.attn_fwd(q, k, v, causal=causal, scale=scale, layout=lay, prepare_v=prep)
    torch.cuda.synchronize()
    del k, v
    for b, p in subs.items():
        o_ref, l_ref = att.attention(p.q, p.k, p.v, 1, Hq, Hkv, Sq, Sk, scale, causal, layout)
        og = host_f64(o[b:b + 1])
        og = og.transpose(0, 2, 1, 3) if layout == gen.BSHD else og
        _, r_o = check_o(og, o_ref, f"batch {b}")
        e_l = check_lse(host_f64(lse[b:b + 1]), l_ref, f"batch {b}")
        print(f"  batch {b}: max O err/tol {r_o:.3f}, max LSE err {e_l:.2e}", flush=True)


def _pool_problem(B, Hq, Hkv, n_pages, lens, seed):
    """Device pools of n_pages 16-token pages; each sequence's pages drawn
    without repeats from the pages past the first 4 GiB of a pool."""
    page_bytes = gen.PAGE * Hkv * gen.D * 2
    first_high = -(-4 * GIB // page_bytes)
    assert n_pages * page_bytes > 4 * GIB and first_high < n_pages
    lens = np.asarray(lens, np.int32)
    nb = (lens + gen.PAGE - 1) // gen.PAGE
    rng = np.random.default_rng([seed, 4])
    ids = rng.choice(np.arange(first_high, n_pages), size=int(nb.sum()), replace=False)
    max_blocks = int(nb.max())
    table = np.full((B, max_blocks), -1, np.int32)
    off = 0
    for b in range(B):
        table[b, :nb[b]] = ids[off:off + nb[b]]
        off += int(nb[b])
    kc = randn((n_pages, gen.PAGE, Hkv, gen.D), seed + 1)
    vc = randn((n_pages, gen.PAGE, Hkv, gen.D), seed + 2)
    q = randn((B, Hq, gen.D), seed + 3)
    return q, kc, vc, table, lens, ids


def _compact(kc, vc, table, ids):
    """Host copies of the pages in use and the table renumbered onto them."""
    ids_t = torch.from_numpy(ids.astype(np.int64)).cuda()
    kp = bits_of(kc.index_select(0, ids_t))
    vp = bits_of(vc.index_select(0, ids_t))
    where = {int(x): n for n, x in enumerate(ids)}
    small = np.where(table >= 0, np.vectorize(lambda x: where.get(int(x), -1))(table), -1)
    return kp, vp, small.astype(np.int32)


@pytest.mark.parametrize("heads", [(32, 8), (8, 1)], ids=["gqa4", "mqa"])
def test_decode_pool_beyond_4gib(heads):
    Hq, Hkv = heads
    B = 6
    lens = [1, 17, 700, 2500, 4096, 3001]
    n_pages = (5 * GIB) // (gen.PAGE * Hkv * gen.D * 2)
    print(f"case: decode Hq{Hq} Hkv{Hkv} pages {n_pages} lens {lens}", flush=True)
    q, kc, vc, table, lens, ids = _pool_problem(B, Hq, Hkv, n_pages, lens, 2000 + Hq)
    kp, vp, small = _compact(kc, vc, table, ids)
    qb = bits_of(q)
    o, lse = ea.attn_decode_paged(q, kc, vc, dev_i32(table), dev_i32(lens), scale=gen.D ** -0.5)
    torch.cuda.synchronize()
    o_ref, l_ref = att.decode_paged(qb, kp, vp, small, lens, Hkv, gen.D ** -0.5)
    _, r_o = check_o(host_f64(o), o_ref, "decode")
    e_l = check_lse(host_f64(lse), l_ref, "decode")
    print(f"  max O err/tol {r_o:.3f}, max LSE err {e_l:.2e}", flush=True)


def test_decode_append_pool_beyond_4gib():
    Hq, Hkv, B = 32, 8, 5
    lens = [1, 16, 17, 1000, 4096]
    n_pages = (5 * GIB) // (gen.PAGE * Hkv * gen.D * 2)
    print(f"case: decode+append Hq{Hq} Hkv{Hkv} pages {n_pages} lens {lens}", flush=True)
    q, kc, vc, table, lens, ids = _pool_problem(B, Hq, Hkv, n_pages, lens, 3000)
    k_new = randn((B, Hkv, gen.D), 3100)
    v_new = randn((B, Hkv, gen.D), 3101)
    kp, vp, small = _compact(kc, vc, table, ids)
    qb, knb, vnb = bits_of(q), bits_of(k_new), bits_of(v_new)
    o, lse = ea.attn_decode_paged_append(q, k_new, v_new, kc, vc, dev_i32(table), dev_i32(lens),
                                         scale=gen.D ** -0.5)
    torch.cuda.synchronize()
    o_ref, l_ref, kp2, vp2 = att.decode_paged_append(qb, knb, vnb, kp, vp, small, lens, Hkv,
                                                     gen.D ** -0.5)
    check_o(host_f64(o), o_ref, "decode+append")
    check_lse(host_f64(lse), l_ref, "decode+append")
    kp_after, vp_after, _ = _compact(kc, vc, table, ids)
    assert np.array_equal(kp_after, kp2), "K pool pages after the append"
    assert np.array_equal(vp_after, vp2), "V pool pages after the append"


def test_backward_beyond_4gib():
    """MHA backward with K, V, dK and dV of 5 GiB each; two heads of the last
    and a middle batch checked against the float64 gradient."""
    B, H, Sq, Sk, d = 40, 32, 77, 16384, 128
    print(f"case: backward B{B} H{H} Sq{Sq} Sk{Sk} bshd", flush=True)
    q = randn((B, Sq, H, d), 4000)
    k = randn((B, Sk, H, d), 4001)
    v = randn((B, Sk, H, d), 4002)
    do = randn((B, Sq, H, d), 4003)
    picks = [(B - 1, H - 1), (B // 2, 0)]
    host = {}
    for b, h in picks:
        host[(b, h)] = tuple(bits_of(t[b:b + 1, :, h:h + 1]) for t in (q, k, v, do))
    scale = d ** -0.5
    o, lse = ea.attn_fwd(q, k, v, scale=scale, layout="bshd")
    dq, dk, dv = ea.attn_bwd(q, k, v, o, lse, do, scale=scale, layout="bshd")
    torch.cuda.synchronize()
    assert dk.numel() * 2 > 4 * GIB
    for (b, h), (qb, kb, vb, dob) in host.items():
        ref = bwd.attention_backward(qb, kb, vb, dob, 1, 1, 1, Sq, Sk, scale, False, gen.BSHD,
                                     magnitudes=True)
        for i, (n, t) in enumerate((("dq", dq), ("dk", dk), ("dv", dv))):
            got = host_f64(t[b:b + 1, :, h:h + 1]).transpose(0, 2, 1, 3)
            err = np.abs(got - ref[i])
            tol = ulp_bf16(ref[i]) + 2.0 ** -7 * ref[i + 3]
            r = float((err / tol).max())
            assert np.all(np.isfinite(got)) and r <= 1.0, f"b{b} h{h} {n}: err/tol {r:.3f}"
            print(f"  b{b} h{h} {n}: max err/tol {r:.3f}", flush=True)
