"""Parity of the ALiBi forward (attn_fwd_alibi) with the fp64 oracle (GPU),
under the forward's tolerance."""
import numpy as np
import pytest
import torch

import attn_inputs as gen
import exact_attention_60_amd as ea
import oracle.attention as att
from gpu_util import dev_bf16, host_f64, logical_o, need_gpu
from tolerance import (P_UNIT_BF16, check_lse, check_lse_bf16_fallback, check_o,
                       check_o_large_v, pv_spread_prefill)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def slopes(H):
    """The geometric slopes of the ALiBi paper for H heads (2^(-8h/H))."""
    return (2.0 ** (-8.0 * np.arange(1, H + 1) / H)).astype(np.float32)


def lay(p):
    return "bshd" if p.layout == gen.BSHD else "bhsd"


def run(p, sl, rounding="rtne"):
    o, lse = ea.attn_fwd(dev_bf16(p.q), dev_bf16(p.k), dev_bf16(p.v), causal=p.causal,
                         scale=p.scale, layout=lay(p), rounding=rounding,
                         alibi_slopes=torch.from_numpy(sl).cuda())
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("B,Hq,Hkv,Sq,Sk,layout,causal", [
    (1, 4, 4, 256, 256, gen.BSHD, False),
    (2, 8, 2, 200, 200, gen.BSHD, True),       # GQA causal, ragged tiles
    (1, 4, 2, 300, 77, gen.BHSD, False),       # cross attention, keys before and after i + off
    (1, 4, 2, 150, 100, gen.BSHD, True),       # rows that see no key
    (1, 4, 1, 70, 600, gen.BHSD, True),        # bottom-right alignment
    (1, 8, 2, 700, 650, gen.BSHD, False),      # pivots inside the keys, ragged tail
    (1, 4, 4, 90, 1000, gen.BHSD, False),      # few rows, pivot near the last key
])
def test_alibi_all_elements(B, Hq, Hkv, Sq, Sk, layout, causal):
    p = gen.prefill_inputs(B, Hq, Hkv, Sq, Sk, layout=layout, causal=causal, seed=Sq + 2 * Sk,
                           n_hot=2)
    sl = slopes(Hq)
    o, lse = run(p, sl)
    o_ref, l_ref = att.attention(p.q, p.k, p.v, B, Hq, Hkv, Sq, Sk, p.scale, causal, p.layout,
                                 alibi_slopes=sl)
    e = check_o(logical_o(o, p.layout), o_ref, "alibi")
    el = check_lse(host_f64(lse), l_ref, "alibi lse")
    print(f"alibi B{B} Hq{Hq} Sq{Sq} Sk{Sk} causal{causal}: err/tol {e[1]:.3f} lse {el:.3g}",
          flush=True)


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_zero_slopes_match_plain_attention(causal):
    """The ALiBi variant takes a workgroup's key tiles from the one holding
    its diagonal down to key 0, then upward, so with zero slopes it is the
    plain attention up to the order of the sums: checked against the oracle
    without a bias, and within a few bf16 ulps of the plain kernel."""
    p = gen.prefill_inputs(1, 4, 2, 333, 333, layout=gen.BSHD, causal=causal, seed=3)
    o1, l1 = run(p, np.zeros(4, np.float32))
    o2, l2 = ea.attn_fwd(dev_bf16(p.q), dev_bf16(p.k), dev_bf16(p.v), causal=causal,
                         scale=p.scale, layout="bshd")
    torch.cuda.synchronize()
    o_ref, l_ref = att.attention(p.q, p.k, p.v, 1, 4, 2, 333, 333, p.scale, causal, p.layout)
    check_o(logical_o(o1, p.layout), o_ref, "zero slopes")
    check_lse(host_f64(l1), l_ref, "zero slopes lse")
    d = (o1.float() - o2.float()).abs()
    assert (d <= 4 * 2.0 ** -8 * o2.float().abs() + 1e-3).all()
    # l sums fp16-rounded probabilities taken against each order's running
    # max: up to 2^-11 relative in l, i.e. about 5e-4 in LSE, per kernel
    assert (l1 - l2).abs().max().item() <= 1e-3


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_alibi_v_beyond_fp16_range(causal):
    """V entries far beyond the fp16 range take the bf16 redo of the tile loop,
    which runs the key tiles in the same order from the diagonal outward;
    a constant V column still gives that constant."""
    p = gen.prefill_inputs(1, 4, 2, 300, 1500, layout=gen.BSHD, causal=causal, seed=84)
    v = (p.v.astype(np.uint32) << 16).view(np.float32).copy()
    v[:, :, :, 5] = 3.0e5
    v[0, 700, 1, 9] = -2.0e6
    p.v = gen.f32_to_bf16_bits(v)
    sl = slopes(4)
    o, lse = run(p, sl)
    o_ref, l_ref = att.attention(p.q, p.k, p.v, 1, 4, 2, 300, 1500, p.scale, causal, p.layout,
                                 alibi_slopes=sl)
    # every tile holds V beyond fp16, so the whole problem runs with bf16
    # probabilities: the large-V bound with the bf16 unit, probabilities of
    # the biased scores (ALiBi makes the rows peaky, where 8 bits of P exceed
    # the plain 2-ulp bound)
    spread = pv_spread_prefill(p, unit=P_UNIT_BF16, alibi_slopes=sl)
    check_o_large_v(logical_o(o, p.layout), o_ref, spread, "alibi huge V")
    check_lse_bf16_fallback(host_f64(lse), l_ref, "alibi huge V lse")
    # 3e5 rounds to the bf16 value 299008 (spacing 2048 there)
    assert np.all(host_f64(o)[..., 5] == 299008.0)


def test_alibi_causal_gqa_full_size_sampled_group():
    """The causal GQA workload (B=8, Hq=32, Hkv=8, S=8192) with ALiBi: every
    row of one K/V head's four query heads."""
    p = gen.config3()
    sl = slopes(32)
    o, lse = run(p, sl)
    b, g, G = 5, 6, 4
    sub = [np.ascontiguousarray(x[b:b + 1, :, h0:h1])
           for x, h0, h1 in ((p.q, g * G, g * G + G), (p.k, g, g + 1), (p.v, g, g + 1))]
    o_ref, l_ref = att.attention(*sub, 1, G, 1, p.Sq, p.Sk, p.scale, True, gen.BSHD,
                                 alibi_slopes=sl[g * G:g * G + G])
    e = check_o(logical_o(o[b:b + 1, :, g * G:g * G + G], gen.BSHD), o_ref, "alibi cfg3")
    check_lse(host_f64(lse[b:b + 1, g * G:g * G + G]), l_ref, "alibi cfg3 lse")
    print(f"alibi causal gqa b{b} g{g}: err/tol {e[1]:.3f}", flush=True)


@pytest.mark.parametrize("B,Hq,Hkv,Sq,Sk,layout,causal", [
    (2, 8, 2, 200, 200, gen.BSHD, True),
    (1, 4, 2, 300, 77, gen.BHSD, False),
    (1, 4, 1, 70, 600, gen.BHSD, True),
])
def test_alibi_backward_all_elements(B, Hq, Hkv, Sq, Sk, layout, causal):
    import oracle.backward as obwd
    from test_gpu_backward import check as check_grad, logical
    p = gen.prefill_inputs(B, Hq, Hkv, Sq, Sk, layout=layout, causal=causal, seed=Sq + 3 * Sk)
    do = gen.output_grad(p, 4)
    sl = slopes(Hq)
    slt = torch.from_numpy(sl).cuda()
    q, k, v = dev_bf16(p.q), dev_bf16(p.k), dev_bf16(p.v)
    o, lse = ea.attn_fwd(q, k, v, causal=causal, scale=p.scale, layout=lay(p), alibi_slopes=slt)
    g = ea.attn_bwd(q, k, v, o, lse, dev_bf16(do), causal=causal, scale=p.scale, layout=lay(p),
                    alibi_slopes=slt)
    torch.cuda.synchronize()
    ref = obwd.attention_backward(p.q, p.k, p.v, do, B, Hq, Hkv, Sq, Sk, p.scale, causal,
                                  p.layout, magnitudes=True, alibi_slopes=sl)
    r = [check_grad(f"alibi {n}", logical(t, p.layout), ref[i], ref[i + 3])
         for i, (n, t) in enumerate(zip(("dq", "dk", "dv"), g))]
    print(f"alibi backward Sq{Sq} Sk{Sk} causal{causal}: max err/tol {max(r):.3f}", flush=True)
