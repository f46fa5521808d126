"""Parity of the head-dim-64 and -256 forwards (attn_fwd with d = 64 or 256)
with the fp64 oracle (GPU), under the forward's tolerance."""
import numpy as np
import pytest
import torch

import attn_inputs as gen
import exact_attention_60_amd as ea
import oracle.attention as att
from gpu_util import dev_bf16, host_f64, logical_o, need_gpu
from tolerance import check_lse, check_o

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def lay(p):
    return "bshd" if p.layout == gen.BSHD else "bhsd"


def run(p, rounding="rtne"):
    o, lse = ea.attn_fwd(dev_bf16(p.q), dev_bf16(p.k), dev_bf16(p.v), causal=p.causal,
                         scale=p.scale, layout=lay(p), rounding=rounding)
    torch.cuda.synchronize()
    return o, lse


def check(p, o, lse, what):
    o_ref, l_ref = att.attention(p.q, p.k, p.v, p.B, p.Hq, p.Hkv, p.Sq, p.Sk, p.scale, p.causal,
                                 p.layout)
    e = check_o(logical_o(o, p.layout), o_ref, what)
    el = check_lse(host_f64(lse), l_ref, what)
    print(f"{what}: err/tol {e[1]:.3f} lse {el:.3g}", flush=True)
    return o_ref


@pytest.mark.parametrize("B,Hq,Hkv,Sq,Sk,layout,causal", [
    (1, 4, 4, 256, 256, gen.BSHD, False),
    (2, 8, 2, 200, 200, gen.BHSD, True),       # GQA causal, ragged blocks and tiles
    (1, 4, 2, 300, 77, gen.BSHD, False),       # cross attention, short keys
    (1, 4, 2, 150, 100, gen.BSHD, True),       # rows that see no key
    (1, 4, 1, 70, 600, gen.BHSD, True),        # MQA, bottom-right alignment
    (1, 2, 2, 1, 1, gen.BSHD, False),
    (1, 2, 1, 129, 1000, gen.BSHD, False),
])
def test_d64_all_elements(B, Hq, Hkv, Sq, Sk, layout, causal):
    p = gen.prefill_inputs(B, Hq, Hkv, Sq, Sk, layout=layout, causal=causal, seed=Sq + Sk,
                           n_hot=min(3, B * Sq * Hq), d=64)
    o, lse = run(p)
    check(p, o, lse, f"d64 B{B} Hq{Hq} Hkv{Hkv} Sq{Sq} Sk{Sk} causal{causal}")


def test_d64_rounding_rules_from_the_same_values():
    p = gen.prefill_inputs(1, 4, 2, 130, 130, layout=gen.BSHD, causal=True, seed=5, d=64)
    outs = {m: run(p, m)[0] for m in ("rtne", "rtna", "rtz")}
    o_ref = check(p, outs["rtne"], run(p)[1], "d64 rtne")
    for m in ("rtna", "rtz"):
        check_o(logical_o(outs[m], p.layout), o_ref, f"d64 {m}")
    # RTZ never exceeds RTNE in magnitude, and the two differ by at most one spacing
    a = host_f64(outs["rtz"])
    b = host_f64(outs["rtne"])
    assert np.all(np.abs(a) <= np.abs(b))


def test_d64_v_beyond_fp16_range_takes_the_bf16_path():
    p = gen.prefill_inputs(1, 2, 1, 64, 90, layout=gen.BSHD, seed=6, d=64)
    v = p.v.copy()
    v[0, 7, 0, 5] = gen.f32_to_bf16_bits(np.array([70000.0], np.float32))[0]
    p = gen.Prefill(p.q, p.k, v, 1, 2, 1, 64, 90, gen.BSHD, False, p.scale)
    o, lse = run(p)
    assert torch.isfinite(o.float()).all()
    check(p, o, lse, "d64 large V")


def test_d64_deterministic():
    p = gen.prefill_inputs(1, 8, 2, 333, 333, layout=gen.BSHD, causal=True, seed=9, d=64)
    a, la = run(p)
    b, lb = run(p)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16)) and torch.equal(la, lb)


def test_d64_causal_gqa_full_size_sampled_group():
    p = gen.headdim64_causal_gqa()
    o, lse = run(p)
    b, g, G = 3, 5, 4
    sub = [np.ascontiguousarray(x[b:b + 1, :, h0:h1])
           for x, h0, h1 in ((p.q, g * G, g * G + G), (p.k, g, g + 1), (p.v, g, g + 1))]
    o_ref, l_ref = att.attention(*sub, 1, G, 1, p.Sq, p.Sk, p.scale, True, gen.BSHD)
    e = check_o(logical_o(o[b:b + 1, :, g * G:g * G + G], gen.BSHD), o_ref, "d64 full size")
    check_lse(host_f64(lse[b:b + 1, g * G:g * G + G]), l_ref, "d64 full size lse")
    print(f"d64 causal gqa full size b{b} g{g}: err/tol {e[1]:.3f}", flush=True)


@pytest.mark.parametrize("B,Hq,Hkv,Sq,Sk,layout,causal", [
    (1, 4, 4, 256, 256, gen.BSHD, False),
    (2, 4, 2, 200, 200, gen.BHSD, True),
    (1, 4, 2, 300, 77, gen.BSHD, False),
    (1, 4, 2, 150, 100, gen.BSHD, True),
    (1, 2, 1, 33, 500, gen.BHSD, True),
])
def test_d256_all_elements(B, Hq, Hkv, Sq, Sk, layout, causal):
    p = gen.prefill_inputs(B, Hq, Hkv, Sq, Sk, layout=layout, causal=causal, seed=Sq + 2 * Sk,
                           n_hot=min(3, B * Sq * Hq), d=256)
    o, lse = run(p)
    check(p, o, lse, f"d256 B{B} Hq{Hq} Hkv{Hkv} Sq{Sq} Sk{Sk} causal{causal}")


def test_d256_v_beyond_fp16_range_takes_the_bf16_path():
    p = gen.prefill_inputs(1, 2, 1, 64, 90, layout=gen.BSHD, seed=16, d=256)
    v = p.v.copy()
    v[0, 11, 0, 200] = gen.f32_to_bf16_bits(np.array([-80000.0], np.float32))[0]
    p = gen.Prefill(p.q, p.k, v, 1, 2, 1, 64, 90, gen.BSHD, False, p.scale)
    o, lse = run(p)
    assert torch.isfinite(o.float()).all()
    check(p, o, lse, "d256 large V")


def test_d256_rounding_rules_and_determinism():
    p = gen.prefill_inputs(1, 4, 2, 200, 300, layout=gen.BHSD, causal=True, seed=15, d=256)
    outs = {m: run(p, m) for m in ("rtne", "rtna", "rtz")}
    o_ref = check(p, outs["rtne"][0], outs["rtne"][1], "d256 rtne")
    for m in ("rtna", "rtz"):
        check_o(logical_o(outs[m][0], p.layout), o_ref, f"d256 {m}")
    a = host_f64(outs["rtz"][0])
    b = host_f64(outs["rtne"][0])
    assert np.all(np.abs(a) <= np.abs(b))
    o2, l2 = run(p)
    assert torch.equal(o2.view(torch.int16), outs["rtne"][0].view(torch.int16))
    assert torch.equal(l2, outs["rtne"][1])


def test_d256_many_tiles_all_elements():
    # several 128-row query blocks and 32-key tiles, ragged on both sides,
    # non-causal and causal (the binding's default: single call at this size)
    for causal in (False, True):
        p = gen.prefill_inputs(1, 4, 1, 700, 1100, layout=gen.BSHD, causal=causal, seed=31,
                               n_hot=3, d=256)
        o, lse = run(p)
        check(p, o, lse, f"d256 Sq700 Sk1100 causal{causal}")


def test_d256_causal_gqa_full_size_sampled_group():
    # the timed head-dim-256 shape (B=4, Hq=32, Hkv=8, S=4096, causal; the
    # binding prepares V here), one K/V head's group against the oracle
    p = gen.prefill_inputs(4, 32, 8, 4096, 4096, layout=gen.BSHD, causal=True, seed=8, d=256)
    assert ea.prepares_v(p.B, p.Hq, p.Hkv, p.Sq, p.Sk, 256)
    o, lse = run(p)
    b, g, G = 2, 3, 4
    sub = [np.ascontiguousarray(x[b:b + 1, :, h0:h1])
           for x, h0, h1 in ((p.q, g * G, g * G + G), (p.k, g, g + 1), (p.v, g, g + 1))]
    o_ref, l_ref = att.attention(*sub, 1, G, 1, p.Sq, p.Sk, p.scale, True, gen.BSHD)
    e = check_o(logical_o(o[b:b + 1, :, g * G:g * G + G], gen.BSHD), o_ref, "d256 full size")
    check_lse(host_f64(lse[b:b + 1, g * G:g * G + G]), l_ref, "d256 full size lse")
    print(f"d256 causal gqa full size b{b} g{g}: err/tol {e[1]:.3f}", flush=True)
