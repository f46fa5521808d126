"""Parity of the HIP attention backward (dQ, dK, dV) with the fp64 gradient
oracle (GPU).

The forward on the GPU supplies O and LSE, as a training step would; the
oracle differentiates the exact definition.  Tolerance, derived from the
arithmetic of the kernels (products of bf16-rounded P and dS with fp32
accumulation, the row term from the bf16 O, outputs rounded to bf16):
    |g - g_ref| <= ulp_bf16(|g_ref|) + 2^-7 * m
elementwise, where m is the oracle's sum of absolute terms behind that entry
(``oracle.backward.grad_magnitudes``): rounding P or dS to bf16 moves each term
by at most 2^-9 of its size and a bf16 O moves the row term by at most about
2^-8 of the sum of |dO_c O_c|, together below 2^-7 of m; the last ulp covers
the final rounding.
"""
import numpy as np
import pytest
import torch

import attn_inputs as gen
import exact_attention_60_amd as ea
import oracle.backward as bwd
from gpu_util import dev_bf16, host_f64, need_gpu
from tolerance import ulp_bf16

pytestmark = pytest.mark.gpu

REL = 2.0 ** -7


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def lay(p):
    return "bshd" if p.layout == gen.BSHD else "bhsd"


def run(p, do_bits):
    q, k, v, do = dev_bf16(p.q), dev_bf16(p.k), dev_bf16(p.v), dev_bf16(do_bits)
    o, lse = ea.attn_fwd(q, k, v, causal=p.causal, scale=p.scale, layout=lay(p))
    dq, dk, dv = ea.attn_bwd(q, k, v, o, lse, do, causal=p.causal, scale=p.scale, layout=lay(p))
    torch.cuda.synchronize()
    return dq, dk, dv


def logical(t, layout):
    x = host_f64(t)
    return x.transpose(0, 2, 1, 3) if layout == gen.BSHD else x


def check(name, got, ref, mag):
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite gradient"
    err = np.abs(got - ref)
    tol = ulp_bf16(ref) + REL * mag
    ratio = err / tol
    w = np.unravel_index(np.argmax(ratio), ratio.shape)
    assert ratio.max() <= 1.0, (f"{name}: mismatch at {w}: got {got[w]!r} ref {ref[w]!r} "
                                f"err {err[w]:.3g} tol {tol[w]:.3g}")
    return float(ratio.max())


def check_problem(p, do, what):
    dq, dk, dv = run(p, do)
    ref = bwd.attention_backward(p.q, p.k, p.v, do, p.B, p.Hq, p.Hkv, p.Sq, p.Sk, p.scale,
                                 p.causal, p.layout, magnitudes=True)
    r = [check(f"{what} {n}", logical(t, p.layout), ref[i], ref[i + 3])
         for i, (n, t) in enumerate((("dq", dq), ("dk", dk), ("dv", dv)))]
    print(f"{what}: max err/tol dq {r[0]:.3f} dk {r[1]:.3f} dv {r[2]:.3f}", flush=True)
    return r


def test_tiny_mha_with_hot_rows_all_elements():
    p = gen.config1()
    check_problem(p, gen.output_grad(p, 1), "config1 shape")


@pytest.mark.parametrize("B,Hq,Hkv,Sq,Sk,layout,causal", [
    (2, 8, 2, 200, 200, gen.BSHD, True),      # GQA causal, ragged tails of every block size
    (1, 4, 1, 129, 129, gen.BHSD, False),     # MQA, one row past a block
    (2, 4, 4, 300, 77, gen.BHSD, False),      # cross attention, Sk < one key block
    (1, 4, 2, 150, 100, gen.BSHD, True),      # causal Sq > Sk: 50 rows see no key
    (1, 4, 2, 70, 300, gen.BSHD, True),       # causal Sq < Sk: bottom-right alignment
    (1, 2, 2, 1, 1, gen.BSHD, False),         # one row, one key
    (1, 2, 1, 64, 1, gen.BHSD, True),         # one key
    (1, 2, 2, 513, 640, gen.BSHD, False),     # several blocks both ways
])
def test_shapes_all_elements(B, Hq, Hkv, Sq, Sk, layout, causal):
    p = gen.prefill_inputs(B, Hq, Hkv, Sq, Sk, layout=layout, causal=causal,
                           seed=1000 + Sq + Sk, n_hot=2)
    check_problem(p, gen.output_grad(p, 7), f"B{B} Hq{Hq} Hkv{Hkv} Sq{Sq} Sk{Sk} causal{causal}")


def test_uniform_v_and_equal_keys():
    p = gen.prefill_inputs(1, 4, 2, 96, 160, layout=gen.BSHD, causal=True, seed=3,
                           v_dist="uniform")
    check_problem(p, gen.output_grad(p, 3), "uniform V")
    p = gen.equal_keys_prefill(1, 4, 2, 64, 130, layout=gen.BHSD, seed=4)
    dq, _, _ = run(p, gen.output_grad(p, 4))
    # identical keys: every row's probabilities are uniform whatever Q is, so
    # dQ vanishes up to the rounding of dS
    ref = bwd.attention_backward(p.q, p.k, p.v, gen.output_grad(p, 4), p.B, p.Hq, p.Hkv, p.Sq,
                                 p.Sk, p.scale, False, p.layout, magnitudes=True)
    check("equal keys dq", logical(dq, p.layout), ref[0], ref[3])


def test_deterministic():
    p = gen.prefill_inputs(1, 8, 2, 333, 333, layout=gen.BSHD, causal=True, seed=9)
    do = gen.output_grad(p, 9)
    a = run(p, do)
    b = run(p, do)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def _head_slice(bits, layout, b, h0, h1):
    if layout == gen.BSHD:
        return np.ascontiguousarray(bits[b:b + 1, :, h0:h1])
    return np.ascontiguousarray(bits[b:b + 1, h0:h1])


def _check_full_size(p, do, picks, what):
    """Full-size problem on the GPU; the oracle recomputes whole K/V heads
    (with every query head of their group) for the (batch, K/V head) pairs in
    picks and compares every element of those heads."""
    dq, dk, dv = run(p, do)
    G = p.Hq // p.Hkv
    for b, g in picks:
        sub = gen.Prefill(_head_slice(p.q, p.layout, b, g * G, (g + 1) * G),
                          _head_slice(p.k, p.layout, b, g, g + 1),
                          _head_slice(p.v, p.layout, b, g, g + 1),
                          1, G, 1, p.Sq, p.Sk, p.layout, p.causal, p.scale)
        dsub = _head_slice(do, p.layout, b, g * G, (g + 1) * G)
        ref = bwd.attention_backward(sub.q, sub.k, sub.v, dsub, 1, G, 1, p.Sq, p.Sk, p.scale,
                                     p.causal, p.layout, magnitudes=True)
        if p.layout == gen.BSHD:
            gq = dq[b:b + 1, :, g * G:(g + 1) * G]
            gk, gv = dk[b:b + 1, :, g:g + 1], dv[b:b + 1, :, g:g + 1]
        else:
            gq = dq[b:b + 1, g * G:(g + 1) * G]
            gk, gv = dk[b:b + 1, g:g + 1], dv[b:b + 1, g:g + 1]
        r = [check(f"{what} b{b} g{g} {n}", logical(t, p.layout), ref[i], ref[i + 3])
             for i, (n, t) in enumerate((("dq", gq), ("dk", gk), ("dv", gv)))]
        print(f"{what} b{b} g{g}: max err/tol {max(r):.3f}", flush=True)


def test_mha_prefill_full_size_sampled_heads():
    p = gen.config2()
    _check_full_size(p, gen.output_grad(p, 2), [(0, 0), (3, 31)], "mha b4 h32 s4096")


def test_causal_gqa_full_size_sampled_group():
    p = gen.config3()
    _check_full_size(p, gen.output_grad(p, 3), [(7, 7)], "gqa causal b8 s8192")


@pytest.mark.parametrize("B,Hq,Hkv,Sq,Sk,layout,causal", [
    (1, 4, 4, 256, 256, gen.BSHD, False),
    (2, 8, 2, 200, 200, gen.BSHD, True),      # GQA causal, ragged
    (1, 4, 1, 129, 129, gen.BHSD, False),     # MQA
    (2, 4, 4, 300, 77, gen.BHSD, False),      # cross attention
    (1, 4, 2, 150, 100, gen.BSHD, True),      # rows that see no key
    (1, 4, 2, 70, 300, gen.BSHD, True),       # bottom-right alignment
])
def test_d64_backward_all_elements(B, Hq, Hkv, Sq, Sk, layout, causal):
    p = gen.prefill_inputs(B, Hq, Hkv, Sq, Sk, layout=layout, causal=causal,
                           seed=500 + Sq + Sk, n_hot=2, d=64)
    check_problem(p, gen.output_grad(p, 8), f"d64 B{B} Hq{Hq} Hkv{Hkv} Sq{Sq} Sk{Sk} causal{causal}")


def test_d64_backward_full_size_sampled_group():
    p = gen.headdim64_causal_gqa()
    _check_full_size(p, gen.output_grad(p, 7), [(2, 3)], "d64 gqa causal b8 s8192")
