"""ALiBi in the oracle: against torch's float64 attention with the bias as a
float mask, special cases that reduce it to plain attention, its shift
property under causal masking, and planted mistakes that those pins catch."""
import importlib.util
import os

import numpy as np
import pytest
import torch

import attn_inputs as gen
import oracle.attention as att

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def slopes(H):
    """The geometric slopes of the ALiBi paper for H heads (2^(-8h/H))."""
    return (2.0 ** (-8.0 * np.arange(1, H + 1) / H)).astype(np.float32)


def torch_alibi(p, sl):
    f = [torch.from_numpy(np.ascontiguousarray(att._logical(att.bf16_to_f64(x), p.layout)))
         for x in (p.q, p.k, p.v)]
    q, k, v = f
    G = p.Hq // p.Hkv
    k, v = k.repeat_interleave(G, dim=1), v.repeat_interleave(G, dim=1)
    i = torch.arange(p.Sq, dtype=torch.float64)[:, None]
    j = torch.arange(p.Sk, dtype=torch.float64)[None, :]
    dist = (i + (p.Sk - p.Sq) - j).abs()
    bias = -torch.from_numpy(sl.astype(np.float64))[:, None, None] * dist      # [Hq, Sq, Sk]
    if p.causal:
        bias = bias.masked_fill(j > i + (p.Sk - p.Sq), float("-inf"))
    sc = float(np.float32(p.scale))
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=bias[None], scale=sc)
    lse = torch.logsumexp(sc * (q @ k.transpose(-1, -2)) + bias[None], dim=-1)
    return o.numpy(), lse.numpy()


CASES = [(2, 4, 2, 37, 37, gen.BSHD, True), (1, 4, 4, 20, 53, gen.BHSD, False),
         (1, 8, 2, 48, 70, gen.BSHD, True)]


def run(m, p, sl):
    return m.attention(p.q, p.k, p.v, p.B, p.Hq, p.Hkv, p.Sq, p.Sk, p.scale, p.causal, p.layout,
                       workers=1, alibi_slopes=sl)


@pytest.mark.parametrize("B,Hq,Hkv,Sq,Sk,layout,causal", CASES)
def test_alibi_matches_torch(B, Hq, Hkv, Sq, Sk, layout, causal):
    p = gen.prefill_inputs(B, Hq, Hkv, Sq, Sk, layout=layout, causal=causal, seed=31)
    sl = slopes(Hq)
    o, lse = run(att, p, sl)
    o_t, lse_t = torch_alibi(p, sl)
    assert np.abs(o - o_t).max() <= 1e-12 and np.abs(lse - lse_t).max() <= 1e-12


def test_zero_slopes_are_plain_attention():
    p = gen.prefill_inputs(1, 4, 2, 30, 45, layout=gen.BSHD, causal=True, seed=32)
    a = run(att, p, np.zeros(4, np.float32))
    b = att.attention(p.q, p.k, p.v, 1, 4, 2, 30, 45, p.scale, True, gen.BSHD, workers=1)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_causal_bias_is_a_per_row_shift_plus_key_ramp():
    """Causal: over the visible keys, -s|i + off - j| = -s(i + off) + s j, and
    a per-row constant leaves O unchanged and moves LSE by it; so O equals
    attention with the key-only bias +s*j, computed here by adding s*j/scale
    to K's scores through an extra feature dimension."""
    p = gen.prefill_inputs(1, 2, 2, 25, 25, layout=gen.BHSD, causal=True, seed=33)
    sl = np.array([0.25, 0.0625], np.float32)
    o, lse = run(att, p, sl)
    q = att.bf16_to_f64(p.q)[0]
    k = att.bf16_to_f64(p.k)[0]
    v = att.bf16_to_f64(p.v)[0]
    sc = float(np.float32(p.scale))
    for h in range(2):
        # append a feature: q gets 1, key j gets s*j/scale
        qx = np.concatenate([q[h], np.ones((25, 1))], axis=1)
        kx = np.concatenate([k[h], (float(sl[h]) * np.arange(25) / sc)[:, None]], axis=1)
        nv = np.arange(1, 26)
        o2, l2 = att.attend_rows(qx, kx, v[h], sc, nv)
        assert np.abs(o2 - o[0, h]).max() <= 1e-12
        assert np.abs((l2 - float(sl[h]) * np.arange(25)) - lse[0, h]).max() <= 1e-9


def fresh():
    spec = importlib.util.spec_from_file_location("alibi_mutant",
                                                  os.path.join(ROOT, "oracle", "attention.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def _mut_sign(m):
    orig = m.alibi_bias
    m.alibi_bias = lambda rows, Sq, Sk, slope: -orig(rows, Sq, Sk, slope)


def _mut_top_left(m):
    orig = m.alibi_bias
    m.alibi_bias = lambda rows, Sq, Sk, slope: orig(rows, Sk, Sk, slope)


def _mut_kv_head_slope(m):
    orig = m.attention

    def a(q, k, v, B, Hq, Hkv, Sq, Sk, scale, causal, layout, chunk=256, workers=None,
          alibi_slopes=None):
        if alibi_slopes is not None:
            G = Hq // Hkv
            alibi_slopes = np.repeat(alibi_slopes[::G], G)
        return orig(q, k, v, B, Hq, Hkv, Sq, Sk, scale, causal, layout, chunk, workers,
                    alibi_slopes)
    m.attention = a


def _mut_unscaled_bias(m):
    orig = m.alibi_bias
    m.alibi_bias = lambda rows, Sq, Sk, slope: orig(rows, Sq, Sk, slope) / np.sqrt(128)


@pytest.mark.parametrize("plant", [_mut_sign, _mut_top_left, _mut_kv_head_slope,
                                   _mut_unscaled_bias],
                         ids=["sign", "top-left alignment", "slope per K/V head", "bias scaled"])
def test_planted_alibi_mistake_is_caught(plant):
    m = fresh()
    plant(m)
    caught = False
    for B, Hq, Hkv, Sq, Sk, layout, causal in CASES:
        p = gen.prefill_inputs(B, Hq, Hkv, Sq, Sk, layout=layout, causal=causal, seed=31)
        sl = slopes(Hq)
        o, lse = run(m, p, sl)
        o_t, lse_t = torch_alibi(p, sl)
        if not (np.abs(o - o_t).max() <= 1e-12 and np.abs(lse - lse_t).max() <= 1e-12):
            caught = True
    assert caught
