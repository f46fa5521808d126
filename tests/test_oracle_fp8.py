"""The FP8 (E4M3) oracle against what fixes it independently: torch's
float8_e4m3fn decoding for every byte, the format's closed forms, a float64
torch attention on the decoded values, and planted mistakes in private copies
that these pins must catch."""
import math

import numpy as np
import pytest
import torch

import attn_inputs as gen
import oracle.fp8 as f8


def _torch_decode_all():
    b = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return b.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def pin_table(decode):
    got = decode(np.arange(256, dtype=np.uint8))
    ref = _torch_decode_all()
    nan_g, nan_r = np.isnan(got), np.isnan(ref)
    assert np.array_equal(nan_g, nan_r), "NaN encodings differ"
    assert np.array_equal(got[~nan_g], ref[~nan_r]), "decoded values differ from torch"
    assert np.array_equal(np.signbit(got[~nan_g]), np.signbit(ref[~nan_r])), "signs of zero"


def pin_closed_forms(decode):
    cases = {0x38: 1.0, 0x40: 2.0, 0x30: 0.5, 0x7E: 448.0, 0xFE: -448.0, 0x08: 2.0 ** -6,
             0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x39: 1.125, 0x00: 0.0, 0x78: 256.0}
    for byte, val in cases.items():
        got = float(decode(np.array([byte], np.uint8))[0])
        assert got == val, (hex(byte), got, val)
    assert math.copysign(1.0, float(decode(np.array([0x80], np.uint8))[0])) == -1.0
    assert np.isnan(decode(np.array([0x7F, 0xFF], np.uint8))).all()


PINS = [pin_table, pin_closed_forms]


def test_decode_pins():
    for p in PINS:
        p(f8.e4m3_to_f64)


def _bias8(b):
    b = np.asarray(b, np.uint8).astype(np.int64)
    e, m = (b >> 3) & 15, (b & 7) / 8.0
    v = np.where(e == 0, m * 2.0 ** -6, (1 + m) * np.exp2(e - 8.0))
    return np.where(b & 0x80, -v, v)


def _subnormal_as_normal(b):
    b = np.asarray(b, np.uint8).astype(np.int64)
    e, m = (b >> 3) & 15, (b & 7) / 8.0
    v = np.where((e == 15) & (b & 7 == 7), np.nan, (1 + m) * np.exp2(e - 7.0))
    return np.where(b & 0x80, -v, v)


def _ieee_like_top_binade(b):
    # exponent field 15 read as inf/NaN (the IEEE convention, not E4M3 FN)
    out = f8.e4m3_to_f64(b)
    e = (np.asarray(b, np.uint8) >> 3) & 15
    return np.where(e == 15, np.nan, out)


def _sign_dropped(b):
    return np.abs(f8.e4m3_to_f64(b))


@pytest.mark.parametrize("mutant", [_bias8, _subnormal_as_normal, _ieee_like_top_binade,
                                    _sign_dropped])
def test_planted_decode_mistake_is_caught(mutant):
    caught = 0
    for p in PINS:
        try:
            p(mutant)
        except AssertionError:
            caught += 1
    assert caught, mutant.__name__


def _torch_attention(p):
    """float64 torch attention on the decoded, descaled values."""
    dec = lambda x, s: torch.from_numpy(s * _torch_decode_all()[x.astype(np.int64)])
    q, k, v = dec(p.q, p.descale_q), dec(p.k, p.descale_k), dec(p.v, p.descale_v)
    if p.layout == gen.BSHD:
        q, k, v = (t.permute(0, 2, 1, 3) for t in (q, k, v))
    G = p.Hq // p.Hkv
    k = k.repeat_interleave(G, dim=1)
    v = v.repeat_interleave(G, dim=1)
    s = float(np.float32(p.scale)) * (q @ k.transpose(-1, -2))
    if p.causal:
        i = torch.arange(p.Sq)[:, None]
        j = torch.arange(p.Sk)[None, :]
        s = s.masked_fill(j > i + (p.Sk - p.Sq), -math.inf)
    lse = torch.logsumexp(s, dim=-1)
    pr = torch.exp(s - lse[..., None])
    pr = torch.nan_to_num(pr, nan=0.0)
    return (pr @ v).numpy(), lse.numpy()


CASES = [
    dict(B=1, Hq=4, Hkv=4, Sq=37, Sk=53, layout=gen.BSHD, causal=False),
    dict(B=2, Hq=4, Hkv=2, Sq=40, Sk=40, layout=gen.BHSD, causal=True),
    dict(B=1, Hq=3, Hkv=1, Sq=50, Sk=20, layout=gen.BSHD, causal=True),   # rows with no key
]


@pytest.mark.parametrize("case", CASES)
def test_attention_fp8_against_torch(case):
    p = gen.fp8_prefill_inputs(**case, seed=11, descales=(0.75, 1.5, 0.3125), amp=(2.0, 1.0, 3.0))
    o, lse = f8.attention_fp8(p.q, p.k, p.v, p.descale_q, p.descale_k, p.descale_v, p.B, p.Hq,
                              p.Hkv, p.Sq, p.Sk, p.scale, p.causal, p.layout, workers=1)
    ro, rl = _torch_attention(p)
    empty = np.isneginf(rl)
    assert np.array_equal(np.isneginf(lse), empty)
    assert np.allclose(o, ro, rtol=1e-12, atol=1e-12)
    assert np.allclose(lse[~empty], rl[~empty], rtol=1e-12, atol=1e-12)
    assert np.all(o[np.broadcast_to(empty[..., None], o.shape)] == 0)


def test_sampled_rows_match_full():
    p = gen.fp8_prefill_inputs(1, 2, 1, 70, 90, causal=True, seed=12)
    o, lse = f8.attention_fp8(p.q, p.k, p.v, 1, 1, 1, 1, 2, 1, 70, 90, p.scale, True, p.layout,
                              workers=1)
    rows = [(0, 0, 3), (0, 1, 69), (0, 1, 0)]
    os_, ls = f8.attention_fp8(p.q, p.k, p.v, 1, 1, 1, 1, 2, 1, 70, 90, p.scale, True, p.layout,
                               rows=rows, workers=1)
    for b, h, i in rows:
        # the same rows of the same definition (key counts, hence BLAS blocking, differ)
        assert np.allclose(os_[b, h, i], o[b, h, i], rtol=1e-12, atol=1e-14)
        assert abs(ls[b, h, i] - lse[b, h, i]) <= 1e-12


def _planted_descale_v_dropped(m):
    orig = m.attention_fp8
    m_attn = lambda q, k, v, dq, dk, dv, *a, **kw: orig(q, k, v, dq, dk, 1.0, *a, **kw)
    return m_attn


def _planted_k_descale_on_v(m):
    orig = m.attention_fp8
    return lambda q, k, v, dq, dk, dv, *a, **kw: orig(q, k, v, dq, dv, dk, *a, **kw)


@pytest.mark.parametrize("plant", [_planted_descale_v_dropped, _planted_k_descale_on_v])
def test_planted_descale_mistake_is_caught(plant):
    fn = plant(f8)
    p = gen.fp8_prefill_inputs(**CASES[0], seed=11, descales=(0.75, 1.5, 0.3125))
    o, _ = fn(p.q, p.k, p.v, p.descale_q, p.descale_k, p.descale_v, p.B, p.Hq, p.Hkv, p.Sq, p.Sk,
              p.scale, p.causal, p.layout, workers=1)
    ro, _ = _torch_attention(p)
    assert not np.allclose(o, ro, rtol=1e-9, atol=1e-9)


def test_generator_encodes_to_nearest():
    # the encoder rounds to the nearest E4M3 value (checked by the oracle's
    # decoder on a fine grid of inputs)
    x = np.linspace(-460, 460, 20001).astype(np.float32)
    x = x[np.abs(x) <= 448]
    b = gen.e4m3_bytes(x)
    dec = f8.e4m3_to_f64(np.arange(256, dtype=np.uint8))
    fin = dec[np.isfinite(dec)]
    best = np.min(np.abs(x[:, None].astype(np.float64) - fin[None, :]), axis=1)
    assert np.all(np.abs(f8.e4m3_to_f64(b) - x) <= best + 1e-12)
