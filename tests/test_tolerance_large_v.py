"""CPU checks of the large-V bound in tests/tolerance.py: an emulation of the
arithmetic it covers (probabilities rounded to fp16 against a running max
that may sit up to 2^12 below the true one, the sum of the rounded values as
denominator, fp32 accumulation, O rounded to bf16) stays inside it on inputs
where the plain bound (2 ulp + 1e-3) does not hold -- so the reading is needed,
and the derived bound is not looser than the emulation requires by more than
a small factor."""
import numpy as np
import pytest

import attn_inputs as gen
import oracle.attention as att
from tolerance import (P_UNIT_F16, check_o, check_o_large_v, o_tolerance, pv_spread_rows)


def bf16_round(x):
    return att.bf16_to_f64(gen.f32_to_bf16_bits(np.asarray(x, np.float32)))


def emulate_fp16_pv(q, k, v, scale, shift, round_out=True):
    """O with probabilities exp(s - m + shift*ln2) rounded to fp16 (shift >= 0
    stands for a running max below the row max), summed in fp32, rounded to
    bf16 unless round_out is False."""
    s = att.scores(q, k, scale)
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m) * 2.0 ** shift
    p16 = p.astype(np.float16).astype(np.float64)
    l = p16.astype(np.float32).sum(axis=1, dtype=np.float32).astype(np.float64)
    acc = (p16.astype(np.float32) @ v.astype(np.float32)).astype(np.float64)
    o = acc / l[:, None]
    return bf16_round(o) if round_out else o


def problem(seed, n, sk, v_amp, q_amp):
    r = np.random.default_rng(seed)
    q = att.bf16_to_f64(gen.f32_to_bf16_bits(q_amp * r.standard_normal((n, 128), np.float32)))
    k = att.bf16_to_f64(gen.f32_to_bf16_bits(r.standard_normal((sk, 128), np.float32)))
    v = att.bf16_to_f64(gen.f32_to_bf16_bits(v_amp * r.standard_normal((sk, 128), np.float32)))
    return q, k, v


@pytest.mark.parametrize("shift", [0, 5, 12])
@pytest.mark.parametrize("sk,q_amp", [(40, 4.0), (700, 1.0), (3000, 2.0)])
def test_emulation_inside_large_v_bound(shift, sk, q_amp):
    q, k, v = problem(sk + shift, 48, sk, 300.0, q_amp)
    sc = att.scale_as_f32(1 / np.sqrt(128))
    o_ref, _ = att.attend_rows(q, k, v, sc)
    o = emulate_fp16_pv(q, k, v, sc, shift)
    spread = pv_spread_rows(q, k, v, sc)
    _, r, r_plain = check_o_large_v(o, o_ref, spread, "emulation")
    assert r <= 1.0
    # on these inputs the plain bound does not hold
    assert r_plain > 1.0, r_plain


def test_plain_bound_holds_for_unit_v():
    """With |V| of order one the fp16 rounding stays inside 2 ulp + 1e-3."""
    q, k, v = problem(9, 64, 500, 1.0, 4.0)
    sc = att.scale_as_f32(1 / np.sqrt(128))
    o_ref, _ = att.attend_rows(q, k, v, sc)
    check_o(emulate_fp16_pv(q, k, v, sc, 0), o_ref, "unit V")


def test_spread_is_not_loose():
    """Before the output rounding, the emulated error reaches a good part of
    the spread term somewhere and never exceeds it (the bound is a first-order
    estimate, not a gross over-estimate)."""
    q, k, v = problem(11, 64, 60, 300.0, 4.0)
    sc = att.scale_as_f32(1 / np.sqrt(128))
    o_ref, _ = att.attend_rows(q, k, v, sc)
    o = emulate_fp16_pv(q, k, v, sc, 0, round_out=False)
    spread = pv_spread_rows(q, k, v, sc)
    big = spread > 1e-2
    frac = (np.abs(o - o_ref)[big] / spread[big]).max()
    assert 0.1 < frac <= 1.0 + 2.0 ** -4, frac


def test_spread_closed_form_for_two_keys():
    """Two keys with probabilities 3/4 and 1/4 (exact in fp16, so the
    emulation is exact up to the output rounding): spread = u * (3/4 |v0 - o| +
    1/4 |v1 - o|)."""
    k = np.zeros((2, 128))
    q = np.zeros((1, 128))
    q[0, 0] = 1.0
    k[0, 0] = np.log(3.0)           # scores log 3 and 0 at scale 1
    v = np.array([[100.0] * 128, [-300.0] * 128])
    o_ref, _ = att.attend_rows(q, k, v, 1.0)
    assert np.allclose(o_ref, 0.0)
    spread = pv_spread_rows(q, k, v, 1.0)
    assert np.allclose(spread, P_UNIT_F16 * (0.75 * 100 + 0.25 * 300))
    assert np.all(o_tolerance(o_ref) < spread)


def test_lse_bound_on_the_bf16_fallback():
    """Emulated bf16 probabilities (exact row max, so the largest one is 1)
    on peaky rows: l sums the rounded values; the LSE error stays within
    1e-3 + 2^-8 and on some rows exceeds the fp16-path bound of 1e-3."""
    import attn_inputs as gen
    from tolerance import LSE_ABS, P_UNIT_BF16
    r = np.random.default_rng(7)
    worst = 0.0
    for _ in range(200):
        n = int(r.integers(2, 64))
        s = r.standard_normal(n) * float(r.choice([0.5, 2.0, 6.0]))   # flat to peaky rows
        m = s.max()
        p = np.exp(s - m).astype(np.float32)
        pb = (gen.f32_to_bf16_bits(p).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        lse_emul = m + np.log(pb.sum())
        lse_exact = m + np.log(np.exp(s - m).sum())
        err = abs(lse_emul - lse_exact)
        assert err <= LSE_ABS + P_UNIT_BF16
        worst = max(worst, err)
    # a row whose probabilities all sit just below a bf16 rounding midpoint,
    # (1 + 0.99 * 2^-8) * 2^-j: every one rounds down by almost 2^-8 of itself
    p = np.concatenate([[1.0], (1.0 + 0.99 * 2.0 ** -8) * 2.0 ** -np.arange(1, 11)])
    s = np.log(p)
    pb = (gen.f32_to_bf16_bits(p.astype(np.float32)).astype(np.uint32) << 16).view(np.float32)
    err = abs(np.log(pb.astype(np.float64).sum()) - np.log(np.exp(s).sum()))
    assert LSE_ABS < err <= LSE_ABS + P_UNIT_BF16
    assert worst <= LSE_ABS + P_UNIT_BF16
