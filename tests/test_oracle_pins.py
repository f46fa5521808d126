"""The fp64 oracle against its pins (CPU only)."""
import math

import numpy as np
import pytest

import oracle.attention as att
import oracle.online as onl
import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(att, onl)


def test_closed_form_three_keys():
    """scale 1, q = e0, keys 0, e0, 2*e0: scores 0, 1, 2, so the weights are
    (1, e, e^2) / (1 + e + e^2); with V = identity rows, O is that weight
    vector and LSE = ln(1 + e + e^2)."""
    d = 4
    q = np.array([[1.0, 0, 0, 0]])
    k = np.array([[0.0, 0, 0, 0], [1.0, 0, 0, 0], [2.0, 0, 0, 0]])
    v = np.eye(3, d)
    o, lse = att.attend_rows(q, k, v, 1.0)
    z = 1 + math.e + math.e ** 2
    assert np.allclose(o[0], [1 / z, math.e / z, math.e ** 2 / z, 0.0], rtol=1e-15, atol=0)
    assert abs(lse[0] - math.log(z)) <= 1e-15


def test_closed_form_two_queries_causal():
    """Causal, Sq = Sk = 2, scale 1: row 0 sees only key 0 (O = V0, LSE = s00);
    row 1 with q1 = (ln 3) e0 against keys 0 and e0 has scores 0, ln 3 and
    weights 1/4, 3/4."""
    ln3 = math.log(3.0)
    q = np.array([[0.5, 0.0], [ln3, 0.0]])
    k = np.array([[0.0, 0.0], [1.0, 0.0]])
    v = np.array([[4.0, 0.0], [0.0, 8.0]])
    nv = [att.visible_keys(i, 2, 2, True) for i in range(2)]
    o, lse = att.attend_rows(q, k, v, 1.0, nv)
    assert np.array_equal(o[0], v[0]) and lse[0] == 0.0
    assert np.allclose(o[1], [1.0, 6.0], rtol=1e-15)
    assert abs(lse[1] - math.log(4.0)) <= 1e-15


def test_golden_fixture_regression():
    """The oracle still reproduces the fixture that tests/golden/make_golden.py
    wrote from it (guards against accidental changes of the oracle)."""
    import json, os
    import attn_inputs as gen
    path = os.path.join(os.path.dirname(__file__), "golden", "oracle_small.json")
    fx = json.load(open(path))
    for case in fx["cases"]:
        p = gen.prefill_inputs(case["B"], case["Hq"], case["Hkv"], case["Sq"], case["Sk"],
                               layout=case["layout"], causal=case["causal"], seed=case["seed"])
        o, lse = att.attention(p.q, p.k, p.v, p.B, p.Hq, p.Hkv, p.Sq, p.Sk, p.scale,
                               p.causal, p.layout)
        assert np.allclose(o.ravel(), np.array(case["o"]), rtol=1e-13, atol=1e-15)
        ref_l = np.array([(-np.inf if x is None else x) for x in case["lse"]])
        assert np.allclose(lse.ravel(), ref_l, rtol=1e-13, atol=1e-15)
