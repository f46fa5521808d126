"""The backward oracle against what the mathematics fixes (finite differences
of the forward oracle, torch's float64 autograd, identities, closed forms),
and planted mistakes in a private copy of it that those pins must catch."""
import importlib.util
import os

import numpy as np
import pytest

import bwd_pins
import oracle.backward as bwd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("name,pin", bwd_pins.ALL, ids=[n for n, _ in bwd_pins.ALL])
def test_backward_pin(name, pin):
    pin(bwd)


def test_magnitudes_bound_the_gradients():
    p, do = bwd_pins._problem(Sq=40, Sk=57, causal=True)
    out = bwd.attention_backward(p.q, p.k, p.v, do, p.B, p.Hq, p.Hkv, p.Sq, p.Sk, p.scale, True,
                                 p.layout, workers=1, magnitudes=True)
    for g, m in zip(out[:3], out[3:]):
        assert np.all(m >= 0) and np.all(np.abs(g) <= m * (1 + 1e-12) + 1e-300)


def test_flops_backward():
    assert bwd.flops_backward(1, 1, 2, 3, 4, False) == 10 * 2 * 3 * 4
    assert bwd.flops_backward(1, 1, 2, 3, 4, True) == 5 * 2 * 3 * 4


def fresh():
    spec = importlib.util.spec_from_file_location("bwd_mutant",
                                                  os.path.join(ROOT, "oracle", "backward.py"),
                                                  submodule_search_locations=None)
    m = importlib.util.module_from_spec(spec)
    m.__package__ = "oracle"
    spec.loader.exec_module(m)
    return m


def _with_grad_rows(body):
    def plant(m):
        def grad_rows(q, k, v, do, scale, n_visible=None, bias=None):
            p = m.probabilities(q, k, scale, n_visible, bias)
            return body(p, q, k, v, do, scale)
        m.grad_rows = grad_rows
    return plant


def _no_row_term(p, q, k, v, do, s):
    ds = p * (do @ v.T)
    return s * ds @ k, s * ds.T @ q, p.T @ do


def _row_term_sign(p, q, k, v, do, s):
    dp = do @ v.T
    ds = p * (dp + (p * dp).sum(axis=1, keepdims=True))
    return s * ds @ k, s * ds.T @ q, p.T @ do


def _dk_unscaled(p, q, k, v, do, s):
    dp = do @ v.T
    ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    return s * ds @ k, ds.T @ q, p.T @ do


def _dq_with_v(p, q, k, v, do, s):
    dp = do @ v.T
    ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    return s * ds @ v, s * ds.T @ q, p.T @ do


def _dv_rows_reversed(p, q, k, v, do, s):
    dp = do @ v.T
    ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    return s * ds @ k, s * ds.T @ q, (p.T @ do)[::-1]


def _row_term_column_sum(p, q, k, v, do, s):
    dp = do @ v.T
    ds = p * (dp - (p * dp).sum(axis=0, keepdims=True))
    return s * ds @ k, s * ds.T @ q, p.T @ do


def _mask_ignored(m):
    orig = m.probabilities
    m.probabilities = lambda q, k, scale, n_visible=None, bias=None: orig(q, k, scale, None, bias)


def _group_overwrites(m):
    # the last query head of a group overwrites dK/dV instead of adding
    orig = m.attention_backward

    def ab(q, k, v, do, B, Hq, Hkv, Sq, Sk, scale, causal, layout, **kw):
        if Hq == Hkv:
            return orig(q, k, v, do, B, Hq, Hkv, Sq, Sk, scale, causal, layout, **kw)
        G = Hq // Hkv
        sl = (slice(None), slice(None), slice(G - 1, None, G)) if layout == 0 else \
            (slice(None), slice(G - 1, None, G))
        r = orig(q[sl], k, v, do[sl], B, Hkv, Hkv, Sq, Sk, scale, causal, layout, **kw)
        full = orig(q, k, v, do, B, Hq, Hkv, Sq, Sk, scale, causal, layout, **kw)
        return (full[0], r[1], r[2]) + tuple(full[3:])
    m.attention_backward = ab


def _alibi_ignored_in_backward(m):
    # the recomputed probabilities leave the bias out
    orig = m.probabilities
    m.probabilities = lambda q, k, scale, n_visible=None, bias=None: orig(q, k, scale, n_visible)


MUTANTS = {
    "ALiBi bias left out of the recomputed P": _alibi_ignored_in_backward,
    "row term dropped": _with_grad_rows(_no_row_term),
    "row term sign": _with_grad_rows(_row_term_sign),
    "dK without the scale": _with_grad_rows(_dk_unscaled),
    "dQ from V instead of K": _with_grad_rows(_dq_with_v),
    "dV rows paired with the wrong keys": _with_grad_rows(_dv_rows_reversed),
    "row term summed over the wrong axis": _with_grad_rows(_row_term_column_sum),
    "causal mask ignored in the backward": _mask_ignored,
    "GQA head gradients overwrite": _group_overwrites,
}


@pytest.mark.parametrize("name", list(MUTANTS))
def test_planted_mistake_is_caught(name):
    m = fresh()
    MUTANTS[name](m)
    caught = []
    for pin_name, pin in bwd_pins.ALL:
        try:
            pin(m)
        except (AssertionError, ValueError) as e:
            caught.append((pin_name, str(e)[:80]))
    assert caught, f"no pin catches: {name}"
