"""Plant plausible mistakes in a private copy of the oracle (on the CPU) and
check that the pins catch every one of them."""
import importlib.util
import os

import numpy as np
import pytest

import oracle.online as onl
import pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def fresh_oracle():
    spec = importlib.util.spec_from_file_location(
        "oracle_mutant", os.path.join(ROOT, "oracle", "attention.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def _mut_no_scale(m):
    m.scores = lambda q, k, scale: q @ k.T


def _mut_exp_sign(m):
    def rs(s):
        mm = s.max(axis=1)
        mx = np.where(mm == -np.inf, 0.0, mm)
        e = np.exp(s + mx[:, None])  # exp(s + m) instead of exp(s - m)
        l = e.sum(axis=1)
        return e / np.where(l > 0, l, 1.0)[:, None], mm, l
    m.row_softmax = rs


def _mut_gqa_modulo(m):
    m.kv_head_of = lambda h, Hq, Hkv: h % Hkv


def _mut_causal_off_by_one(m):
    m.visible_keys = lambda i, Sq, Sk, causal: Sk if not causal else max(0, min(Sk, i + (Sk - Sq)))


def _mut_causal_top_left(m):
    m.visible_keys = lambda i, Sq, Sk, causal: Sk if not causal else max(0, min(Sk, i + 1))


def _mut_pv_transposed(m):
    orig_scores = m.scores

    def attend_rows(q, k, v, scale, n_visible=None):
        s = orig_scores(q, k, scale)
        if n_visible is not None:
            j = np.arange(k.shape[0])
            s = np.where(j[None, :] >= np.asarray(n_visible)[:, None], -np.inf, s)
        p, mm, l = m.row_softmax(s)
        vv = v[::-1]  # rows of V paired with the wrong keys
        return p @ vv, mm + np.log(np.where(l > 0, l, 1))
    m.attend_rows = attend_rows


def _mut_lse_log2(m):
    orig = m.attend_rows

    def attend_rows(q, k, v, scale, n_visible=None):
        o, lse = orig(q, k, v, scale, n_visible)
        s = m.scores(q, k, scale)
        mx = s.max(axis=1) if s.size else np.zeros(q.shape[0])
        return o, np.where(np.isinf(lse), lse, mx + (lse - mx) / np.log(2))
    m.attend_rows = attend_rows


def _mut_lse_no_max(m):
    orig = m.attend_rows

    def attend_rows(q, k, v, scale, n_visible=None):
        o, lse = orig(q, k, v, scale, n_visible)
        s = m.scores(q, k, scale)
        mx = s.max(axis=1) if s.size else np.zeros(q.shape[0])
        return o, np.where(np.isinf(lse), lse, lse - mx)
    m.attend_rows = attend_rows


def _mut_layout_swapped(m):
    m._logical = lambda x, layout: x.transpose(0, 2, 1, 3) if layout == m.BHSD else x


def _mut_page_slot_swapped(m):
    def gather_pages(pool, table, n, b, g):
        t = np.arange(int(n))
        return pool[table[b, t % m.PAGE], (t // m.PAGE) % m.PAGE, g]
    m.gather_pages = gather_pages


def _mut_no_normalisation(m):
    orig = m.row_softmax

    def rs(s):
        p, mm, l = orig(s)
        return p * np.where(l > 0, l, 1)[:, None], mm, l
    m.row_softmax = rs


def _mut_scale_not_f32(m):
    m.scale_as_f32 = lambda s: float(s) * (1 + 1e-6)


def _mut_append_past_end(m):
    def append_token(k_pool, v_pool, table, lens, k_new, v_new):
        kp, vp = k_pool.copy(), v_pool.copy()
        for b in range(len(lens)):
            t = int(lens[b])          # one slot too far
            kp[table[b, t // m.PAGE], t % m.PAGE] = k_new[b]
            vp[table[b, t // m.PAGE], t % m.PAGE] = v_new[b]
        return kp, vp
    m.append_token = append_token


def _mut_append_k_only(m):
    orig = m.append_token

    def append_token(k_pool, v_pool, table, lens, k_new, v_new):
        kp, _ = orig(k_pool, v_pool, table, lens, k_new, v_new)
        return kp, v_pool.copy()
    m.append_token = append_token


def _mut_append_heads_reversed(m):
    orig = m.append_token

    def append_token(k_pool, v_pool, table, lens, k_new, v_new):
        return orig(k_pool, v_pool, table, lens, k_new[:, ::-1], v_new[:, ::-1])
    m.append_token = append_token


MUTANTS = [_mut_no_scale, _mut_exp_sign, _mut_gqa_modulo, _mut_causal_off_by_one,
           _mut_causal_top_left, _mut_pv_transposed, _mut_lse_log2, _mut_lse_no_max,
           _mut_layout_swapped, _mut_page_slot_swapped, _mut_no_normalisation,
           _mut_scale_not_f32, _mut_append_past_end, _mut_append_k_only,
           _mut_append_heads_reversed]


@pytest.mark.parametrize("mutate", MUTANTS, ids=lambda f: f.__name__)
def test_pins_catch_mutant(mutate):
    m = fresh_oracle()
    mutate(m)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(m, onl)
        except Exception as e:  # noqa: BLE001 - any failure counts as caught
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin caught {mutate.__name__}"
