"""Pin of the oracle's per-row entry point (`attention_sampled`, the checker of
the full-size parity tests): on small problems it must give, for every query
row, exactly what the materialised oracle gives for that row ("IO-aware
tiling strategy in FlashAttention-4", body: the rows of the softmax are
independent, so any subset of rows has the definition's values).  Mistakes
planted in a private copy of its source (on the CPU) must be caught."""
import importlib.util
import os

import numpy as np
import pytest

import attn_inputs as gen
import oracle.attention as att

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CASES = [
    # B, Hq, Hkv, Sq, Sk, causal, layout
    (2, 4, 4, 37, 37, False, gen.BSHD),
    (2, 4, 4, 37, 37, True, gen.BHSD),
    (1, 8, 2, 23, 61, True, gen.BSHD),     # GQA, Sq < Sk (bottom-right offset)
    (2, 6, 1, 29, 40, False, gen.BHSD),    # MQA
    (1, 4, 2, 70, 9, True, gen.BSHD),      # Sq > Sk: rows 0..60 see no key
    (2, 2, 1, 50, 3, True, gen.BHSD),      # most rows empty
]


def all_rows(B, Hq, Sq):
    return [(b, h, i) for b in range(B) for h in range(Hq) for i in range(Sq)]


def sampled_vs_full(mod, case, seed, rows=None, d=32):
    B, Hq, Hkv, Sq, Sk, causal, layout = case
    p = gen.prefill_inputs(B, Hq, Hkv, Sq, Sk, causal=causal, layout=layout, seed=seed, d=d)
    o, lse = att.attention(p.q, p.k, p.v, B, Hq, Hkv, Sq, Sk, p.scale, causal, layout)
    rows = rows if rows is not None else all_rows(B, Hq, Sq)
    os_, ls = mod.attention_sampled(p.q, p.k, p.v, B, Hq, Hkv, Sq, Sk, p.scale, causal,
                                    layout, rows)
    ref_o = np.stack([o[b, h, i] for b, h, i in rows])
    ref_l = np.array([lse[b, h, i] for b, h, i in rows])
    same_inf = np.array_equal(np.isinf(ls), np.isinf(ref_l)) and \
        np.array_equal(ls[np.isinf(ls)], ref_l[np.isinf(ref_l)])
    fin = ~np.isinf(ref_l)
    return (same_inf and np.allclose(os_, ref_o, rtol=1e-12, atol=1e-13)
            and np.allclose(ls[fin], ref_l[fin], rtol=1e-12, atol=1e-13))


@pytest.mark.parametrize("case", CASES)
def test_every_row_matches_the_full_oracle(case):
    assert sampled_vs_full(att, case, seed=71)


def test_shuffled_and_repeated_rows():
    case = CASES[2]
    rows = all_rows(case[0], case[1], case[3])
    r = np.random.default_rng(5)
    pick = [rows[int(i)] for i in r.integers(len(rows), size=300)]   # repeats, any order
    assert sampled_vs_full(att, case, seed=72, rows=pick)


def test_group_of_empty_rows_only():
    # every sampled row of the (b, h) group sees no key: kmax = 0
    case = CASES[4]
    rows = [(0, h, i) for h in range(case[1]) for i in (0, 5, 60)]
    assert sampled_vs_full(att, case, seed=73, rows=rows)
    p = gen.prefill_inputs(*case[:5], causal=True, layout=case[6], seed=73, d=32)
    o, lse = att.attention_sampled(p.q, p.k, p.v, *case[:5], p.scale, True, case[6], rows)
    assert np.all(o == 0) and np.all(lse == -np.inf)


def mutant(old, new):
    """A copy of oracle/attention.py whose attention_sampled has `old`
    replaced by `new` (the text must occur inside that function)."""
    src = open(os.path.join(ROOT, "oracle", "attention.py")).read()
    start = src.index("def attention_sampled(")
    end = src.index("\ndef ", start + 1)
    body = src[start:end]
    assert old in body, old
    src = src[:start] + body.replace(old, new) + src[end:]
    spec = importlib.util.spec_from_loader("oracle_sampled_mutant", loader=None)
    m = importlib.util.module_from_spec(spec)
    exec(compile(src, "oracle_sampled_mutant", "exec"), m.__dict__)
    return m


MUTANTS = {
    # causal alignment top-left instead of bottom-right
    "top_left": ("visible_keys(int(i), Sq, Sk, causal)", "visible_keys(int(i), Sk, Sk, causal)"),
    # batch and head swapped when picking the query rows
    "swap_b_h": ("qv[b, h, rows]", "qv[h % qv.shape[0], b % qv.shape[1], rows]"),
    # wrong K/V head for GQA (modulo instead of contiguous groups)
    "gqa_modulo": ("g = kv_head_of(h, Hq, Hkv)", "g = h % Hkv"),
    # keys truncated to the shortest visible prefix of the group
    "kmax_min": ("kmax = int(nv.max())", "kmax = int(nv.min())"),
    # results written back in the wrong order within a group
    "scatter_order": ("o[n] = oo[r]", "o[n] = oo[len(items) - 1 - r]"),
    # V rows taken from the K tensor
    "v_from_k": ("vv_ = bf16_to_f64(vv[b, g, :kmax])", "vv_ = bf16_to_f64(kv[b, g, :kmax])"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes_are_caught(name):
    m = mutant(*MUTANTS[name])
    caught = [not sampled_vs_full(m, case, seed=74) for case in CASES]
    assert any(caught), f"mutant {name} passed every case"


def test_unmutated_copy_passes():
    m = mutant("kmax = int(nv.max())", "kmax = int(nv.max())")
    assert all(sampled_vs_full(m, case, seed=74) for case in CASES)
