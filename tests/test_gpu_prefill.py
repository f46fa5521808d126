"""Parity of the HIP attention forward with the fp64 oracle (GPU)."""
import json
import os

import numpy as np
import pytest
import torch

import attn_inputs as gen
import exact_attention_60_amd as ea
import oracle.attention as att
from gpu_util import (bits_of, check_full, dev_bf16, host_f64, logical_o,
                      need_gpu, run_fwd)
from tolerance import check_lse, check_o, check_o_large_v, pv_spread_prefill

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def test_config1_tiny_mha_all_elements():
    p = gen.config1()
    o, lse = run_fwd(p)
    check_full(p, o, lse, "config1")


def test_golden_fixture_cases():
    fx = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "oracle_small.json")))
    for c in fx["cases"]:
        p = gen.prefill_inputs(c["B"], c["Hq"], c["Hkv"], c["Sq"], c["Sk"], layout=c["layout"],
                               causal=c["causal"], seed=c["seed"])
        o, lse = run_fwd(p)
        o_ref = np.array(c["o"]).reshape(p.B, p.Hq, p.Sq, 128)
        l_ref = np.array([(-np.inf if x is None else x) for x in c["lse"]]).reshape(p.B, p.Hq, p.Sq)
        check_o(logical_o(o, p.layout), o_ref, "golden")
        check_lse(host_f64(lse), l_ref, "golden")


SHAPES = [
    # B, Hq, Hkv, Sq, Sk, layout, causal
    (1, 2, 2, 1, 1, gen.BSHD, False),
    (1, 2, 1, 17, 15, gen.BSHD, False),
    (2, 4, 2, 63, 65, gen.BHSD, False),
    (1, 3, 3, 129, 127, gen.BSHD, True),
    (1, 8, 2, 300, 300, gen.BSHD, True),
    (2, 4, 1, 257, 257, gen.BHSD, True),
    (1, 4, 4, 513, 200, gen.BSHD, False),
    (1, 2, 2, 100, 700, gen.BHSD, True),    # Sq < Sk: bottom-right causal
    (1, 2, 1, 400, 150, gen.BSHD, True),    # Sq > Sk: first rows see no key
    (1, 16, 2, 64, 1000, gen.BSHD, False),
    (3, 2, 2, 1, 333, gen.BHSD, True),      # one query row sees every key
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B%d_Hq%d_Hkv%d_Sq%d_Sk%d_%s_%s" % (
    s[0], s[1], s[2], s[3], s[4], "bshd" if s[5] == 0 else "bhsd", "causal" if s[6] else "full"))
def test_ragged_shapes_all_elements(shape):
    B, Hq, Hkv, Sq, Sk, lay, causal = shape
    p = gen.prefill_inputs(B, Hq, Hkv, Sq, Sk, layout=lay, causal=causal, seed=B * 1000 + Sq + Sk,
                           n_hot=min(4, Sq * Hq))
    o, lse = run_fwd(p)
    check_full(p, o, lse, str(shape))


def test_scaled_rows_and_other_scales():
    for scale in (0.02, 0.5):
        p = gen.prefill_inputs(1, 2, 2, 200, 333, layout=gen.BSHD, seed=7, scale=scale, n_hot=16)
        o, lse = run_fwd(p)
        check_full(p, o, lse, f"scale={scale}")


def test_causal_row0_is_v0_bitwise():
    p = gen.prefill_inputs(2, 4, 2, 300, 300, layout=gen.BSHD, causal=True, seed=77)
    o, _ = run_fwd(p)
    ob = bits_of(o)
    for b in range(2):
        for h in range(4):
            assert np.array_equal(ob[b, 0, h], p.v[b, 0, h // 2])


def test_layouts_agree_bitwise():
    p = gen.prefill_inputs(2, 4, 2, 270, 190, layout=gen.BSHD, causal=True, seed=78)
    o1, l1 = run_fwd(p)
    q2 = dev_bf16(p.q.transpose(0, 2, 1, 3))
    k2 = dev_bf16(p.k.transpose(0, 2, 1, 3))
    v2 = dev_bf16(p.v.transpose(0, 2, 1, 3))
    o2, l2 = ea.attn_fwd(q2, k2, v2, causal=True, scale=p.scale, layout="bhsd")
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(o1).transpose(0, 2, 1, 3), bits_of(o2))
    assert torch.equal(l1, l2)


def test_gqa_equals_repeated_mha():
    """GQA/MQA equals MHA over repeated K/V heads (pin P9): both meet the bound
    against the oracle, and within one kernel the results are bitwise equal.
    Group sizes that are a multiple of 4 run the kernel whose workgroups share
    K/V tiles among 4 query heads; groups of 1 and 2 run the other one, so the
    bitwise check pairs groups of 2 with MHA and groups of 8 with groups of 4
    over duplicated K/V heads."""
    for Hkv in (1, 2, 4):
        p = gen.prefill_inputs(1, 8, Hkv, 150, 260, layout=gen.BSHD, causal=False, seed=79 + Hkv)
        o1, l1 = run_fwd(p)
        check_full(p, o1, l1, f"gqa Hkv={Hkv}")
        G = 8 // Hkv
        q = dev_bf16(p.q)
        o2, l2 = ea.attn_fwd(q, dev_bf16(np.repeat(p.k, G, axis=2)),
                             dev_bf16(np.repeat(p.v, G, axis=2)), causal=False, scale=p.scale,
                             layout="bshd")
        torch.cuda.synchronize()
        check_full(p, o2, l2, f"repeated mha Hkv={Hkv}")
        if G == 2:        # both on the kernel for groups of 1 and 2
            assert torch.equal(o1, o2) and torch.equal(l1, l2), Hkv
        if G == 8:        # the same K/V head twice: groups of 4, same kernel as groups of 8
            o3, l3 = ea.attn_fwd(q, dev_bf16(np.repeat(p.k, 2, axis=2)),
                                 dev_bf16(np.repeat(p.v, 2, axis=2)), causal=False,
                                 scale=p.scale, layout="bshd")
            torch.cuda.synchronize()
            assert torch.equal(o1, o3) and torch.equal(l1, l3), Hkv


def test_deterministic_repeat():
    p = gen.prefill_inputs(1, 8, 2, 700, 700, layout=gen.BSHD, causal=True, seed=80)
    o1, l1 = run_fwd(p)
    o2, l2 = run_fwd(p)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_outputs_stay_inside_their_buffers():
    """Guard zones around O and LSE keep their sentinel values."""
    p = gen.prefill_inputs(1, 4, 2, 333, 222, layout=gen.BHSD, causal=True, seed=81)
    q, k, v = dev_bf16(p.q), dev_bf16(p.k), dev_bf16(p.v)
    n_o = q.numel()
    G = 4096  # guard elements (8 KB, keeps 16-byte alignment)
    ob = torch.full((n_o + 2 * G,), 7.0, dtype=torch.bfloat16, device="cuda")
    lb = torch.full((4 * 333 + 2 * G,), 7.0, dtype=torch.float32, device="cuda")
    o = ob[G:G + n_o].view(q.shape)
    lse = lb[G:G + 4 * 333].view(1, 4, 333)
    ea.attn_fwd(q, k, v, causal=True, scale=p.scale, layout="bhsd", out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.all(ob[:G] == 7.0) and torch.all(ob[G + n_o:] == 7.0)
    assert torch.all(lb[:G] == 7.0) and torch.all(lb[G + 4 * 333:] == 7.0)
    check_full(p, o, lse, "guarded")


def test_nonfinite_stays_in_its_rows():
    """A NaN in one query row only spoils that row (non-finite inputs are
    outside the parity contract; this checks containment only)."""
    p = gen.prefill_inputs(1, 2, 2, 130, 140, layout=gen.BSHD, seed=82)
    q = p.q.copy()
    q[0, 5, 1, 3] = 0x7FC0
    o, lse = ea.attn_fwd(dev_bf16(q), dev_bf16(p.k), dev_bf16(p.v), scale=p.scale)
    torch.cuda.synchronize()
    of = host_f64(o)
    bad = ~np.isfinite(of)
    assert bad[0, 5, 1].all()
    bad[0, 5, 1] = False
    assert not bad.any()


def test_v_beyond_fp16_range():
    """V entries far beyond the fp16 range (3e5 and -2e6) take the bf16 path
    and still meet the bound; a constant V column gives that constant."""
    p = gen.prefill_inputs(1, 4, 2, 300, 1500, layout=gen.BSHD, causal=True, seed=83)
    v = (p.v.astype(np.uint32) << 16).view(np.float32).copy()
    v[:, :, :, 5] = 3.0e5
    v[0, 700, 1, 9] = -2.0e6
    p.v = gen.f32_to_bf16_bits(v)
    o, lse = run_fwd(p)
    check_full(p, o, lse, "huge V")
    # 3e5 rounds to the bf16 value 299008 (spacing 2048 there)
    assert np.all(host_f64(o)[..., 5] == 299008.0)


# ---- the full-size workloads (launch configuration of the benchmark): every
# element of O and LSE against the whole oracle

def _full_size(p):
    print(f"case: {p.name} (every element)", flush=True)
    o, lse = run_fwd(p)
    assert bool(torch.isfinite(o.float()).all()), "non-finite output"
    (eo, ro), el = check_full(p, o, lse, p.name)
    print(f"{p.name}: every element, max err {eo:.3g} err/tol {ro:.3f} lse err {el:.3g}",
          flush=True)
    return ro


def test_config2_mha_prefill_every_element():
    _full_size(gen.config2())


def test_config3_causal_gqa_every_element():
    _full_size(gen.config3())


def test_config4_self_every_element():
    _full_size(gen.config4_self())


def test_config4_cross_every_element():
    _full_size(gen.config4_cross())


# ---- large V: the bound that the fp16 rounding of the probabilities allows

@pytest.mark.parametrize("Sq,Sk,causal,Hkv", [(300, 333, True, 2), (200, 40, False, 1),
                                              (100, 1300, False, 4)])
def test_large_v_under_derived_bound(Sq, Sk, causal, Hkv):
    """V ~ 300 N(0, 1) (every value in the fp16 range, so the fp16 path runs)
    and peaky rows: checked against the large-V bound of tests/tolerance.py
    (2 ulp + 1e-3 + the spread of the fp16 probability rounding)."""
    p = gen.prefill_inputs(1, 4, Hkv, Sq, Sk, layout=gen.BSHD, causal=causal, seed=Sq + Sk + 5,
                           n_hot=24, v_amp=300.0)
    o, lse = run_fwd(p)
    o_ref, l_ref = att.attention(p.q, p.k, p.v, p.B, p.Hq, p.Hkv, p.Sq, p.Sk, p.scale,
                                 p.causal, p.layout)
    spread = pv_spread_prefill(p)
    e, r, r_plain = check_o_large_v(logical_o(o, p.layout), o_ref, spread, "large V")
    check_lse(host_f64(lse), l_ref, "large V lse")
    print(f"large V Sq{Sq} Sk{Sk}: max err {e:.3g}, err/tol {r:.3f} "
          f"(err/tol under the plain bound {r_plain:.2f})", flush=True)


def _random_shapes(n, seed):
    """Seeded random small shapes: any group size, both layouts, causal or
    not, lengths not multiples of the 256-row / 64-key tiles."""
    r = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        Hkv = int(r.choice([1, 2, 3, 4]))
        G = int(r.choice([1, 2, 3, 5, 8]))
        out.append((int(r.integers(1, 3)), Hkv * G, Hkv, int(r.integers(1, 600)),
                    int(r.integers(1, 700)), int(r.integers(0, 2)), bool(r.integers(0, 2))))
    return out


@pytest.mark.parametrize("shape", _random_shapes(24, 2024),
                         ids=lambda s: "B%d_Hq%d_Hkv%d_Sq%d_Sk%d_L%d_C%d" % (
                             s[0], s[1], s[2], s[3], s[4], s[5], int(s[6])))
def test_random_shapes_all_elements(shape):
    B, Hq, Hkv, Sq, Sk, lay, causal = shape
    p = gen.prefill_inputs(B, Hq, Hkv, Sq, Sk, layout=lay, causal=causal,
                           seed=7 * Sq + 13 * Sk + Hq, n_hot=min(3, Sq * Hq))
    o, lse = run_fwd(p)
    check_full(p, o, lse, str(shape))


# ---- the GQA kernel (query-head groups that are a multiple of 4: the 4 waves
# of a workgroup are 4 query heads sharing each K/V tile; 64-row query tiles,
# 32-key K/V tiles)

GQA4_SHAPES = [
    # B, Hq, Hkv, Sq, Sk, layout, causal
    (1, 4, 1, 1, 1, gen.BSHD, False),        # MQA, one row, one key
    (1, 4, 1, 31, 33, gen.BHSD, True),       # ragged 32-key tiles
    (2, 8, 2, 64, 64, gen.BSHD, True),       # exactly one row tile
    (1, 8, 2, 65, 700, gen.BSHD, False),     # one row past a tile, many key tiles
    (1, 8, 1, 200, 130, gen.BHSD, True),     # Sq > Sk: first rows see no key
    (1, 16, 2, 129, 129, gen.BSHD, True),    # group of 8: two workgroups per K/V head
    (2, 12, 3, 100, 37, gen.BHSD, False),    # three K/V heads, short keys
    (1, 8, 2, 333, 1000, gen.BSHD, True),    # Sq < Sk bottom-right, diagonal masks
]


@pytest.mark.parametrize("shape", GQA4_SHAPES, ids=lambda s: "B%d_Hq%d_Hkv%d_Sq%d_Sk%d_%s_%s" % (
    s[0], s[1], s[2], s[3], s[4], "bshd" if s[5] == 0 else "bhsd", "causal" if s[6] else "full"))
def test_gqa_group4_kernel_all_elements(shape):
    B, Hq, Hkv, Sq, Sk, lay, causal = shape
    p = gen.prefill_inputs(B, Hq, Hkv, Sq, Sk, layout=lay, causal=causal,
                           seed=3 * Sq + 5 * Sk + Hq, n_hot=min(6, Sq * Hq))
    o, lse = run_fwd(p)
    check_full(p, o, lse, str(shape))


def test_gqa_group4_kernel_v_beyond_fp16_range():
    """The GQA kernel's bf16 fallback: V entries far beyond the fp16 range."""
    p = gen.prefill_inputs(1, 8, 2, 150, 300, layout=gen.BSHD, causal=True, seed=84)
    v = (p.v.astype(np.uint32) << 16).view(np.float32).copy()
    v[:, :, :, 7] = 3.0e5
    v[0, 120, 1, 11] = -2.0e6
    p.v = gen.f32_to_bf16_bits(v)
    o, lse = run_fwd(p)
    check_full(p, o, lse, "huge V, gqa kernel")
    assert np.all(host_f64(o)[..., 7] == 299008.0)


def test_gqa_group4_kernel_large_v_under_derived_bound():
    p = gen.prefill_inputs(1, 8, 2, 140, 400, layout=gen.BHSD, causal=True, seed=85, n_hot=24,
                           v_amp=300.0)
    o, lse = run_fwd(p)
    o_ref, l_ref = att.attention(p.q, p.k, p.v, p.B, p.Hq, p.Hkv, p.Sq, p.Sk, p.scale,
                                 p.causal, p.layout)
    e, r, r_plain = check_o_large_v(logical_o(o, p.layout), o_ref, pv_spread_prefill(p),
                                    "large V, gqa kernel")
    check_lse(host_f64(lse), l_ref, "large V lse, gqa kernel")
    print(f"large V (gqa kernel): err/tol {r:.3f} (plain bound {r_plain:.2f})", flush=True)
