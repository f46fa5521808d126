"""Parity of the FP8 (E4M3) forward (attn_fwd_fp8) with the fp64 oracle on
the decoded, descaled inputs (GPU), under the forward's tolerance:
|O - O_ref| <= 2 ulp_bf16(|O_ref|) + 1e-3 and |LSE - LSE_ref| <= 1e-3.  The
products of E4M3 values in Q.K^T are exact in fp32 and the widening of V to
fp16 is exact, so the arithmetic after them is that of the bf16 forward (fp32
accumulation, fp16 probabilities for P.V, bf16 output)."""
import numpy as np
import pytest
import torch

import attn_inputs as gen
import exact_attention_60_amd as ea
import oracle.fp8 as f8
from gpu_util import host_f64, logical_o, need_gpu, oracle_workers
from tolerance import check_lse, check_o

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def dev_u8(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def run(p):
    o, lse = ea.attn_fwd_fp8(dev_u8(p.q), dev_u8(p.k), dev_u8(p.v), descale_q=p.descale_q,
                             descale_k=p.descale_k, descale_v=p.descale_v, causal=p.causal,
                             scale=p.scale, layout="bshd" if p.layout == gen.BSHD else "bhsd")
    torch.cuda.synchronize()
    return o, lse


def check_all(p, what):
    print(f"case: {what}", flush=True)
    o, lse = run(p)
    o_ref, l_ref = f8.attention_fp8(p.q, p.k, p.v, p.descale_q, p.descale_k, p.descale_v, p.B,
                                    p.Hq, p.Hkv, p.Sq, p.Sk, p.scale, p.causal, p.layout)
    e = check_o(logical_o(o, p.layout), o_ref, what)
    el = check_lse(host_f64(lse), l_ref, what)
    print(f"{what}: err/tol {e[1]:.3f} lse {el:.3g}", flush=True)


@pytest.mark.parametrize("B,Hq,Hkv,Sq,Sk,layout,causal", [
    (1, 4, 4, 256, 256, gen.BSHD, False),      # the tiny MHA shape
    (2, 8, 2, 200, 200, gen.BHSD, True),       # GQA causal, ragged blocks and tiles
    (1, 4, 2, 300, 77, gen.BSHD, False),       # cross attention, short keys
    (1, 4, 2, 150, 100, gen.BSHD, True),       # rows that see no key
    (1, 4, 1, 70, 600, gen.BHSD, True),        # MQA, bottom-right alignment
    (1, 2, 2, 1, 1, gen.BSHD, False),          # one row, one key
    (1, 2, 1, 129, 1000, gen.BSHD, False),     # one row past a block, many tiles
    (1, 4, 4, 600, 333, gen.BHSD, True),       # several 256-row workgroups, ragged tile
    (2, 6, 3, 513, 700, gen.BSHD, False),      # group 2, a 256-row block plus one row
    (1, 8, 8, 1000, 1000, gen.BSHD, True),     # 8 heads: the XCD-grouped causal order
])
def test_shapes_all_elements(B, Hq, Hkv, Sq, Sk, layout, causal):
    p = gen.fp8_prefill_inputs(B, Hq, Hkv, Sq, Sk, layout=layout, causal=causal, seed=Sq + Sk)
    check_all(p, f"fp8 B{B} Hq{Hq} Hkv{Hkv} Sq{Sq} Sk{Sk} causal{causal}")


def test_descales_and_peaky_rows():
    # descales far from 1 and a large Q (amp 6): sharp softmax rows
    p = gen.fp8_prefill_inputs(1, 4, 2, 160, 230, layout=gen.BSHD, causal=True, seed=21,
                               descales=(1.75, 0.625, 0.0390625), amp=(6.0, 1.0, 1.0))
    check_all(p, "fp8 descales, peaky rows")


def test_subnormal_inputs():
    # amp 0.02: most bytes are E4M3 subnormals (|x| < 2^-6): subnormal
    # operands of the fp8 MFMA, and fp16 subnormals after the widening of V;
    # the descales bring the scores back to order one
    p = gen.fp8_prefill_inputs(1, 4, 4, 128, 192, layout=gen.BHSD, seed=22,
                               descales=(64.0, 64.0, 32.0), amp=(0.02, 0.02, 0.02))
    frac = np.mean((p.q & 0x78) == 0)
    assert frac > 0.3, frac
    check_all(p, "fp8 subnormal inputs")


def test_extreme_values():
    """The largest finite E4M3 bytes (+-448) among V values of order 200, with
    descales 1, so the real values are of order hundreds.  The fp16 rounding
    of the probabilities then moves a nearly cancelling row by far more than
    1e-3, so O is checked against the large-V bound of tests/tolerance.py (the
    spread of that rounding, computed by the oracle's arithmetic on the
    decoded values); LSE keeps its bound."""
    from tolerance import check_o_large_v, pv_spread_rows
    import oracle.attention as att
    p = gen.fp8_prefill_inputs(1, 2, 1, 64, 100, layout=gen.BSHD, seed=23, amp=(1.0, 1.0, 200.0))
    p.v[0, ::7, 0, ::5] = 0x7E
    p.v[0, 3::11, 0, 1::9] = 0xFE
    assert np.abs(f8.e4m3_to_f64(p.v)).max() == 448.0
    print("case: fp8 extreme V", flush=True)
    o, lse = run(p)
    o_ref, l_ref = f8.attention_fp8(p.q, p.k, p.v, p.descale_q, p.descale_k, p.descale_v, p.B,
                                    p.Hq, p.Hkv, p.Sq, p.Sk, p.scale, p.causal, p.layout)
    kk = p.descale_k * f8.e4m3_to_f64(p.k[0, :, 0])
    vv = p.descale_v * f8.e4m3_to_f64(p.v[0, :, 0])
    spread = np.zeros_like(o_ref)
    for h in range(p.Hq):
        qq = p.descale_q * f8.e4m3_to_f64(p.q[0, :, h])
        spread[0, h] = pv_spread_rows(qq, kk, vv, att.scale_as_f32(p.scale))
    e, r, r_plain = check_o_large_v(logical_o(o, p.layout), o_ref, spread, "fp8 extreme V")
    el = check_lse(host_f64(lse), l_ref, "fp8 extreme V")
    print(f"fp8 extreme V: max err {e:.3g} err/tol {r:.3f} (plain bound {r_plain:.2f}) "
          f"lse {el:.3g}", flush=True)


def test_mha_full_size_sampled_rows():
    p = gen.fp8_mha_prefill()
    print(f"case: {p.name}", flush=True)
    o, lse = run(p)
    rng = np.random.default_rng(5)
    rows = [(int(rng.integers(p.B)), int(rng.integers(p.Hq)), int(i))
            for i in rng.integers(0, p.Sq, size=48)] + [(3, 31, p.Sq - 1), (0, 0, 0)]
    o_ref, l_ref = f8.attention_fp8(p.q, p.k, p.v, 1, 1, 1, p.B, p.Hq, p.Hkv, p.Sq, p.Sk, p.scale,
                                    False, p.layout, rows=rows)
    got = logical_o(o, p.layout)
    gl = host_f64(lse)
    idx = tuple(np.array(rows).T)
    e = check_o(got[idx], o_ref[idx], p.name)
    el = check_lse(gl[idx], l_ref[idx], p.name)
    print(f"{p.name}: sampled err/tol {e[1]:.3f} lse {el:.3g}", flush=True)


def test_mha_full_size_every_element():
    """The benchmark's FP8 MHA workload (B=4, H=32, S=4096, BHSD), every
    element of O and LSE against the whole oracle."""
    p = gen.fp8_mha_prefill()
    print(f"case: {p.name} (every element)", flush=True)
    o, lse = run(p)
    o_ref, l_ref = f8.attention_fp8(p.q, p.k, p.v, p.descale_q, p.descale_k, p.descale_v, p.B,
                                    p.Hq, p.Hkv, p.Sq, p.Sk, p.scale, p.causal, p.layout,
                                    workers=oracle_workers())
    e = check_o(logical_o(o, p.layout), o_ref, p.name)
    el = check_lse(host_f64(lse), l_ref, p.name)
    print(f"{p.name}: every element err/tol {e[1]:.3f} lse {el:.3g}", flush=True)


def test_float8_dtype_accepted_and_deterministic():
    p = gen.fp8_prefill_inputs(1, 4, 2, 100, 140, causal=True, seed=24)
    q = dev_u8(p.q).view(torch.float8_e4m3fn)
    k = dev_u8(p.k).view(torch.float8_e4m3fn)
    v = dev_u8(p.v).view(torch.float8_e4m3fn)
    a = ea.attn_fwd_fp8(q, k, v, causal=True)
    b = run(p)
    torch.cuda.synchronize()
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16))
    assert torch.equal(a[1], b[1])


def test_causal_gqa_full_size_sampled_rows():
    # the causal GQA workload's shape (B=8, Hq=32, Hkv=8, S=8192, BSHD) in E4M3
    p = gen.fp8_prefill_inputs(8, 32, 8, 8192, 8192, layout=gen.BSHD, causal=True, seed=9,
                               descales=(0.5, 0.5, 2.0))
    print("case: fp8 causal gqa b8 hq32 hkv8 s8192", flush=True)
    o, lse = run(p)
    rng = np.random.default_rng(6)
    rows = [(int(rng.integers(p.B)), int(rng.integers(p.Hq)), int(i))
            for i in rng.integers(0, p.Sq, size=40)] + [(7, 31, p.Sq - 1), (0, 0, 0), (3, 5, 64)]
    o_ref, l_ref = f8.attention_fp8(p.q, p.k, p.v, p.descale_q, p.descale_k, p.descale_v, p.B,
                                    p.Hq, p.Hkv, p.Sq, p.Sk, p.scale, True, p.layout, rows=rows)
    idx = tuple(np.array(rows).T)
    e = check_o(logical_o(o, p.layout)[idx], o_ref[idx], "fp8 causal gqa")
    el = check_lse(host_f64(lse)[idx], l_ref[idx], "fp8 causal gqa")
    print(f"fp8 causal gqa s8192: sampled err/tol {e[1]:.3f} lse {el:.3g}", flush=True)
